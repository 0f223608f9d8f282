// kda_prologue.hip -- KDA input prologue for gfx950: ShortConv + Swish (+ L2Norm per head).
//
// [K3 note] = "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
//   §3.2  q, k = L2Norm(Swish(ShortConv(W x))), v = Swish(ShortConv(W_v x)); in decoding the
//         layer reads and writes a short-convolution cache C^conv of the few most recent
//         inputs.  The projections need trained weights; the projected inputs are the input.
// Readings: causal depthwise convolution of width W (1..4) per channel, the last tap on the
// current token; history before a sequence's first token from cache_in (oldest first) or
// zero; Swish(u) = u Sigmoid(u); L2Norm divides each group of l2 channels (one head) by
// sqrt(sum u^2 + 1e-6); cache_out = the last W - 1 inputs of each sequence.
//
// Packed tokens are cut into fixed 64-token segments regardless of sequence boundaries; a
// segment finds its first token's sequence by binary search and restarts the sliding
// window whenever it crosses into the next sequence.  Each lane owns 8 consecutive channels
// (16-byte accesses) and keeps the last W - 1 inputs of them in registers; the L2Norm sum is
// a butterfly over the lanes of one head.  A second small kernel writes the caches.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {
constexpr int kSegT = 64;          // tokens per segment
constexpr int kChanPerBlock = 2048;  // 256 threads x 8 channels

template <typename T> struct V8;
template <> struct V8<bf16_t> {
    struct Raw { uint4 a; };  // eight channels as loaded, converted later (a use would wait)
    __device__ __forceinline__ static Raw load_raw(const bf16_t* p) { return Raw{ld_stream16(p)}; }
    __device__ __forceinline__ static void convert(const Raw& r, float* x) {
        const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = lo_bf16(w[i]); x[2 * i + 1] = hi_bf16(w[i]); }
    }
    __device__ __forceinline__ static void load(const bf16_t* p, float* x) { convert(load_raw(p), x); }
    __device__ __forceinline__ static void store(bf16_t* p, const float* x) {
        st_stream16(p, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                  pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
    }
};
template <> struct V8<float> {
    struct Raw { float4 a, b; };
    __device__ __forceinline__ static Raw load_raw(const float* p) {
        return Raw{ld_stream_f4(p), ld_stream_f4(p + 4)};
    }
    __device__ __forceinline__ static void convert(const Raw& r, float* x) {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w; x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
    __device__ __forceinline__ static void load(const float* p, float* x) { convert(load_raw(p), x); }
    __device__ __forceinline__ static void store(float* p, const float* x) {
        st_stream_f4(p, make_float4(x[0], x[1], x[2], x[3]));
        st_stream_f4(p + 4, make_float4(x[4], x[5], x[6], x[7]));
    }
};

// x of another lane of the same row of 16, chosen by a DPP control code
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// sequence containing packed token t (the last sequence whose start is <= t)
__device__ __forceinline__ int seq_of(const int32_t* cu, int n_seqs, int64_t T, int64_t t) {
    if (!cu) return static_cast<int>(t / T);
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}
}  // namespace

// L2 = a.l2 (0, 64 or 128) as a constant, so the per-head sum is an unrolled butterfly
template <int W, int L2, typename T>
__global__ void __launch_bounds__(256) short_conv_kernel(ShortConvArgs a) {
    constexpr int HIST = W - 1;
    // workgroup -> (segment, channel block) with the channel block fastest: the workgroups
    // in flight together cover whole token rows
    const int ncb = (a.C + kChanPerBlock - 1) / kChanPerBlock;
    const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(ncb));
    const int64_t seg = static_cast<int64_t>(blockIdx.x / static_cast<unsigned>(ncb));
    const int c0 = cb * kChanPerBlock + threadIdx.x * 8;
    const bool live = c0 < a.C;
    const int64_t tb = seg * kSegT;
    const int64_t te = tb + kSegT < a.total ? tb + kSegT : a.total;
    const T* x = static_cast<const T*>(a.x);
    T* y = static_cast<T*>(a.y);

    // With L2Norm the weights carry -log2(e): the convolution then yields Swish's exp2
    // argument directly, and the normalisation, being scale-invariant (its epsilon scaled by
    // log2(e)^2 and its sign flipped), removes the factor again
    constexpr float kWs = L2 > 0 ? -kLog2e : 1.f;
    float wt[8][W];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < W; ++i) wt[e][i] = live ? kWs * a.w[static_cast<int64_t>(c0 + e) * W + i] : 0.f;

    int n = seq_of(a.cu, a.n_seqs, a.T, tb);
    int64_t s0 = seq_start(a.cu, a.T, n), s1 = seq_start(a.cu, a.T, n + 1);
    float win[HIST > 0 ? HIST : 1][8];  // win[i] = input at position t - HIST + i
    auto fill = [&](int64_t t) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < HIST; ++i) {
            const int64_t p = t - HIST + i;
            if (p >= s0) {
                if (live) V8<T>::load(x + p * a.C + c0, win[i]);
                else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) win[i][e] = 0.f;
                }
            } else {
                const int64_t j = HIST + (p - s0);  // index into this sequence's cache
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    win[i][e] = (a.cache_in && live) ? a.cache_in[(static_cast<int64_t>(n) * a.C + c0 + e) * HIST + j] : 0.f;
            }
        }
    };
    // one token: convolution over the window and the current input, Swish, optional L2Norm,
    // store, then slide the window
    auto token = [&](int64_t t, const float* cur, bool store) __attribute__((always_inline)) {
        float out[8];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = wt[e][HIST] * cur[e];
#pragma unroll
            for (int i = 0; i < HIST; ++i) acc += wt[e][i] * win[i][e];
            if constexpr (L2 > 0)
                out[e] = acc * fast_rcp(1.f + fast_exp2(acc));  // -log2(e) Swish
            else
                out[e] = acc * fast_rcp(1.f + fast_exp2(-acc * kLog2e));  // Swish
            ss += out[e] * out[e];
        }
        if constexpr (L2 > 0) {
            // sum over the L2 / 8 lanes of one head with DPP lane permutations (no LDS trips):
            // quads, then the two quads of each half row (mirror), then the two half rows
            static_assert(L2 == 64 || L2 == 128, "L2Norm over 64 or 128 channels");
            ss += dpp_f32<0xB1>(ss);   // quad_perm [1,0,3,2]
            ss += dpp_f32<0x4E>(ss);   // quad_perm [2,3,0,1]
            ss += dpp_f32<0x141>(ss);  // row_half_mirror
            if constexpr (L2 == 128) ss += dpp_f32<0x128>(ss);  // row_ror:8
            const float inv = -__builtin_amdgcn_rsqf(ss + 1e-6f * kLog2e * kLog2e);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] *= inv;
        }
        if (store) V8<T>::store(y + t * a.C + c0, out);
#pragma unroll
        for (int i = 0; i + 1 < HIST; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) win[i][e] = win[i + 1][e];
        if (HIST > 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[HIST > 0 ? HIST - 1 : 0][e] = cur[e];
        }
    };
    if (te <= s1 && te - tb == kSegT && tb - HIST >= s0 && live) {
        // the common case, a whole segment inside one sequence with its history: every load is
        // issued ahead of its use -- the history rows together, then each group of kU tokens
        // while the previous group is computed -- so each lane keeps up to 2 kU loads in flight
        constexpr int kU = 16, kG = kSegT / kU;
        typename V8<T>::Raw hist[HIST > 0 ? HIST : 1], raw[2][kU];
#pragma unroll
        for (int i = 0; i < HIST; ++i) hist[i] = V8<T>::load_raw(x + (tb - HIST + i) * a.C + c0);
        auto issue = [&](int gi) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < kU; ++u) raw[gi & 1][u] = V8<T>::load_raw(x + (tb + gi * kU + u) * a.C + c0);
        };
        issue(0);
#pragma unroll
        for (int i = 0; i < HIST; ++i) V8<T>::convert(hist[i], win[i]);
#pragma unroll
        for (int gi = 0; gi < kG; ++gi) {
            if (gi + 1 < kG) issue(gi + 1);
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                float cur[8];
                V8<T>::convert(raw[gi & 1][u], cur);
                token(tb + gi * kU + u, cur, true);  // every lane here is live
            }
        }
        return;
    }
    fill(tb);
    for (int64_t t = tb; t < te; ++t) {
        if (t >= s1) {  // crossed into the next non-empty sequence
            while (seq_start(a.cu, a.T, n + 1) <= t) ++n;
            s0 = seq_start(a.cu, a.T, n);
            s1 = seq_start(a.cu, a.T, n + 1);
            fill(t);
        }
        float cur[8];
        if (live) V8<T>::load(x + t * a.C + c0, cur);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) cur[e] = 0.f;
        }
        token(t, cur, live);
    }
}

// cache_out[n][c][j] = input at position L_n - (W-1) + j of sequence n (from cache_in when
// that position precedes the sequence); every value is read before any is written, so
// cache_out may be cache_in.
template <typename T>
__global__ void __launch_bounds__(256) conv_cache_kernel(ShortConvArgs a) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= static_cast<int64_t>(a.n_seqs) * a.C) return;
    const int n = static_cast<int>(idx / a.C), c = static_cast<int>(idx - static_cast<int64_t>(n) * a.C);
    const int hist = a.W - 1;
    const int64_t s0 = seq_start(a.cu, a.T, n), L = seq_start(a.cu, a.T, n + 1) - s0;
    float v[3];
    for (int j = 0; j < hist; ++j) {
        const int64_t p = L - hist + j;
        v[j] = p >= 0 ? Elem<T>::load1(static_cast<const T*>(a.x) + (s0 + p) * a.C + c)
                      : (a.cache_in ? a.cache_in[idx * hist + (hist + p)] : 0.f);
    }
    for (int j = 0; j < hist; ++j) a.cache_out[idx * hist + j] = v[j];
}

template <int L2, typename T>
static void launch_conv_w(const ShortConvArgs& a, dim3 grid, hipStream_t stream) {
    switch (a.W) {
        case 1: hipLaunchKernelGGL((short_conv_kernel<1, L2, T>), grid, dim3(256), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((short_conv_kernel<2, L2, T>), grid, dim3(256), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((short_conv_kernel<3, L2, T>), grid, dim3(256), 0, stream, a); break;
        default: hipLaunchKernelGGL((short_conv_kernel<4, L2, T>), grid, dim3(256), 0, stream, a); break;
    }
}

template <typename T>
static hipError_t launch_conv_t(const ShortConvArgs& a, hipStream_t stream) {
    if (a.total > 0) {
        const dim3 grid(static_cast<unsigned>((a.total + kSegT - 1) / kSegT *
                                              ((a.C + kChanPerBlock - 1) / kChanPerBlock)));
        if (a.l2 == 128) launch_conv_w<128, T>(a, grid, stream);
        else if (a.l2 == 64) launch_conv_w<64, T>(a, grid, stream);
        else launch_conv_w<0, T>(a, grid, stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.cache_out && a.W > 1) {
        const int64_t n = static_cast<int64_t>(a.n_seqs) * a.C;
        hipLaunchKernelGGL((conv_cache_kernel<T>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_short_conv(const ShortConvArgs& a, bool bf16, hipStream_t stream) {
    return bf16 ? launch_conv_t<bf16_t>(a, stream) : launch_conv_t<float>(a, stream);
}

}  // namespace kda
