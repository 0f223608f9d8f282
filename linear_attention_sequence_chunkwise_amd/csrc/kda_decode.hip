// kda_decode.hip -- single-token KDA decode step for gfx950 (MI355X).
//
// [K3 note] = "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
//   §3.2  per-token map (x_t, S_{t-1}) -> (y_t, S_t): decay Sbar = Diag(alpha) S, predict
//         vhat = Sbar^T k, write S = Sbar + beta k (v - vhat)^T, read o = S^T q afterwards
//   §3.3  recurrent decoding one token at a time; g = g_min Sigmoid(e^A z), alpha = e^g
//
// The step is bound by HBM traffic: each (sequence, head) streams its dk x dv fp32 state
// in and back out (128 KiB at d = 128) against a few hundred bytes of inputs.  One
// workgroup of NT threads (1024 at d = 128) owns one (sequence, head); each thread keeps
// RPT rows x 4 columns of the state in registers (16-byte loads/stores along dv, coalesced,
// marked nontemporal: the state is touched once per step).  Small per-thread tiles keep
// many state loads in flight per CU, which is what sustains the bandwidth.  Both
// reductions over key channels happen in one pass because
//   o = S_t^T q = Sbar^T q + (k.q) beta (v - Sbar^T k),
// so the state is read once, updated in registers, and written once.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int D, int NT, typename TIn>
__global__ void __launch_bounds__(NT) decode_kernel(DecodeArgs args) {
    constexpr int COLG = D / 4;         // float4 column groups
    constexpr int ROWG = NT / COLG;     // row groups
    constexpr int RPT = D / ROWG;       // rows per thread
    constexpr int NWV = NT / 64;        // waves
    static_assert(NT % COLG == 0 && D % ROWG == 0 && COLG <= 64 && D <= NT, "thread tiling");

    __shared__ float s_alpha[D], s_k[D], s_q[D], s_u[D];
    __shared__ float s_red[NWV][2][D];
    __shared__ float s_kq[NWV];

    const int tid = threadIdx.x;
    const int pair = blockIdx.x;  // (sequence, head)
    const int H = args.H;
    const int h = pair % H;
    const size_t vec = static_cast<size_t>(pair) * D;  // offset of this pair in q/k/v/z/o

    // state tile of this thread: rows rg + ROWG*i, columns 4cg .. 4cg+3.  Issued first, so the
    // threads that also compute the gate do not wait for its inputs before streaming the state.
    const int cg = tid % COLG, rg = tid / COLG;
    f32x4_t* __restrict__ st = reinterpret_cast<f32x4_t*>(args.state + static_cast<size_t>(pair) * D * D);
    float4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const f32x4_t t = __builtin_nontemporal_load(&st[(rg + ROWG * i) * COLG + cg]);
        S[i] = make_float4(t[0], t[1], t[2], t[3]);
    }
    // per-channel gate and inputs
    float kqp = 0.f;
    if (tid < D) {
        const float a = -expf(args.A[h * D + tid]) * kLog2e;
        const float z = args.z[vec + tid];
        const float s = fast_rcp(1.f + fast_exp2(a * z));
        s_alpha[tid] = fast_exp2(args.g_min * kLog2e * s);
        const float kk = Elem<TIn>::load1(static_cast<const TIn*>(args.k) + vec + tid);
        const float qq = Elem<TIn>::load1(static_cast<const TIn*>(args.q) + vec + tid);
        s_k[tid] = kk;
        s_q[tid] = qq;
        kqp = kk * qq;
    }

    // k.q: wave reduction, then across waves
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kqp += __shfl_xor(kqp, off);
    if ((tid & 63) == 0) s_kq[tid >> 6] = kqp;
    __syncthreads();

    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + ROWG * i;
        const float al = s_alpha[r], kr = s_k[r], qr = s_q[r];
        S[i].x *= al; S[i].y *= al; S[i].z *= al; S[i].w *= al;  // Sbar
        pk.x += S[i].x * kr; pk.y += S[i].y * kr; pk.z += S[i].z * kr; pk.w += S[i].w * kr;
        pq.x += S[i].x * qr; pq.y += S[i].y * qr; pq.z += S[i].z * qr; pq.w += S[i].w * qr;
    }
    // reduce over the row groups of this wave (lanes that share cg)
#pragma unroll
    for (int off = COLG; off < 64; off <<= 1) {
        pk.x += __shfl_xor(pk.x, off); pk.y += __shfl_xor(pk.y, off);
        pk.z += __shfl_xor(pk.z, off); pk.w += __shfl_xor(pk.w, off);
        pq.x += __shfl_xor(pq.x, off); pq.y += __shfl_xor(pq.y, off);
        pq.z += __shfl_xor(pq.z, off); pq.w += __shfl_xor(pq.w, off);
    }
    const int wv = tid >> 6;
    if ((tid & 63) < COLG) {
        *reinterpret_cast<float4*>(&s_red[wv][0][4 * cg]) = pk;
        *reinterpret_cast<float4*>(&s_red[wv][1][4 * cg]) = pq;
    }
    __syncthreads();
    if (tid < D) {
        float vk = 0.f, vq = 0.f, kq = 0.f;
#pragma unroll
        for (int x = 0; x < NWV; ++x) {
            vk += s_red[x][0][tid];
            vq += s_red[x][1][tid];
            kq += s_kq[x];
        }
        const float beta = Elem<TIn>::load1(static_cast<const TIn*>(args.beta) + pair);
        const float vv = Elem<TIn>::load1(static_cast<const TIn*>(args.v) + vec + tid);
        const float u = beta * (vv - vk);
        s_u[tid] = u;
        Elem<TIn>::store1(static_cast<TIn*>(args.o) + vec + tid, vq + kq * u);
    }
    __syncthreads();
    const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float kr = s_k[rg + ROWG * i];
        S[i].x += kr * u4.x; S[i].y += kr * u4.y; S[i].z += kr * u4.z; S[i].w += kr * u4.w;
        __builtin_nontemporal_store(f32x4_t{S[i].x, S[i].y, S[i].z, S[i].w}, &st[(rg + ROWG * i) * COLG + cg]);
    }
}

// ---- several tokens per call: speculative verify and commit ----------------------------
// [K3 hood] "Serving two incompatible cache types": rejected draft tokens must not advance
// the recurrent state, and saving a full state per draft position would multiply memory
// traffic; instead the (small) projected inputs are kept and the accepted tokens replayed
// on chip.  verify: from the committed state, the outputs of draft tokens 0..K-1 (each after
// its own write, [K3 note] §3.2), the state only read.  commit: the state advanced in place
// by the first accepted[n] of the same tokens.  Each reads the state once per call (and
// commit writes it once) instead of once per token.  Layout and thread tiling as in the
// single-token kernel; the K tokens' inputs are staged in LDS first.
template <int D, int NT, typename TIn, bool COMMIT>
__global__ void __launch_bounds__(NT) decode_multi_kernel(DecodeMultiArgs args) {
    constexpr int COLG = D / 4;
    constexpr int ROWG = NT / COLG;
    constexpr int RPT = D / ROWG;
    constexpr int NWV = NT / 64;
    constexpr int KM = kDecodeMaxDraft;
    static_assert(NT % COLG == 0 && D % ROWG == 0 && COLG <= 64 && D <= NT && NWV >= 1, "thread tiling");

    __shared__ float s_alpha[KM][D], s_k[KM][D], s_q[COMMIT ? 1 : KM][D], s_v[KM][D];
    __shared__ float s_beta[KM], s_kq[KM], s_u[D];
    __shared__ float s_red[NWV][2][D];

    const int tid = threadIdx.x;
    const int pair = blockIdx.x;
    const int H = args.H, K = args.K;
    const int n = pair / H, h = pair - n * H;
    int ntok = K;
    if constexpr (COMMIT) {
        const int acc = args.accepted[n];
        ntok = acc < 0 ? 0 : acc > K ? K : acc;
        if (ntok == 0) return;  // nothing accepted: the state stays as it is
    }

    // stage the inputs of the ntok tokens: gate, k, q, v per channel; beta per token
    for (int idx = tid; idx < ntok * D; idx += NT) {
        const int t = idx / D, c = idx - t * D;
        const size_t vec = ((static_cast<size_t>(n) * K + t) * H + h) * D + c;
        const float a = -expf(args.A[h * D + c]) * kLog2e;
        const float sg = fast_rcp(1.f + fast_exp2(a * args.z[vec]));
        s_alpha[t][c] = fast_exp2(args.g_min * kLog2e * sg);
        s_k[t][c] = Elem<TIn>::load1(static_cast<const TIn*>(args.k) + vec);
        if constexpr (!COMMIT) s_q[t][c] = Elem<TIn>::load1(static_cast<const TIn*>(args.q) + vec);
        s_v[t][c] = Elem<TIn>::load1(static_cast<const TIn*>(args.v) + vec);
    }
    for (int t = tid; t < ntok; t += NT)
        s_beta[t] = Elem<TIn>::load1(static_cast<const TIn*>(args.beta) + (static_cast<size_t>(n) * K + t) * H + h);

    const int cg = tid % COLG, rg = tid / COLG;
    const size_t sofs = static_cast<size_t>(pair) * D * D;
    const f32x4_t* __restrict__ sin = reinterpret_cast<const f32x4_t*>((COMMIT ? args.state : args.state_in) + sofs);
    float4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const f32x4_t t4 = __builtin_nontemporal_load(&sin[(rg + ROWG * i) * COLG + cg]);
        S[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
    }
    __syncthreads();
    if constexpr (!COMMIT) {  // k . q of every token (one wave per token)
        const int wv = tid >> 6, ln = tid & 63;
        for (int t = wv; t < ntok; t += NWV) {
            float x = 0.f;
            for (int c = ln; c < D; c += 64) x += s_k[t][c] * s_q[t][c];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
            if (ln == 0) s_kq[t] = x;
        }
    }

    const int wv = tid >> 6;
    for (int t = 0; t < ntok; ++t) {
        float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + ROWG * i;
            const float al = s_alpha[t][r], kr = s_k[t][r];
            S[i].x *= al; S[i].y *= al; S[i].z *= al; S[i].w *= al;  // Sbar
            pk.x += S[i].x * kr; pk.y += S[i].y * kr; pk.z += S[i].z * kr; pk.w += S[i].w * kr;
            if constexpr (!COMMIT) {
                const float qr = s_q[t][r];
                pq.x += S[i].x * qr; pq.y += S[i].y * qr; pq.z += S[i].z * qr; pq.w += S[i].w * qr;
            }
        }
#pragma unroll
        for (int off = COLG; off < 64; off <<= 1) {
            pk.x += __shfl_xor(pk.x, off); pk.y += __shfl_xor(pk.y, off);
            pk.z += __shfl_xor(pk.z, off); pk.w += __shfl_xor(pk.w, off);
            if constexpr (!COMMIT) {
                pq.x += __shfl_xor(pq.x, off); pq.y += __shfl_xor(pq.y, off);
                pq.z += __shfl_xor(pq.z, off); pq.w += __shfl_xor(pq.w, off);
            }
        }
        if ((tid & 63) < COLG) {
            *reinterpret_cast<float4*>(&s_red[wv][0][4 * cg]) = pk;
            if constexpr (!COMMIT) *reinterpret_cast<float4*>(&s_red[wv][1][4 * cg]) = pq;
        }
        __syncthreads();
        if (tid < D) {
            float vk = 0.f, vq = 0.f;
#pragma unroll
            for (int x = 0; x < NWV; ++x) {
                vk += s_red[x][0][tid];
                if constexpr (!COMMIT) vq += s_red[x][1][tid];
            }
            const float u = s_beta[t] * (s_v[t][tid] - vk);
            s_u[tid] = u;
            if constexpr (!COMMIT)
                Elem<TIn>::store1(static_cast<TIn*>(args.o) + ((static_cast<size_t>(n) * K + t) * H + h) * D + tid,
                                  vq + s_kq[t] * u);
        }
        __syncthreads();
        const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float kr = s_k[t][rg + ROWG * i];
            S[i].x += kr * u4.x; S[i].y += kr * u4.y; S[i].z += kr * u4.z; S[i].w += kr * u4.w;
        }
    }
    if constexpr (COMMIT) {
        f32x4_t* __restrict__ st = reinterpret_cast<f32x4_t*>(args.state + sofs);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            __builtin_nontemporal_store(f32x4_t{S[i].x, S[i].y, S[i].z, S[i].w}, &st[(rg + ROWG * i) * COLG + cg]);
    }
}

// Commit uses the single-step kernel's thread tiling, so its sums run in the same order and the
// committed state equals single steps bit for bit.  Verify, which only has to match within
// rounding, uses a quarter of the threads (16 state rows per thread): per draft token it
// synchronizes a quarter as many waves.
template <int D, int NT, typename TIn>
static void launch_multi_t(const DecodeMultiArgs& a, bool commit, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H));
    if (commit) hipLaunchKernelGGL((decode_multi_kernel<D, NT, TIn, true>), grid, dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL((decode_multi_kernel<D, NT / 4, TIn, false>), grid, dim3(NT / 4), 0, stream, a);
}

hipError_t launch_decode_multi(const DecodeMultiArgs& a, int d, bool bf16, bool commit, hipStream_t stream) {
    if (d == 128) {
        if (bf16) launch_multi_t<128, 1024, bf16_t>(a, commit, stream);
        else launch_multi_t<128, 1024, float>(a, commit, stream);
    } else {
        if (bf16) launch_multi_t<64, 512, bf16_t>(a, commit, stream);
        else launch_multi_t<64, 512, float>(a, commit, stream);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H));
    if (d == 128) {
        if (bf16) hipLaunchKernelGGL((decode_kernel<128, 1024, bf16_t>), grid, dim3(1024), 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<128, 1024, float>), grid, dim3(1024), 0, stream, a);
    } else {
        if (bf16) hipLaunchKernelGGL((decode_kernel<64, 512, bf16_t>), grid, dim3(512), 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<64, 512, float>), grid, dim3(512), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kda
