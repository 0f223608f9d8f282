// kda_gate.hip -- lower-bounded decay gate and chunk-local cumulative log-decay (gfx950).
//
// [K3 note] = "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
//   §3.3  g = g_min Sigmoid(e^{A} z) in (g_min, 0) with g_min = -5; the chunk algorithm
//         works with cumulative log-decay inside a chunk, whose reciprocal the bound keeps
//         finite.
//
// Elementwise and bandwidth bound.  Each workgroup takes a window of `chunk` packed tokens
// and processes every chunk that STARTS in that window (a chunk is `chunk` tokens from its
// sequence's start, the last one possibly shorter), so the running sum never crosses a
// workgroup.  A window holds at most one chunk start per sequence boundary plus one, and
// the chunks starting in it end before the next window ends, so per-window work is at
// most 2*chunk tokens.  Each thread owns four consecutive (head, channel) columns and
// moves 16 bytes per token per tensor; consecutive threads cover consecutive columns.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// Sequence containing packed token t (sequences may be empty): the last n with start <= t.
__device__ __forceinline__ int find_seq(const int32_t* cu, int64_t T, int n_seqs, int64_t t) {
    if (!cu) return static_cast<int>(t / T);
    int lo = 0, hi = n_seqs;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (static_cast<int64_t>(cu[mid]) <= t) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ void __launch_bounds__(256) gate_kernel(GateArgs a) {
    const int64_t ncol4 = static_cast<int64_t>(a.H) * a.dk / 4;
    // workgroup -> (token window, column block) with the column block fastest: the
    // workgroups in flight together cover whole token rows
    const unsigned ncb = static_cast<unsigned>((ncol4 + 255) / 256);
    const int64_t col = static_cast<int64_t>(blockIdx.x % ncb) * 256 + threadIdx.x;
    const bool active = col < ncol4;
    const int64_t w_lo = static_cast<int64_t>(blockIdx.x / ncb) * a.chunk;
    const int64_t w_hi = w_lo + a.chunk < a.total ? w_lo + a.chunk : a.total;
    if (w_lo >= a.total) return;

    float4 ae = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) {
        const float4 A4 = reinterpret_cast<const float4*>(a.A)[col];
        ae = make_float4(-expf(A4.x) * kLog2e, -expf(A4.y) * kLog2e, -expf(A4.z) * kLog2e,
                         -expf(A4.w) * kLog2e);
    }
    const float gm = a.g_min;
    const float4* __restrict__ z4 = reinterpret_cast<const float4*>(a.z);
    float4* __restrict__ g4 = reinterpret_cast<float4*>(a.g);
    float4* __restrict__ c4 = reinterpret_cast<float4*>(a.gcum);

    int n = find_seq(a.cu, a.T, a.n_seqs, w_lo);
    int64_t s_n = seq_start(a.cu, a.T, n);
    int64_t e_n = a.cu ? static_cast<int64_t>(a.cu[n + 1]) : s_n + a.T;
    // first chunk start at or after w_lo inside sequence n
    int64_t s = s_n + ((w_lo - s_n + a.chunk - 1) / a.chunk) * a.chunk;
    while (true) {
        while (s >= e_n) {  // move to the next non-empty sequence
            if (++n >= a.n_seqs) return;
            s_n = e_n;
            e_n = a.cu ? static_cast<int64_t>(a.cu[n + 1]) : s_n + a.T;
            s = s_n;
        }
        if (s >= w_hi) return;
        const int64_t e = s + a.chunk < e_n ? s + a.chunk : e_n;
        if (active) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            auto token = [&](int64_t idx, float4 z) __attribute__((always_inline)) {
                float4 gv;
                gv.x = gm * fast_rcp(1.f + fast_exp2(ae.x * z.x));
                gv.y = gm * fast_rcp(1.f + fast_exp2(ae.y * z.y));
                gv.z = gm * fast_rcp(1.f + fast_exp2(ae.z * z.z));
                gv.w = gm * fast_rcp(1.f + fast_exp2(ae.w * z.w));
                acc.x += gv.x; acc.y += gv.y; acc.z += gv.z; acc.w += gv.w;
                if (g4) st_stream_f4(g4 + idx, gv);
                if (c4) st_stream_f4(c4 + idx, acc);
            };
            constexpr int kU = 4;
            int64_t t = s;
            if ((e - s) % kU == 0) {
                // whole groups of kU tokens: each group's inputs are loaded while the previous
                // group is computed, so a thread keeps up to 2 kU loads in flight
                float4 zb[2][kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) zb[0][u] = ld_stream_f4(z4 + (s + u) * ncol4 + col);
                for (int gi = 0; s + gi * kU < e; gi += 2) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int64_t tg = s + (gi + h2) * kU;
                        if (tg >= e) break;
                        if (tg + kU < e) {
#pragma unroll
                            for (int u = 0; u < kU; ++u) zb[h2 ^ 1][u] = ld_stream_f4(z4 + (tg + kU + u) * ncol4 + col);
                        }
#pragma unroll
                        for (int u = 0; u < kU; ++u) token((tg + u) * ncol4 + col, zb[h2][u]);
                    }
                }
                t = e;
            }
            for (; t < e; ++t) token(t * ncol4 + col, ld_stream_f4(z4 + t * ncol4 + col));
        }
        s = e;
    }
}

hipError_t launch_gate(const GateArgs& a, hipStream_t stream) {
    const int64_t windows = (a.total + a.chunk - 1) / a.chunk;
    const int64_t ncol4 = static_cast<int64_t>(a.H) * a.dk / 4;
    const dim3 grid(static_cast<unsigned>(windows * ((ncol4 + 255) / 256)));
    hipLaunchKernelGGL(gate_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
