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
    // state tile of this thread: rows rg + ROWG*i, columns 4cg .. 4cg+3
    const int cg = tid % COLG, rg = tid / COLG;
    f32x4_t* __restrict__ st = reinterpret_cast<f32x4_t*>(args.state + static_cast<size_t>(pair) * D * D);
    float4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const f32x4_t t = __builtin_nontemporal_load(&st[(rg + ROWG * i) * COLG + cg]);
        S[i] = make_float4(t[0], t[1], t[2], t[3]);
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
