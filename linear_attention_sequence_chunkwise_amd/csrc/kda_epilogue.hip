// kda_epilogue.hip -- fused KDA output epilogue for gfx950: y = Sigmoid(gate) * RMSNorm(o).
//
// [K3 note] = "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
//   §3.2  the K3 output path W_o[Sigmoid(W_g x_t) (.) RMSNorm(o~_t)]: RMSNorm stabilises the
//         recurrent readout, the current token's full-rank channel gate selects what reaches
//         the residual stream.  The projections W_g, W_o need trained weights; the gate logits
//         arrive as an input.  RMSNorm is taken per (token, head) over the d_v readout
//         channels with a per-channel weight w and eps inside the root.
//
// One row = one token of one head (d_v contiguous elements).  Each lane owns 8 consecutive
// channels (one 16-byte load of bf16), so a row of 128 is 16 lanes and a wave covers four
// rows per step; the sum of squares is a butterfly over the row's lanes.  Memory-bound:
// 2 reads and 1 write of the row in the element type.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
    __device__ __forceinline__ static void load(const bf16_t* p, float* x) {
        const uint4 u = ld_stream16(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = lo_bf16(w[i]); x[2 * i + 1] = hi_bf16(w[i]); }
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float* x) {
        st_stream16(p, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                  pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
    }
};
template <> struct Vec8<float> {
    __device__ __forceinline__ static void load(const float* p, float* x) {
        const float4 a = ld_stream_f4(p), b = ld_stream_f4(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
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

}  // namespace

template <int DV, typename T>
__global__ void __launch_bounds__(256) output_gate_kernel(OutputGateArgs a) {
    constexpr int LPR = DV / 8;           // lanes per row
    constexpr int RPW = 64 / LPR;         // rows per wave per step
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR, c8 = (lane % LPR) * 8;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
    float w[8];
    {
        const float4 w0 = *reinterpret_cast<const float4*>(a.w + c8);
        const float4 w1 = *reinterpret_cast<const float4*>(a.w + c8 + 4);
        w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w; w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
    }
    const T* o = static_cast<const T*>(a.o);
    const T* gt = static_cast<const T*>(a.gate);
    T* y = static_cast<T*>(a.y);
    constexpr int U = 4;  // row groups in flight per lane
    for (int64_t r0 = wave * RPW * U; r0 < a.rows; r0 += nwaves * RPW * U) {
        float x[U][8], g[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = r0 + u * RPW + sub;
            if (r < a.rows) {
                Vec8<T>::load(o + r * DV + c8, x[u]);
                Vec8<T>::load(gt + r * DV + c8, g[u]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) { x[u][i] = 0.f; g[u][i] = 0.f; }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = r0 + u * RPW + sub;
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += x[u][i] * x[u][i];
            // the row's LPR lanes are one DPP row (16) or half-row (8): quads, then the two
            // quads of each half-row (mirror), then the two half-rows, all without LDS
            static_assert(LPR == 8 || LPR == 16, "rows of 64 or 128 channels");
            ss += dpp_f32<0xB1>(ss);   // quad_perm [1,0,3,2]
            ss += dpp_f32<0x4E>(ss);   // quad_perm [2,3,0,1]
            ss += dpp_f32<0x141>(ss);  // row_half_mirror
            if constexpr (LPR == 16) ss += dpp_f32<0x128>(ss);  // row_ror:8
            const float inv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + a.eps);
            float out[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float sg = fast_rcp(1.f + fast_exp2(-g[u][i] * kLog2e));
                out[i] = x[u][i] * inv * w[i] * sg;
            }
            if (r < a.rows) Vec8<T>::store(y + r * DV + c8, out);
        }
    }
}

hipError_t launch_output_gate(const OutputGateArgs& a, int dv, bool bf16, hipStream_t stream) {
    const int64_t rows_per_block = 4 * 4 * (64 / (dv / 8));
    int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 16384) blocks = 16384;  // grid-stride beyond that
    const dim3 grid(static_cast<unsigned>(blocks));
    if (dv == 128) {
        if (bf16) hipLaunchKernelGGL((output_gate_kernel<128, bf16_t>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((output_gate_kernel<128, float>), grid, dim3(256), 0, stream, a);
    } else {
        if (bf16) hipLaunchKernelGGL((output_gate_kernel<64, bf16_t>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((output_gate_kernel<64, float>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kda
