// kda_prefill.hip -- fused chunkwise KDA prefill for gfx950 (MI355X).
//
// Sources (page title, section):
//   [K3 note] "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
//     §3.1  S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//           o_t = S_t^T q_t; Diag(alpha) scales rows (key channels) of S
//     §3.2  order of one edit: decay, predict at k, write beta k (v - vhat)^T, read after
//     §3.3  chunked prefill (X_[c], S_in) -> (Y_[c], S_out), state crossing only chunk
//           boundaries; lower-bounded gate g = g_min Sigmoid(e^A z), g_min = -5; a
//           16-token tile's cumulative log-decay lies in (-80, 0), so reciprocal decay
//           factors stay below e^80 and diagonal tiles use the same dense bf16 matrix
//           product as off-diagonal tiles.
//
// Chunk algebra (derived from §3.1/§3.2; the pages defer the WY/UT derivation to a note that
// is not among them).  For a chunk of n <= 64 tokens, incoming state S, chunk-local
// inclusive Gamma_r = sum_{i<=r} g_i (per key channel):
//   A_kk[i][j] = beta_i <k_i e^{Gamma_i}, k_j e^{-Gamma_j}>   (j < i)
//   A_qk[i][j] =        <q_i e^{Gamma_i}, k_j e^{-Gamma_j}>   (j <= i)
//   U  = (I + A_kk)^{-1} diag(beta) (V - (K e^{Gamma}) S)
//   O  = (Q e^{Gamma}) S + A_qk U
//   S' = diag(e^{Gamma_n}) S + (K e^{Gamma_n - Gamma})^T U
// The decayed products are factored per 16-token tile around rho_a (Gamma just before tile
// a): row operands carry e^{Gamma_i - rho_a} in [e^-80, 1], column operands e^{rho_a -
// Gamma_j}, which is <= 1 off the diagonal and < e^80 on it -- the pages' bound.
//
// Execution: one workgroup per (sequence, head, dv slice) walks that sequence's chunks in
// order, holding its dk x dv_slice fp32 state in MFMA accumulator registers.  Per chunk:
//   1. k, q, v, beta -> LDS; each gate item (tile, channel) evaluates 16 gates from z.
//   2. scaled bf16 operands -> LDS (tile-relative and chunk-relative decays).
//   3. the 10 lower 16x16 tiles of A_kk and A_qk (dense bf16 MFMA, diagonal included).
//   4. the four 16x16 diagonal blocks of (I + A_kk) inverted in fp32 (one wave).
//   5. wave w owns dv columns [16w, 16w+16) of the slice and, with no further barrier:
//      X = K~ S, Y = Q~ S (MFMA, S from registers); R = beta (V - X); block forward
//      substitution U_a = T_aa (R_a - sum_{b<a} L_ab U_b) in registers; O = Y + A_qk U;
//      S = diag(e^{Gamma_n}) S + K^n^T U.
// The state's rows are held in a permuted order pi(m, i) = 32(m/2) + 8(i/4) + 4(m%2) +
// i%4 (tile m, accumulator row i) so that a lane's accumulator rows are eight consecutive
// key channels: the K~ S product then takes S straight from registers as its B operand.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kChunk = 64;

template <int DK, int NW>
struct PrefillSmem {
    static constexpr int DVS = 16 * NW;    // dv columns per workgroup (16 per wave)
    static constexpr int KROW = DK + 8;    // bf16 row stride of [token][channel] arrays
    static constexpr int TROW = kChunk + 4;  // bf16 row stride of [*][token] arrays
    struct Raw {
        bf16_t k[kChunk][KROW];
        bf16_t q[kChunk][KROW];
    };
    struct Fac {
        float Ld[4][16][20];          // diagonal blocks of A_kk, [block][col j][row i]
        bf16_t negL[kChunk][TROW];    // -A_kk, row-major, off-diagonal blocks used
        bf16_t Td[kChunk][24];        // (I + L_aa)^{-1}, row 16a+i, column j
        bf16_t Aqk[kChunk][TROW];     // A_qk, row-major, lower blocks used
    };
    union {
        Raw raw;  // live while the operands are built
        Fac fac;  // live from the tile products to the end of the chunk
    } u;
    bf16_t Kr[kChunk][KROW];   // k_i e^{Gamma_i - rho_a}
    bf16_t Qr[kChunk][KROW];   // q_i e^{Gamma_i - rho_a}
    bf16_t Kc[kChunk][KROW];   // k_j e^{rho_{b+1} - Gamma_j}   (b = tile of j)
    bf16_t Kt[kChunk][KROW];   // k_i e^{Gamma_i}
    bf16_t Qt[kChunk][KROW];   // q_i e^{Gamma_i}
    bf16_t KnT[DK][TROW];      // (k_j e^{Gamma_n - Gamma_j})^T
    bf16_t Vt[DVS][TROW];      // v^T of this slice
    float beta[kChunk];
    float P[4][DK];            // e^{tile sum of g}, per tile and channel
    float colscale[7][DK];     // column-operand scales: 1/P_a (diagonal), P_1, P_1P_2, P_2
    float decayN[DK];          // e^{Gamma_n}
};

// Column-operand scale index of tile pair (a, b): -1 means 1.
__device__ __forceinline__ int colscale_index(int a, int b) {
    if (a == b) return a;
    if (a == 2 && b == 0) return 4;
    if (a == 3 && b == 0) return 5;
    if (a == 3 && b == 1) return 6;
    return -1;
}

__device__ __forceinline__ uint4 mask4(uint4 x, uint32_t m) {
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

__device__ __forceinline__ uint4 scale8(uint4 x, float4 s0, float4 s1) {
    return make_uint4(pack_bf16x2(lo_bf16(x.x) * s0.x, hi_bf16(x.x) * s0.y),
                      pack_bf16x2(lo_bf16(x.y) * s0.z, hi_bf16(x.y) * s0.w),
                      pack_bf16x2(lo_bf16(x.z) * s1.x, hi_bf16(x.z) * s1.y),
                      pack_bf16x2(lo_bf16(x.w) * s1.z, hi_bf16(x.w) * s1.w));
}

template <int DK, int NW, typename TIn>
__global__ void __launch_bounds__(NW * 64, 1) prefill_chain_kernel(PrefillArgs args) {
    using Smem = PrefillSmem<DK, NW>;
    constexpr int NT = NW * 64;
    constexpr int DVS = Smem::DVS;
    constexpr int IPT = 4 * DK / NT;     // gate items (tile, channel) per thread
    constexpr int KSTEPS = DK / 32;      // 32-channel steps of the K~ S product
    constexpr int MT = DK / 16;          // 16-row tiles of the state
    static_assert(4 * DK % NT == 0 && IPT >= 1, "gate items must divide the workgroup");

    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;

    // (sequence, head, slice) of this workgroup.  Consecutive workgroups are spread over
    // the 8 XCDs round-robin; the slices of one (sequence, head) land on the same XCD so
    // their shared q/k/z reads can hit that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, kq = bid >> 3;
    const int pair = (kq / args.nslices) * 8 + xcd;
    const int slice = kq % args.nslices;
    if (pair >= args.npairs) return;
    const int H = args.H;
    const int n = pair / H, h = pair - n * H;
    const int64_t tok0 = seq_start(args.cu, args.T, n);
    const int64_t tok1 = args.cu ? static_cast<int64_t>(args.cu[n + 1]) : tok0 + args.T;
    const int64_t len = tok1 - tok0;
    const int dv = DK;
    const int col0 = slice * DVS + 16 * w;  // first dv column of this wave
    const int64_t rowK = static_cast<int64_t>(H) * DK;
    const int64_t rowV = static_cast<int64_t>(H) * dv;

    const TIn* __restrict__ qg = static_cast<const TIn*>(args.q) + h * DK;
    const TIn* __restrict__ kg = static_cast<const TIn*>(args.k) + h * DK;
    const TIn* __restrict__ vg = static_cast<const TIn*>(args.v) + h * dv + slice * DVS;
    const TIn* __restrict__ bg = static_cast<const TIn*>(args.beta) + h;
    const float* __restrict__ zg = args.z + h * DK;
    TIn* __restrict__ og = static_cast<TIn*>(args.o) + h * dv;

    // gate constants per item: -e^{A} log2(e), and g_min log2(e)
    float aexp[IPT];
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
        const int c = (tid + it * NT) % DK;
        aexp[it] = -expf(args.A[h * DK + c]) * kLog2e;
    }
    const float gscale = args.g_min * kLog2e;

    // ---- state: Sacc[m][r] = S[pi(m, 4g + r)][col0 + li] --------------------------------
    f32x4_t Sacc[MT];
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * dv + col0 + li;
    if (args.s0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 32 * (m >> 1) + 8 * g + 4 * (m & 1) + r;
                Sacc[m][r] = args.s0[sbase + static_cast<size_t>(row) * dv];
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) Sacc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // ---- global loads of one chunk, issued back to back into registers ------------------
    // Rows past the sequence end are clamped to its last row (always a valid address) and
    // zeroed (k, q, v, beta) or given g = 0 (z) where they are consumed.  The next chunk's
    // loads are issued as soon as the current chunk's registers are consumed, so their
    // latency overlaps the current chunk's arithmetic.
    constexpr int KQ_PER = kChunk * (DK / 8) / NT;
    constexpr int V_PER = kChunk * (DVS / 8) / NT;
    static_assert(KQ_PER >= 1 && V_PER >= 1, "load split");
    uint4 pk[KQ_PER], pq[KQ_PER], pv[V_PER];
    float pz[IPT][16];
    float pb = 0.f;
    auto issue_loads = [&](int64_t t0, int clen) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KQ_PER; ++i) {
            const int idx = tid + i * NT, r = idx / (DK / 8), o8 = (idx % (DK / 8)) * 8;
            const int64_t off = (t0 + (r < clen ? r : clen - 1)) * rowK + o8;
            pk[i] = Elem<TIn>::load8(kg + off);
            pq[i] = Elem<TIn>::load8(qg + off);
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int idx = tid + i * NT, r = idx / (DVS / 8), o8 = (idx % (DVS / 8)) * 8;
            pv[i] = Elem<TIn>::load8(vg + (t0 + (r < clen ? r : clen - 1)) * rowV + o8);
        }
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int item = tid + it * NT, a = item / DK, c = item % DK;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * a + i;
                pz[it][i] = zg[(t0 + (r < clen ? r : clen - 1)) * rowK + c];
            }
        }
        const int rb = (tid & (kChunk - 1)) < clen ? (tid & (kChunk - 1)) : clen - 1;
        pb = Elem<TIn>::load1(bg + (t0 + rb) * H);
    };
    if (len > 0) issue_loads(tok0, len < kChunk ? static_cast<int>(len) : kChunk);

    for (int64_t c0 = 0; c0 < len; c0 += kChunk) {
        const int clen = static_cast<int>(len - c0 < kChunk ? len - c0 : kChunk);
        const int64_t t0 = tok0 + c0;

        __syncthreads();  // the previous chunk's readers are done with every buffer

        // ---- 1. raw k, q, v^T, beta -> LDS (rows past the sequence end are zero) ---------
#pragma unroll
        for (int i = 0; i < KQ_PER; ++i) {
            const int idx = tid + i * NT, r = idx / (DK / 8), o8 = (idx % (DK / 8)) * 8;
            const uint32_t keep = r < clen ? 0xffffffffu : 0u;  // mask by value, not by select
            *reinterpret_cast<uint4*>(&sm.u.raw.k[r][o8]) = mask4(pk[i], keep);
            *reinterpret_cast<uint4*>(&sm.u.raw.q[r][o8]) = mask4(pq[i], keep);
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int idx = tid + i * NT, r = idx / (DVS / 8), o8 = (idx % (DVS / 8)) * 8;
            const uint4 vv = mask4(pv[i], r < clen ? 0xffffffffu : 0u);
            const uint32_t wv[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sm.Vt[o8 + 2 * e][r] = static_cast<bf16_t>(wv[e] & 0xffffu);
                sm.Vt[o8 + 2 * e + 1][r] = static_cast<bf16_t>(wv[e] >> 16);
            }
        }
        if (tid < kChunk) sm.beta[tid] = tid < clen ? pb : 0.f;

        // gate, pass 1: alpha = e^g for 16 tokens of one (tile, channel); tile product P.
        // Masked tokens get alpha = 1 (g = 0) so they leave every decay factor unchanged.
        float alpha[IPT][16];
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int item = tid + it * NT, a = item / DK, c = item % DK;
            float F = 1.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float ex = fast_exp2(aexp[it] * pz[it][i]);  // e^{-e^A z}
                const float s = fast_rcp(1.f + ex);                 // Sigmoid(e^A z)
                const float al = fast_exp2(gscale * s);             // e^{g_min Sigmoid}
                alpha[it][i] = (16 * a + i < clen) ? al : 1.f;
                F *= alpha[it][i];
            }
            sm.P[a][c] = F;
        }
        // every prefetch register is consumed: start the next chunk's loads
        if (c0 + kChunk < len) {
            const int64_t rem = len - c0 - kChunk;
            issue_loads(t0 + kChunk, rem < kChunk ? static_cast<int>(rem) : kChunk);
        }
        __syncthreads();

        // ---- 2. scaled operands ---------------------------------------------------------
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int item = tid + it * NT, a = item / DK, c = item % DK;
            const float P0 = sm.P[0][c], P1 = sm.P[1][c], P2 = sm.P[2][c], P3 = sm.P[3][c];
            const float Pa[4] = {P0, P1, P2, P3};
            float eR = 1.f, eN = 1.f;  // e^{rho_a}, e^{Gamma_n - rho_{a+1}}
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                eR *= (t < a) ? Pa[t] : 1.f;
                eN *= (t > a) ? Pa[t] : 1.f;
            }
            float E[16];  // e^{rho_{a+1} - Gamma_i}: product of the later alphas in the tile
            E[15] = 1.f;
#pragma unroll
            for (int i = 14; i >= 0; --i) E[i] = E[i + 1] * alpha[it][i + 1];
            float F = 1.f;
            float kn[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * a + i;
                F *= alpha[it][i];  // e^{Gamma_i - rho_a}
                const float kf = bf16_to_f32(sm.u.raw.k[r][c]);
                const float qf = bf16_to_f32(sm.u.raw.q[r][c]);
                const float kr = kf * F, qr = qf * F, kc = kf * E[i];
                sm.Kr[r][c] = f32_to_bf16(kr);
                sm.Qr[r][c] = f32_to_bf16(qr);
                sm.Kc[r][c] = f32_to_bf16(kc);
                sm.Kt[r][c] = f32_to_bf16(kr * eR);
                sm.Qt[r][c] = f32_to_bf16(qr * eR);
                kn[i] = kc * eN;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint2*>(&sm.KnT[c][16 * a + 4 * j]) =
                    make_uint2(pack_bf16x2(kn[4 * j], kn[4 * j + 1]),
                               pack_bf16x2(kn[4 * j + 2], kn[4 * j + 3]));
            if (a == 0) {
                sm.colscale[0][c] = fast_rcp(P0);
                sm.colscale[1][c] = fast_rcp(P1);
                sm.colscale[2][c] = fast_rcp(P2);
                sm.colscale[3][c] = fast_rcp(P3);
                sm.colscale[4][c] = P1;
                sm.colscale[5][c] = P1 * P2;
                sm.colscale[6][c] = P2;
                sm.decayN[c] = P0 * P1 * P2 * P3;
            }
        }
        __syncthreads();

        // ---- 3. lower 16x16 tiles of A_kk and A_qk -----------------------------------------
        // The product is taken transposed (column operand as MFMA A) so that each lane ends
        // with four consecutive columns j of one row i.
        for (int job = w; job < 10; job += NW) {
            const int a = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
            const int b = job - (a * (a + 1)) / 2;
            const int si = colscale_index(a, b);
            f32x4_t ckk = {0.f, 0.f, 0.f, 0.f}, cqk = ckk;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int ch = 32 * s + 8 * g;
                uint4 col = *reinterpret_cast<const uint4*>(&sm.Kc[16 * b + li][ch]);
                if (si >= 0)
                    col = scale8(col, *reinterpret_cast<const float4*>(&sm.colscale[si][ch]),
                                 *reinterpret_cast<const float4*>(&sm.colscale[si][ch + 4]));
                const uint4 kr = *reinterpret_cast<const uint4*>(&sm.Kr[16 * a + li][ch]);
                const uint4 qr = *reinterpret_cast<const uint4*>(&sm.Qr[16 * a + li][ch]);
                ckk = mfma32(col, kr, ckk);
                cqk = mfma32(col, qr, cqk);
            }
            // ckk[r] = <k~_i, k^_j> with i = 16a + li, j = 16b + 4g + r
            const float bi = sm.beta[16 * a + li];
            if (a == b) {
                float qv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jj = 4 * g + r;
                    sm.u.fac.Ld[a][jj][li] = jj < li ? bi * ckk[r] : 0.f;  // strictly lower
                    qv[r] = jj <= li ? cqk[r] : 0.f;                      // lower incl. diag
                }
                *reinterpret_cast<uint2*>(&sm.u.fac.Aqk[16 * a + li][16 * b + 4 * g]) =
                    make_uint2(pack_bf16x2(qv[0], qv[1]), pack_bf16x2(qv[2], qv[3]));
            } else {
                *reinterpret_cast<uint2*>(&sm.u.fac.negL[16 * a + li][16 * b + 4 * g]) =
                    make_uint2(pack_bf16x2(-bi * ckk[0], -bi * ckk[1]),
                               pack_bf16x2(-bi * ckk[2], -bi * ckk[3]));
                *reinterpret_cast<uint2*>(&sm.u.fac.Aqk[16 * a + li][16 * b + 4 * g]) =
                    make_uint2(pack_bf16x2(cqk[0], cqk[1]), pack_bf16x2(cqk[2], cqk[3]));
            }
        }
        __syncthreads();

        // ---- 4. diagonal inverses (last wave) while every wave forms X = K~S, Y = Q~S -----
        if (w == NW - 1) {
            const int a = lane >> 4, j = lane & 15;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                float Lm[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 v4 = *reinterpret_cast<const float4*>(&sm.u.fac.Ld[a][m][4 * q4]);
                    Lm[4 * q4] = v4.x; Lm[4 * q4 + 1] = v4.y; Lm[4 * q4 + 2] = v4.z; Lm[4 * q4 + 3] = v4.w;
                }
                const float tm = t[m];
#pragma unroll
                for (int i = m + 1; i < 16; ++i) t[i] -= Lm[i] * tm;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.u.fac.Td[16 * a + i][j] = f32_to_bf16(t[i]);
        }

        uint4 Sb[KSTEPS];  // bf16 S as the B operand: slot e of lane g <-> channel 32s+8g+e
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            Sb[s] = make_uint4(pack_bf16x2(Sacc[2 * s][0], Sacc[2 * s][1]),
                               pack_bf16x2(Sacc[2 * s][2], Sacc[2 * s][3]),
                               pack_bf16x2(Sacc[2 * s + 1][0], Sacc[2 * s + 1][1]),
                               pack_bf16x2(Sacc[2 * s + 1][2], Sacc[2 * s + 1][3]));
        f32x4_t R[4], Y[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t X = {0.f, 0.f, 0.f, 0.f};
            Y[a] = X;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int ch = 32 * s + 8 * g;
                X = mfma32(*reinterpret_cast<const uint4*>(&sm.Kt[16 * a + li][ch]), Sb[s], X);
                Y[a] = mfma32(*reinterpret_cast<const uint4*>(&sm.Qt[16 * a + li][ch]), Sb[s], Y[a]);
            }
            // R = beta (V - X) at rows 16a + 4g + r, column col0 + li
            const uint2 vv = *reinterpret_cast<const uint2*>(&sm.Vt[16 * w + li][16 * a + 4 * g]);
            const float4 bb = *reinterpret_cast<const float4*>(&sm.beta[16 * a + 4 * g]);
            R[a][0] = bb.x * (lo_bf16(vv.x) - X[0]);
            R[a][1] = bb.y * (hi_bf16(vv.x) - X[1]);
            R[a][2] = bb.z * (lo_bf16(vv.y) - X[2]);
            R[a][3] = bb.w * (hi_bf16(vv.y) - X[3]);
        }
        __syncthreads();

        // ---- 5. forward substitution, output, state update (wave-local) -------------------
        uint2 Ub[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t acc = R[a];
#pragma unroll
            for (int b = 0; b < a; ++b)
                acc = mfma16(*reinterpret_cast<const uint2*>(&sm.u.fac.negL[16 * a + li][16 * b + 4 * g]),
                             Ub[b], acc);
            const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t uf = mfma16(*reinterpret_cast<const uint2*>(&sm.u.fac.Td[16 * a + li][4 * g]),
                                      pack_bf16x4(acc), zero);
            Ub[a] = pack_bf16x4(uf);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t oacc = Y[a];
#pragma unroll
            for (int b = 0; b <= a; ++b)
                oacc = mfma16(*reinterpret_cast<const uint2*>(&sm.u.fac.Aqk[16 * a + li][16 * b + 4 * g]),
                              Ub[b], oacc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * a + 4 * g + r;
                if (tr < clen) Elem<TIn>::store1(og + (t0 + tr) * rowV + col0 + li, oacc[r]);
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int s = m >> 1, hh = m & 1;
            const float4 dn = *reinterpret_cast<const float4*>(&sm.decayN[32 * s + 8 * g + 4 * hh]);
            Sacc[m][0] *= dn.x;
            Sacc[m][1] *= dn.y;
            Sacc[m][2] *= dn.z;
            Sacc[m][3] *= dn.w;
            const int krow = 32 * s + 8 * (li >> 2) + 4 * hh + (li & 3);  // pi(m, li)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const uint2 a0 = *reinterpret_cast<const uint2*>(&sm.KnT[krow][32 * sp + 4 * g]);
                const uint2 a1 = *reinterpret_cast<const uint2*>(&sm.KnT[krow][32 * sp + 16 + 4 * g]);
                Sacc[m] = mfma32(make_uint4(a0.x, a0.y, a1.x, a1.y),
                                 make_uint4(Ub[2 * sp].x, Ub[2 * sp].y, Ub[2 * sp + 1].x,
                                            Ub[2 * sp + 1].y),
                                 Sacc[m]);
            }
        }
    }

    if (args.sN) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 32 * (m >> 1) + 8 * g + 4 * (m & 1) + r;
                args.sN[sbase + static_cast<size_t>(row) * dv] = Sacc[m][r];
            }
        }
    }
}

template <int DK, int NW, typename TIn>
static hipError_t launch_chain(const PrefillArgs& a, hipStream_t stream) {
    PrefillArgs args = a;
    args.nslices = DK / (16 * NW);
    const int groups = (args.npairs + 7) / 8;
    const dim3 grid(static_cast<unsigned>(groups) * 8u * static_cast<unsigned>(args.nslices));
    hipLaunchKernelGGL((prefill_chain_kernel<DK, NW, TIn>), grid, dim3(NW * 64), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int dk, bool bf16, int waves, hipStream_t stream) {
    if (dk == 128) {
        if (waves == 8)
            return bf16 ? launch_chain<128, 8, bf16_t>(a, stream) : launch_chain<128, 8, float>(a, stream);
        return bf16 ? launch_chain<128, 4, bf16_t>(a, stream) : launch_chain<128, 4, float>(a, stream);
    }
    return bf16 ? launch_chain<64, 4, bf16_t>(a, stream) : launch_chain<64, 4, float>(a, stream);
}

}  // namespace kda
