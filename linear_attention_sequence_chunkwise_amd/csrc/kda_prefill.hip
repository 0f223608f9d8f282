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
// Gamma_j}, which is <= 1 off the diagonal and < e^80 on it -- the pages' bound.  Decays
// are cumulative products of alpha = e^g, never exponentials of large sums.
//
// Execution: one workgroup per (sequence, head, dv slice) walks that sequence's chunks in
// order, holding its dk x dv_slice fp32 state in MFMA accumulator registers.  Per chunk:
//   1. v rows and beta -> LDS; each gate item (segment of SEG tokens, channel pair)
//      evaluates its gates from z held in registers.
//   2. scaled bf16 operands -> LDS (tile-relative and chunk-relative decays); the next
//      chunk's global loads are issued.
//   3. the 10 lower 16x16 tiles of A_kk and A_qk (dense bf16 MFMA, diagonal included).
//   4. the four 16x16 diagonal blocks of (I + A_kk) inverted in fp32 (one wave) while
//      every wave forms X = K~ S and Y = Q~ S with S taken from its registers.
//   5. wave w owns dv columns [16w, 16w+16) of the slice and, with no further barrier:
//      R = beta (V - X); block forward substitution U_a = T_aa (R_a - sum_{b<a} L_ab U_b)
//      in registers; O = Y + A_qk U (staged through LDS, stored 16 bytes per lane);
//      S = diag(e^{Gamma_n}) S + K^n^T U.
// The state's rows are held in a permuted order pi(m, i) = 32(m/2) + 8(i/4) + 4(m%2) +
// i%4 (tile m, accumulator row i) so that a lane's accumulator rows are eight consecutive
// key channels: the K~ S product then takes S straight from registers as its B operand.
//
// Global memory goes through buffer descriptors rebased at each chunk's first token with a
// size of (valid rows) x (row bytes): rows past a sequence's end read as zero and their
// stores are dropped.  LDS rows are padded (288-byte rows for 16-byte operand reads,
// 144-byte rows for 8-byte reads), strides at which 16 rows by 4 columns of those reads
// hit distinct banks on gfx950.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kChunk = 64;

template <int DK, int NW>
struct PrefillSmem {
    static constexpr int NT = 64 * NW;
    static constexpr int DVS = 16 * NW;      // dv columns per workgroup (16 per wave)
    static constexpr int KROW = DK + 16;     // [token][channel] rows
    static constexpr int TROW = kChunk + 8;  // [channel or token][token] rows
    static constexpr int VROW = DVS + 16;    // [token][dv] rows of v / staged output
    static constexpr int SEG = 32 * DK / NT; // tokens per gate item (items = segments x pairs)
    static constexpr int NSEG = kChunk / SEG;
    struct Fac {
        float Ld[4][16][20];          // diagonal blocks of A_kk, [block][col j][row i]
        bf16_t negL[kChunk][TROW];    // -A_kk, row-major, off-diagonal blocks used
        bf16_t Td[kChunk][24];        // (I + L_aa)^{-1}, row 16a+i, column j
        bf16_t Aqk[kChunk][TROW];     // A_qk, row-major, lower blocks used
    };
    union {
        float Pseg[NSEG][DK];  // per-segment alpha products (steps 1-2)
        Fac fac;               // steps 3-5
    } u;
    bf16_t Kr[kChunk][KROW];   // k_i e^{Gamma_i - rho_a}
    bf16_t Qr[kChunk][KROW];   // q_i e^{Gamma_i - rho_a}
    bf16_t Kc[kChunk][KROW];   // k_j e^{rho_{b+1} - Gamma_j}   (b = tile of j)
    bf16_t Kt[kChunk][KROW];   // k_i e^{Gamma_i}
    bf16_t Qt[kChunk][KROW];   // q_i e^{Gamma_i}
    bf16_t KnT[DK][TROW];      // (k_j e^{Gamma_n - Gamma_j})^T
    bf16_t V[kChunk][VROW];    // v of this slice; each wave's 16 columns then stage its O
    float beta[kChunk];
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

__device__ __forceinline__ uint4 scale8(uint4 x, float4 s0, float4 s1) {
    return make_uint4(pack_bf16x2(lo_bf16(x.x) * s0.x, hi_bf16(x.x) * s0.y),
                      pack_bf16x2(lo_bf16(x.y) * s0.z, hi_bf16(x.y) * s0.w),
                      pack_bf16x2(lo_bf16(x.z) * s1.x, hi_bf16(x.z) * s1.y),
                      pack_bf16x2(lo_bf16(x.w) * s1.z, hi_bf16(x.w) * s1.w));
}

// Per-element-type access for the gate items (two channels per token) and v rows.
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
    typedef uint32_t raw;  // two bf16
    __device__ __forceinline__ static raw load(rsrc_t r, uint32_t off) { return bload4(r, off); }
    __device__ __forceinline__ static float2 get(raw x) { return make_float2(lo_bf16(x), hi_bf16(x)); }
    struct Row8 { uint4 a; };  // eight bf16
    __device__ __forceinline__ static Row8 load8(rsrc_t r, uint32_t off) { return Row8{bload16(r, off)}; }
    __device__ __forceinline__ static uint4 bf16x8(const Row8& x) { return x.a; }
    __device__ __forceinline__ static float load_beta(rsrc_t r, uint32_t off) {
        return __uint_as_float(bload2(r, off) << 16);
    }
};
template <> struct Pair<float> {
    typedef uint2 raw;  // two fp32
    __device__ __forceinline__ static raw load(rsrc_t r, uint32_t off) { return bload8(r, off); }
    __device__ __forceinline__ static float2 get(raw x) {
        return make_float2(__uint_as_float(x.x), __uint_as_float(x.y));
    }
    struct Row8 { uint4 a, b; };  // eight fp32
    __device__ __forceinline__ static Row8 load8(rsrc_t r, uint32_t off) {
        return Row8{bload16(r, off), bload16(r, off + 16)};
    }
    __device__ __forceinline__ static uint4 bf16x8(const Row8& x) {
        return make_uint4(pack_bf16x2(__uint_as_float(x.a.x), __uint_as_float(x.a.y)),
                          pack_bf16x2(__uint_as_float(x.a.z), __uint_as_float(x.a.w)),
                          pack_bf16x2(__uint_as_float(x.b.x), __uint_as_float(x.b.y)),
                          pack_bf16x2(__uint_as_float(x.b.z), __uint_as_float(x.b.w)));
    }
    __device__ __forceinline__ static float load_beta(rsrc_t r, uint32_t off) {
        return __uint_as_float(bload4(r, off));
    }
};

template <int DK, int NW, typename TIn>
__global__ void __launch_bounds__(NW * 64, 1) prefill_chain_kernel(PrefillArgs args) {
    using Smem = PrefillSmem<DK, NW>;
    using P = Pair<TIn>;
    constexpr int NT = Smem::NT;
    constexpr int DVS = Smem::DVS;
    constexpr int SEG = Smem::SEG;
    constexpr int NSEG = Smem::NSEG;
    constexpr int SPT = 16 / SEG;             // segments per 16-token tile (1 or 2)
    constexpr int NCP = DK / 2;               // channel pairs
    constexpr int KSTEPS = DK / 32;           // 32-channel steps of the K~ S product
    constexpr int MT = DK / 16;               // 16-row tiles of the state
    constexpr int ES = static_cast<int>(sizeof(TIn));
    constexpr int V_PER = kChunk * (DVS / 8) / NT;  // 8-element v loads per thread
    static_assert(NSEG * NCP == NT && SEG * NSEG == kChunk && (SEG == 8 || SEG == 16), "items");
    static_assert(V_PER >= 1, "v load split");

    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;

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
    const uint32_t rowK = static_cast<uint32_t>(H) * DK * ES;  // bytes per token of q, k
    const uint32_t rowZ = static_cast<uint32_t>(H) * DK * 4;   // bytes per token of z
    const uint32_t rowV = static_cast<uint32_t>(H) * dv * ES;  // bytes per token of v, o
    const uint32_t rowB = static_cast<uint32_t>(H) * ES;       // bytes per token of beta

    const char* kbase = static_cast<const char*>(args.k) + static_cast<size_t>(h) * DK * ES;
    const char* qbase = static_cast<const char*>(args.q) + static_cast<size_t>(h) * DK * ES;
    const char* vbase = static_cast<const char*>(args.v) + (static_cast<size_t>(h) * dv + slice * DVS) * ES;
    const char* bbase = static_cast<const char*>(args.beta) + static_cast<size_t>(h) * ES;
    const char* zbase = reinterpret_cast<const char*>(args.z) + static_cast<size_t>(h) * DK * 4;
    char* obase = static_cast<char*>(args.o) + (static_cast<size_t>(h) * dv + col0) * ES;

    // gate item of this thread: segment iseg (tokens SEG*iseg ..), channels ch0, ch0 + 1
    const int icp = tid % NCP, iseg = tid / NCP, ch0 = 2 * icp;
    const int itile = iseg / SPT, isub = iseg % SPT;
    const float ae0 = -expf(args.A[h * DK + ch0]) * kLog2e;  // -e^{A} log2(e)
    const float ae1 = -expf(args.A[h * DK + ch0 + 1]) * kLog2e;
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

    // ---- global loads of one chunk into registers ---------------------------------------
    // Each gate item loads its own k, q, z (two channels x SEG tokens); v rows and beta go
    // to LDS.  The next chunk's loads are issued once the current ones are consumed, so
    // their latency overlaps the tile products and the state pass.
    typename P::raw pk[SEG], pq[SEG];
    uint2 pz[SEG];
    typename P::Row8 pv[V_PER];
    float pb = 0.f;
    auto issue_loads = [&](int64_t t0, int clen) __attribute__((always_inline)) {
        const rsrc_t rk = make_rsrc(kbase + t0 * rowK, clen * rowK);
        const rsrc_t rq = make_rsrc(qbase + t0 * rowK, clen * rowK);
        const rsrc_t rz = make_rsrc(zbase + t0 * rowZ, clen * rowZ);
        const rsrc_t rv = make_rsrc(vbase + t0 * rowV, clen * rowV);
        const rsrc_t rb = make_rsrc(bbase + t0 * rowB, clen * rowB);
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const uint32_t row = static_cast<uint32_t>(iseg * SEG + i);
            pk[i] = P::load(rk, row * rowK + ch0 * ES);
            pq[i] = P::load(rq, row * rowK + ch0 * ES);
            pz[i] = bload8(rz, row * rowZ + ch0 * 4);
        }
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int idx = tid + i * NT, r = idx / (DVS / 8), o8 = (idx % (DVS / 8)) * 8;
            pv[i] = P::load8(rv, r * rowV + o8 * ES);
        }
        pb = P::load_beta(rb, (tid & (kChunk - 1)) * rowB);
    };
    if (len > 0) issue_loads(tok0, len < kChunk ? static_cast<int>(len) : kChunk);

    for (int64_t c0 = 0; c0 < len; c0 += kChunk) {
        const int clen = static_cast<int>(len - c0 < kChunk ? len - c0 : kChunk);
        const int64_t t0 = tok0 + c0;

        lds_barrier();  // the previous chunk's readers are done with every buffer

        // ---- 1. v rows and beta -> LDS; gates -> alpha; per-segment alpha products --------
#pragma unroll
        for (int i = 0; i < V_PER; ++i) {
            const int idx = tid + i * NT, r = idx / (DVS / 8), o8 = (idx % (DVS / 8)) * 8;
            *reinterpret_cast<uint4*>(&sm.V[r][o8]) = P::bf16x8(pv[i]);
        }
        if (tid < kChunk) sm.beta[tid] = pb;
        // alpha = e^{g}, g = g_min Sigmoid(e^A z); tokens past the end get alpha = 1 (g = 0)
        float2 al[SEG];
        float2 Pq = make_float2(1.f, 1.f);
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const bool valid = iseg * SEG + i < clen;
            const float s0 = fast_rcp(1.f + fast_exp2(ae0 * __uint_as_float(pz[i].x)));
            const float s1 = fast_rcp(1.f + fast_exp2(ae1 * __uint_as_float(pz[i].y)));
            al[i].x = valid ? fast_exp2(gscale * s0) : 1.f;
            al[i].y = valid ? fast_exp2(gscale * s1) : 1.f;
            Pq.x *= al[i].x;
            Pq.y *= al[i].y;
        }
        *reinterpret_cast<float2*>(&sm.u.Pseg[iseg][ch0]) = Pq;
        lds_barrier();

        // ---- 2. scaled operands --------------------------------------------------------
        {
            float2 ps[NSEG];
#pragma unroll
            for (int s = 0; s < NSEG; ++s) ps[s] = *reinterpret_cast<const float2*>(&sm.u.Pseg[s][ch0]);
            float2 T[4];  // tile products e^{rho_{a+1} - rho_a}
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                T[a] = ps[a * SPT];
                if (SPT == 2) { T[a].x *= ps[a * SPT + 1].x; T[a].y *= ps[a * SPT + 1].y; }
            }
            float2 eR = make_float2(1.f, 1.f), eN = eR;  // e^{rho_a}, e^{Gamma_n - rho_{a+1}}
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                if (a < itile) { eR.x *= T[a].x; eR.y *= T[a].y; }
                if (a > itile) { eN.x *= T[a].x; eN.y *= T[a].y; }
            }
            // products of the tile's other segment before / after this one
            float2 pre = make_float2(1.f, 1.f), post = pre;
            if (SPT == 2) {
                const float2 other = *reinterpret_cast<const float2*>(&sm.u.Pseg[iseg ^ 1][ch0]);
                if (isub == 1) pre = other;
                else post = other;
            }
            float2 E[SEG];  // e^{rho_{a+1} - Gamma_i}
            E[SEG - 1] = post;
#pragma unroll
            for (int i = SEG - 2; i >= 0; --i)
                E[i] = make_float2(E[i + 1].x * al[i + 1].x, E[i + 1].y * al[i + 1].y);
            float2 F = pre;  // e^{Gamma_i - rho_a}
            float2 kn[SEG];
#pragma unroll
            for (int i = 0; i < SEG; ++i) {
                const int r = iseg * SEG + i;
                F.x *= al[i].x;
                F.y *= al[i].y;
                const float2 kf = P::get(pk[i]), qf = P::get(pq[i]);
                const float2 FR = make_float2(F.x * eR.x, F.y * eR.y);
                *reinterpret_cast<uint32_t*>(&sm.Kr[r][ch0]) = pack_bf16x2(kf.x * F.x, kf.y * F.y);
                *reinterpret_cast<uint32_t*>(&sm.Qr[r][ch0]) = pack_bf16x2(qf.x * F.x, qf.y * F.y);
                *reinterpret_cast<uint32_t*>(&sm.Kc[r][ch0]) = pack_bf16x2(kf.x * E[i].x, kf.y * E[i].y);
                *reinterpret_cast<uint32_t*>(&sm.Kt[r][ch0]) = pack_bf16x2(kf.x * FR.x, kf.y * FR.y);
                *reinterpret_cast<uint32_t*>(&sm.Qt[r][ch0]) = pack_bf16x2(qf.x * FR.x, qf.y * FR.y);
                kn[i] = make_float2(kf.x * (E[i].x * eN.x), kf.y * (E[i].y * eN.y));
            }
#pragma unroll
            for (int j = 0; j < SEG / 4; ++j) {
                const int tk = iseg * SEG + 4 * j;
                *reinterpret_cast<uint2*>(&sm.KnT[ch0][tk]) =
                    make_uint2(pack_bf16x2(kn[4 * j].x, kn[4 * j + 1].x),
                               pack_bf16x2(kn[4 * j + 2].x, kn[4 * j + 3].x));
                *reinterpret_cast<uint2*>(&sm.KnT[ch0 + 1][tk]) =
                    make_uint2(pack_bf16x2(kn[4 * j].y, kn[4 * j + 1].y),
                               pack_bf16x2(kn[4 * j + 2].y, kn[4 * j + 3].y));
            }
            if (iseg == 0) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float T0 = e ? T[0].y : T[0].x, T1 = e ? T[1].y : T[1].x;
                    const float T2 = e ? T[2].y : T[2].x, T3 = e ? T[3].y : T[3].x;
                    const int c = ch0 + e;
                    sm.colscale[0][c] = fast_rcp(T0);
                    sm.colscale[1][c] = fast_rcp(T1);
                    sm.colscale[2][c] = fast_rcp(T2);
                    sm.colscale[3][c] = fast_rcp(T3);
                    sm.colscale[4][c] = T1;
                    sm.colscale[5][c] = T1 * T2;
                    sm.colscale[6][c] = T2;
                    sm.decayN[c] = T0 * T1 * T2 * T3;
                }
            }
        }
        // every prefetch register is consumed: start the next chunk's loads
        if (c0 + kChunk < len) {
            const int64_t rem = len - c0 - kChunk;
            issue_loads(t0 + kChunk, rem < kChunk ? static_cast<int>(rem) : kChunk);
        }
        lds_barrier();

        // ---- 3. lower 16x16 tiles of A_kk and A_qk -----------------------------------------
        // The product is taken transposed (column operand as MFMA A) so that each lane ends
        // with four consecutive columns j of one row i.  Wave w takes jobs w, w+NW, ...
#pragma unroll
        for (int slot = 0; slot < (10 + NW - 1) / NW; ++slot) {
            const int job = w + slot * NW;
            if (job < 10) {
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
        }
        lds_barrier();

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
            const float4 bb = *reinterpret_cast<const float4*>(&sm.beta[16 * a + 4 * g]);
            const int vc = 16 * w + li;
            R[a][0] = bb.x * (bf16_to_f32(sm.V[16 * a + 4 * g + 0][vc]) - X[0]);
            R[a][1] = bb.y * (bf16_to_f32(sm.V[16 * a + 4 * g + 1][vc]) - X[1]);
            R[a][2] = bb.z * (bf16_to_f32(sm.V[16 * a + 4 * g + 2][vc]) - X[2]);
            R[a][3] = bb.w * (bf16_to_f32(sm.V[16 * a + 4 * g + 3][vc]) - X[3]);
        }
        lds_barrier();

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
        const rsrc_t ro = make_rsrc(obase + t0 * rowV, clen * rowV);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t oacc = Y[a];
#pragma unroll
            for (int b = 0; b <= a; ++b)
                oacc = mfma16(*reinterpret_cast<const uint2*>(&sm.u.fac.Aqk[16 * a + li][16 * b + 4 * g]),
                              Ub[b], oacc);
            if constexpr (sizeof(TIn) == 2) {
                // stage in this wave's own v columns (no other wave reads them any more)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.V[16 * a + 4 * g + r][16 * w + li] = f32_to_bf16(oacc[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    bstore4(ro, (16 * a + 4 * g + r) * rowV + li * 4, __float_as_uint(oacc[r]));
            }
        }
        if constexpr (sizeof(TIn) == 2) {
            // each lane stores one token row of the wave's 16 columns: 2 x 16 bytes
            const uint4 o0 = *reinterpret_cast<const uint4*>(&sm.V[lane][16 * w]);
            const uint4 o1 = *reinterpret_cast<const uint4*>(&sm.V[lane][16 * w + 8]);
            bstore16(ro, lane * rowV, o0);
            bstore16(ro, lane * rowV + 16, o1);
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
