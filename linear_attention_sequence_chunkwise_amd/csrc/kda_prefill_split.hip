// kda_prefill_split.hip -- chunkwise KDA prefill for gfx950 in two kernels:
//   K1 (intra): every (chunk, head) in parallel -- gate, decays, the 16-token tile products,
//               T = (I + A_kk)^{-1} and M = A_qk T -- written as one compact factor block
//   K2 (state): per (sequence, head, dv slice), the serial inter-chunk pass
//               X = K~ S, R = beta (V - X), U = T R, O = Q~ S + M R,
//               S <- diag(e^{Gamma_n}) S + K^n^T U
// Only K2's short dependent chain is serial over chunks; everything that does not depend on
// the state runs at full-GPU parallelism in K1.
//
// Sources (page title, section):
//   [K3 note] "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
//     §3.1  S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t
//     §3.2  edit/read order: decay, predict at k, write beta k (v - vhat)^T, read after
//     §3.3  chunked prefill (X_[c], S_in) -> (Y_[c], S_out) with S_in[c+1] = S_out[c], matrix
//           work inside a chunk; g = g_min Sigmoid(e^A z), g_min = -5; a 16-token tile's
//           cumulative log-decay lies in (-80, 0), so diagonal and off-diagonal tiles are the
//           same dense bf16 matrix product.
//
// Chunk algebra (derived from §3.1/§3.2; the pages defer the WY/UT derivation to a note that
// is not among them).  For a chunk of n <= 64 tokens with chunk-local inclusive
// Gamma_r = sum_{i<=r} g_i per key channel and incoming state S:
//   A_kk[i][j] = beta_i <k_i e^{Gamma_i}, k_j e^{-Gamma_j}> (j < i),  T = (I + A_kk)^{-1}
//   A_qk[i][j] =        <q_i e^{Gamma_i}, k_j e^{-Gamma_j}> (j <= i), M = A_qk T
//   U = T diag(beta)(V - K~ S),  O = Q~ S + A_qk U = Q~ S + M diag(beta)(V - K~ S)
//   S' = diag(e^{Gamma_n}) S + (K e^{Gamma_n - Gamma})^T U,  K~ = K e^{Gamma}, Q~ = Q e^{Gamma}
// Decayed products are factored per 16-token tile around rho_a (Gamma just before tile a):
// row operands carry e^{Gamma_i - rho_a} in [e^-80, 1], column operands e^{rho_a - Gamma_j},
// <= 1 off the diagonal and < e^80 on it -- the pages' bound.  Decays are cumulative
// products of alpha = e^g, never exponentials of large sums.
//
// Factor block of one (chunk, head), bf16 unless noted (offsets in the kernels below):
//   Kt [64][DK] = K~, Qt [64][DK] = Q~, KnT [DK][64] = (K e^{Gamma_n - Gamma})^T,
//   T and M as their 10 lower 16x16 blocks (row-major, block order (a,b) = a(a+1)/2 + b),
//   decayN [DK] fp32 = e^{Gamma_n}.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC = 64;  // chunk

template <int DK>
struct Block {
    static constexpr size_t KT = 0;
    static constexpr size_t QT = KT + size_t(kC) * DK * 2;
    static constexpr size_t KN = QT + size_t(kC) * DK * 2;
    static constexpr size_t TB = KN + size_t(DK) * kC * 2;
    static constexpr size_t MB = TB + 10 * 512;
    static constexpr size_t DN = MB + 10 * 512;
    static constexpr size_t BYTES = DN + size_t(DK) * 4;  // multiple of 256
    static_assert(BYTES % 256 == 0, "block alignment");
};

__device__ __forceinline__ int tri_index(int a, int b) { return a * (a + 1) / 2 + b; }

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

template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
    typedef uint32_t raw;  // two bf16
    __device__ __forceinline__ static raw load(rsrc_t r, uint32_t off) { return bload4(r, off); }
    __device__ __forceinline__ static float2 get(raw x) { return make_float2(lo_bf16(x), hi_bf16(x)); }
    struct Row8 { uint4 a; };
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
    struct Row8 { uint4 a, b; };
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

// Sequence and chunk of chunk slot s: chunk_start[n] <= s < chunk_start[n+1].
__device__ __forceinline__ int slot_seq(const int32_t* cs, int n_seqs, int s) {
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cs[mid] <= s) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace

// ---- chunk table: chunk_start[n] = sum_{m<n} ceil(L_m / 64); one workgroup --------------
__global__ void __launch_bounds__(1024) chunk_table_kernel(const int32_t* cu, int n_seqs,
                                                          int32_t* chunk_start) {
    __shared__ int32_t part[1024];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n_seqs; base += 1024) {
        const int n = base + tid;
        const int32_t c = n < n_seqs ? (cu[n + 1] - cu[n] + kC - 1) / kC : 0;
        part[tid] = c;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
            const int32_t x = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        if (n < n_seqs) chunk_start[n + 1] = carry + part[tid];
        __syncthreads();
        if (tid == 1023) carry += part[1023];
        __syncthreads();
    }
    if (tid == 0) chunk_start[0] = 0;
}

// ---- K1: intra-chunk factors ------------------------------------------------------------
template <int DK>
struct IntraSmem {
    static constexpr int NT = 256;
    static constexpr int KROW = DK + 16;      // 16-byte operand reads over 16 rows: no conflict
    static constexpr int TROW = kC + 8;
    static constexpr int SEG = 32 * DK / NT;  // gate item: SEG tokens x 2 channels
    static constexpr int NSEG = kC / SEG;
    struct Ops {
        bf16_t Kr[kC][KROW];   // k_i e^{Gamma_i - rho_a}
        bf16_t Qr[kC][KROW];   // q_i e^{Gamma_i - rho_a}
        bf16_t Kc[kC][KROW];   // k_j e^{rho_{b+1} - Gamma_j}
    };
    struct Out {
        bf16_t T[kC][TROW];    // T, row-major
        bf16_t Tt[kC][TROW];   // T transposed
        bf16_t M[kC][TROW];    // M = A_qk T, row-major
    };
    union { Ops ops; Out out; } u;
    float Pseg[NSEG][DK];
    float colscale[7][DK];
    float beta[kC];
    float Ld[4][16][20];       // diagonal blocks of A_kk (fp32), [block][col j][row i]
    bf16_t L[kC][TROW];        // A_kk row-major (off-diagonal blocks)
    bf16_t Aqk[kC][TROW];      // A_qk row-major (lower blocks, diagonal included)
};

template <int DK, typename TIn>
__global__ void __launch_bounds__(256) prefill_intra_kernel(SplitArgs args) {
    using Smem = IntraSmem<DK>;
    using P = Pair<TIn>;
    using B = Block<DK>;
    constexpr int NT = Smem::NT;
    constexpr int SEG = Smem::SEG;
    constexpr int NSEG = Smem::NSEG;
    constexpr int SPT = 16 / SEG;
    constexpr int NCP = DK / 2;
    constexpr int KSTEPS = DK / 32;
    constexpr int ES = static_cast<int>(sizeof(TIn));
    static_assert(NSEG * NCP == NT && (SEG == 8 || SEG == 16), "items");

    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;

    // chunk slot -> (sequence, chunk of the sequence)
    const int slot = blockIdx.x, h = blockIdx.y, H = args.H;
    int n;
    int64_t tok0, len, c0;
    if (args.cu) {
        if (slot >= args.chunk_start[args.n_seqs]) return;
        n = slot_seq(args.chunk_start, args.n_seqs, slot);
        tok0 = args.cu[n];
        len = static_cast<int64_t>(args.cu[n + 1]) - tok0;
        c0 = static_cast<int64_t>(slot - args.chunk_start[n]) * kC;
    } else {
        const int nc = static_cast<int>((args.T + kC - 1) / kC);
        n = slot / nc;
        if (n >= args.n_seqs) return;
        tok0 = static_cast<int64_t>(n) * args.T;
        len = args.T;
        c0 = static_cast<int64_t>(slot - n * nc) * kC;
    }
    const int clen = static_cast<int>(len - c0 < kC ? len - c0 : kC);
    const int64_t t0 = tok0 + c0;
    char* blk = static_cast<char*>(args.blocks) + (static_cast<size_t>(slot) * H + h) * B::BYTES;

    const uint32_t rowK = static_cast<uint32_t>(H) * DK * ES;
    const uint32_t rowZ = static_cast<uint32_t>(H) * DK * 4;
    const uint32_t rowB = static_cast<uint32_t>(H) * ES;
    const char* kbase = static_cast<const char*>(args.k) + static_cast<size_t>(h) * DK * ES;
    const char* qbase = static_cast<const char*>(args.q) + static_cast<size_t>(h) * DK * ES;
    const char* bbase = static_cast<const char*>(args.beta) + static_cast<size_t>(h) * ES;
    const char* zbase = reinterpret_cast<const char*>(args.z) + static_cast<size_t>(h) * DK * 4;

    // gate item: segment iseg (tokens SEG*iseg ..), channels ch0, ch0 + 1
    const int icp = tid % NCP, iseg = tid / NCP, ch0 = 2 * icp;
    const int itile = iseg / SPT, isub = iseg % SPT;
    const float ae0 = -expf(args.A[h * DK + ch0]) * kLog2e;  // -e^{A} log2(e)
    const float ae1 = -expf(args.A[h * DK + ch0 + 1]) * kLog2e;
    const float gscale = args.g_min * kLog2e;

    // ---- loads (rows past the sequence end read as zero) --------------------------------
    typename P::raw pk[SEG], pq[SEG];
    uint2 pz[SEG];
    {
        const rsrc_t rk = make_rsrc(kbase + t0 * rowK, clen * rowK);
        const rsrc_t rq = make_rsrc(qbase + t0 * rowK, clen * rowK);
        const rsrc_t rz = make_rsrc(zbase + t0 * rowZ, clen * rowZ);
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const uint32_t row = static_cast<uint32_t>(iseg * SEG + i);
            pk[i] = P::load(rk, row * rowK + ch0 * ES);
            pq[i] = P::load(rq, row * rowK + ch0 * ES);
            pz[i] = bload8(rz, row * rowZ + ch0 * 4);
        }
        if (tid < kC) {
            const rsrc_t rb = make_rsrc(bbase + t0 * rowB, clen * rowB);
            sm.beta[tid] = P::load_beta(rb, tid * rowB);
        }
    }

    // ---- gates: alpha = e^g, tokens past the end get alpha = 1 (g = 0) -----------------------
    float2 al[SEG];
    {
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
        *reinterpret_cast<float2*>(&sm.Pseg[iseg][ch0]) = Pq;
    }
    lds_barrier();

    // ---- operands: Kr, Qr, Kc to LDS; Kt, Qt, KnT, decayN to the factor block -----------
    {
        float2 ps[NSEG];
#pragma unroll
        for (int s = 0; s < NSEG; ++s) ps[s] = *reinterpret_cast<const float2*>(&sm.Pseg[s][ch0]);
        float2 Tt[4];  // tile products e^{rho_{a+1} - rho_a}
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            Tt[a] = ps[a * SPT];
            if (SPT == 2) { Tt[a].x *= ps[a * SPT + 1].x; Tt[a].y *= ps[a * SPT + 1].y; }
        }
        float2 eR = make_float2(1.f, 1.f), eN = eR;  // e^{rho_a}, e^{Gamma_n - rho_{a+1}}
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if (a < itile) { eR.x *= Tt[a].x; eR.y *= Tt[a].y; }
            if (a > itile) { eN.x *= Tt[a].x; eN.y *= Tt[a].y; }
        }
        float2 pre = make_float2(1.f, 1.f), post = pre;
        if (SPT == 2) {
            const float2 other = *reinterpret_cast<const float2*>(&sm.Pseg[iseg ^ 1][ch0]);
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
            *reinterpret_cast<uint32_t*>(&sm.u.ops.Kr[r][ch0]) = pack_bf16x2(kf.x * F.x, kf.y * F.y);
            *reinterpret_cast<uint32_t*>(&sm.u.ops.Qr[r][ch0]) = pack_bf16x2(qf.x * F.x, qf.y * F.y);
            *reinterpret_cast<uint32_t*>(&sm.u.ops.Kc[r][ch0]) = pack_bf16x2(kf.x * E[i].x, kf.y * E[i].y);
            *reinterpret_cast<uint32_t*>(blk + B::KT + (r * DK + ch0) * 2) = pack_bf16x2(kf.x * FR.x, kf.y * FR.y);
            *reinterpret_cast<uint32_t*>(blk + B::QT + (r * DK + ch0) * 2) = pack_bf16x2(qf.x * FR.x, qf.y * FR.y);
            kn[i] = make_float2(kf.x * (E[i].x * eN.x), kf.y * (E[i].y * eN.y));
        }
#pragma unroll
        for (int j = 0; j < SEG / 4; ++j) {
            const int tk = iseg * SEG + 4 * j;
            *reinterpret_cast<uint2*>(blk + B::KN + (ch0 * kC + tk) * 2) =
                make_uint2(pack_bf16x2(kn[4 * j].x, kn[4 * j + 1].x), pack_bf16x2(kn[4 * j + 2].x, kn[4 * j + 3].x));
            *reinterpret_cast<uint2*>(blk + B::KN + ((ch0 + 1) * kC + tk) * 2) =
                make_uint2(pack_bf16x2(kn[4 * j].y, kn[4 * j + 1].y), pack_bf16x2(kn[4 * j + 2].y, kn[4 * j + 3].y));
        }
        if (iseg == 0) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float T0 = e ? Tt[0].y : Tt[0].x, T1 = e ? Tt[1].y : Tt[1].x;
                const float T2 = e ? Tt[2].y : Tt[2].x, T3 = e ? Tt[3].y : Tt[3].x;
                const int c = ch0 + e;
                sm.colscale[0][c] = fast_rcp(T0);
                sm.colscale[1][c] = fast_rcp(T1);
                sm.colscale[2][c] = fast_rcp(T2);
                sm.colscale[3][c] = fast_rcp(T3);
                sm.colscale[4][c] = T1;
                sm.colscale[5][c] = T1 * T2;
                sm.colscale[6][c] = T2;
            }
            *reinterpret_cast<float2*>(blk + B::DN + ch0 * 4) =
                make_float2(Tt[0].x * Tt[1].x * Tt[2].x * Tt[3].x, Tt[0].y * Tt[1].y * Tt[2].y * Tt[3].y);
        }
    }
    lds_barrier();

    // ---- lower 16x16 tiles of A_kk and A_qk (transposed product: lane ends with four
    // consecutive columns j of one row i) -----------------------------------------------
#pragma unroll
    for (int slot2 = 0; slot2 < 3; ++slot2) {
        const int job = w + slot2 * 4;
        if (job < 10) {
            const int a = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
            const int b = job - (a * (a + 1)) / 2;
            const int si = colscale_index(a, b);
            f32x4_t ckk = {0.f, 0.f, 0.f, 0.f}, cqk = ckk;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int ch = 32 * s + 8 * g;
                uint4 col = *reinterpret_cast<const uint4*>(&sm.u.ops.Kc[16 * b + li][ch]);
                if (si >= 0)
                    col = scale8(col, *reinterpret_cast<const float4*>(&sm.colscale[si][ch]),
                                 *reinterpret_cast<const float4*>(&sm.colscale[si][ch + 4]));
                ckk = mfma32(col, *reinterpret_cast<const uint4*>(&sm.u.ops.Kr[16 * a + li][ch]), ckk);
                cqk = mfma32(col, *reinterpret_cast<const uint4*>(&sm.u.ops.Qr[16 * a + li][ch]), cqk);
            }
            const float bi = sm.beta[16 * a + li];
            if (a == b) {
                float qv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jj = 4 * g + r;
                    sm.Ld[a][jj][li] = jj < li ? bi * ckk[r] : 0.f;  // strictly lower
                    qv[r] = jj <= li ? cqk[r] : 0.f;                // lower incl. diagonal
                }
                *reinterpret_cast<uint2*>(&sm.Aqk[16 * a + li][16 * b + 4 * g]) =
                    make_uint2(pack_bf16x2(qv[0], qv[1]), pack_bf16x2(qv[2], qv[3]));
            } else {
                *reinterpret_cast<uint2*>(&sm.L[16 * a + li][16 * b + 4 * g]) =
                    make_uint2(pack_bf16x2(bi * ckk[0], bi * ckk[1]), pack_bf16x2(bi * ckk[2], bi * ckk[3]));
                *reinterpret_cast<uint2*>(&sm.Aqk[16 * a + li][16 * b + 4 * g]) =
                    make_uint2(pack_bf16x2(cqk[0], cqk[1]), pack_bf16x2(cqk[2], cqk[3]));
            }
        }
    }
    lds_barrier();

    // ---- diagonal blocks T_aa = (I + L_aa)^{-1}, fp32 forward substitution (wave 3) -------
    if (w == 3) {
        const int a = lane >> 4, j = lane & 15;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            float Lm[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 v4 = *reinterpret_cast<const float4*>(&sm.Ld[a][m][4 * q4]);
                Lm[4 * q4] = v4.x; Lm[4 * q4 + 1] = v4.y; Lm[4 * q4 + 2] = v4.z; Lm[4 * q4 + 3] = v4.w;
            }
            const float tm = t[m];
#pragma unroll
            for (int i = m + 1; i < 16; ++i) t[i] -= Lm[i] * tm;
        }
        // column j of T_aa -> T (row-major) and Tt (row j)
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.u.out.T[16 * a + i][16 * a + j] = f32_to_bf16(t[i]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<uint2*>(&sm.u.out.Tt[16 * a + j][16 * a + 4 * q4]) =
                make_uint2(pack_bf16x2(t[4 * q4], t[4 * q4 + 1]), pack_bf16x2(t[4 * q4 + 2], t[4 * q4 + 3]));
    }
    lds_barrier();

    // ---- off-diagonal blocks: T_ab = -T_aa sum_{m=b}^{a-1} L_am T_mb, column block b = wave
    if (w < 3) {
        const int b = w;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        for (int a = b + 1; a < 4; ++a) {
            f32x4_t acc = zero;
            for (int m = b; m < a; ++m)
                acc = mfma16(*reinterpret_cast<const uint2*>(&sm.L[16 * a + li][16 * m + 4 * g]),
                             *reinterpret_cast<const uint2*>(&sm.u.out.Tt[16 * b + li][16 * m + 4 * g]), acc);
            const f32x4_t tab = mfma16(*reinterpret_cast<const uint2*>(&sm.u.out.T[16 * a + li][16 * a + 4 * g]),
                                       pack_bf16x4(acc), zero);
            // tab[r] = -T_ab[4g + r][li]
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.u.out.T[16 * a + 4 * g + r][16 * b + li] = f32_to_bf16(-tab[r]);
            *reinterpret_cast<uint2*>(&sm.u.out.Tt[16 * b + li][16 * a + 4 * g]) =
                make_uint2(pack_bf16x2(-tab[0], -tab[1]), pack_bf16x2(-tab[2], -tab[3]));
        }
    }
    lds_barrier();

    // ---- M = A_qk T (lower blocks): M_ab = sum_{m=b}^{a} A_qk[a][m] T_mb --------------------
#pragma unroll
    for (int slot2 = 0; slot2 < 3; ++slot2) {
        const int job = w + slot2 * 4;
        if (job < 10) {
            const int a = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
            const int b = job - (a * (a + 1)) / 2;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int m = b; m <= a; ++m)
                acc = mfma16(*reinterpret_cast<const uint2*>(&sm.Aqk[16 * a + li][16 * m + 4 * g]),
                             *reinterpret_cast<const uint2*>(&sm.u.out.Tt[16 * b + li][16 * m + 4 * g]), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.u.out.M[16 * a + 4 * g + r][16 * b + li] = f32_to_bf16(acc[r]);
        }
    }
    lds_barrier();

    // ---- T and M lower blocks -> factor block (512 bytes per block, 16-byte pieces) -------
    for (int idx = tid; idx < 2 * 10 * 32; idx += NT) {
        const int which = idx / 320, rem = idx % 320, blk_i = rem / 32, piece = rem % 32;
        const int a = blk_i < 1 ? 0 : blk_i < 3 ? 1 : blk_i < 6 ? 2 : 3;
        const int b = blk_i - (a * (a + 1)) / 2;
        const int row = piece >> 1, half = piece & 1;
        const bf16_t* src = which == 0 ? &sm.u.out.T[16 * a + row][16 * b + 8 * half]
                                       : &sm.u.out.M[16 * a + row][16 * b + 8 * half];
        *reinterpret_cast<uint4*>(blk + (which == 0 ? B::TB : B::MB) + blk_i * 512 + row * 32 + half * 16) =
            *reinterpret_cast<const uint4*>(src);
    }
}

// ---- K2: serial state pass ----------------------------------------------------------------
template <int DK, int NW>
struct StateSmem {
    static constexpr int NT = 64 * NW;
    static constexpr int DVS = 16 * NW;
    static constexpr int KROW = DK + 16;
    static constexpr int TROW = kC + 8;
    static constexpr int VROW = DVS + 16;
    bf16_t Kt[kC][KROW];
    bf16_t Qt[kC][KROW];
    bf16_t KnT[DK][TROW];
    bf16_t T[kC][TROW];    // lower 16x16 blocks used
    bf16_t M[kC][TROW];
    bf16_t V[kC][VROW];    // v of this slice; each wave's 16 columns then stage its O
    float beta[kC];
    float decayN[DK];
};

template <int DK, int NW, typename TIn>
__global__ void __launch_bounds__(NW * 64, 1) prefill_state_kernel(SplitArgs args) {
    using Smem = StateSmem<DK, NW>;
    using P = Pair<TIn>;
    using B = Block<DK>;
    constexpr int NT = Smem::NT;
    constexpr int DVS = Smem::DVS;
    constexpr int KSTEPS = DK / 32;
    constexpr int MT = DK / 16;
    constexpr int ES = static_cast<int>(sizeof(TIn));
    // 16-byte pieces of one factor block and of the v slice
    constexpr int NKT = kC * DK / 8;             // per Kt / Qt / KnT
    constexpr int NTB = 10 * 32;                 // per T / M
    constexpr int NDN = DK / 4;
    constexpr int NV = kC * DVS / 8;
    constexpr int PK = NKT / NT;                 // Kt, Qt, KnT pieces per thread
    constexpr int PT = (NTB + NT - 1) / NT;      // T, M pieces per thread (guarded)
    constexpr int PV = NV / NT;
    static_assert(NKT % NT == 0 && NV % NT == 0 && PV >= 1, "piece split");

    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;

    const int bid = blockIdx.x;
    const int xcd = bid & 7, kq = bid >> 3;
    const int pair = (kq / args.nslices) * 8 + xcd;
    const int slice = kq % args.nslices;
    if (pair >= args.npairs) return;
    const int H = args.H;
    const int n = pair / H, h = pair - n * H;
    int64_t tok0, len;
    int slot0;
    if (args.cu) {
        tok0 = args.cu[n];
        len = static_cast<int64_t>(args.cu[n + 1]) - tok0;
        slot0 = args.chunk_start[n];
    } else {
        tok0 = static_cast<int64_t>(n) * args.T;
        len = args.T;
        slot0 = n * static_cast<int>((args.T + kC - 1) / kC);
    }
    const int dv = DK;
    const int col0 = slice * DVS + 16 * w;
    const uint32_t rowV = static_cast<uint32_t>(H) * dv * ES;
    const uint32_t rowB = static_cast<uint32_t>(H) * ES;
    const char* vbase = static_cast<const char*>(args.v) + (static_cast<size_t>(h) * dv + slice * DVS) * ES;
    const char* bbase = static_cast<const char*>(args.beta) + static_cast<size_t>(h) * ES;
    char* obase = static_cast<char*>(args.o) + (static_cast<size_t>(h) * dv + col0) * ES;
    const char* blocks = static_cast<const char*>(args.blocks);

    f32x4_t Sacc[MT];  // Sacc[m][r] = S[pi(m, 4g + r)][col0 + li]
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * dv + col0 + li;
    if (args.s0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sacc[m][r] = args.s0[sbase + static_cast<size_t>(32 * (m >> 1) + 8 * g + 4 * (m & 1) + r) * dv];
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) Sacc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // prefetch registers for one chunk
    uint4 pkt[PK], pqt[PK], pkn[PK], ptb[PT], pmb[PT];
    uint4 pdn = make_uint4(0, 0, 0, 0);
    typename P::Row8 pv[PV];
    float pb = 0.f;
    auto issue_loads = [&](int64_t t0, int clen, int slot) __attribute__((always_inline)) {
        const rsrc_t rf = make_rsrc(blocks + (static_cast<size_t>(slot) * H + h) * B::BYTES, B::BYTES);
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const uint32_t p = static_cast<uint32_t>(tid + i * NT) * 16;
            pkt[i] = bload16(rf, B::KT + p);
            pqt[i] = bload16(rf, B::QT + p);
            pkn[i] = bload16(rf, B::KN + p);
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const uint32_t p = static_cast<uint32_t>(tid + i * NT);
            ptb[i] = p < NTB ? bload16(rf, B::TB + p * 16) : make_uint4(0, 0, 0, 0);
            pmb[i] = p < NTB ? bload16(rf, B::MB + p * 16) : make_uint4(0, 0, 0, 0);
        }
        if (tid < NDN) pdn = bload16(rf, B::DN + tid * 16);
        const rsrc_t rv = make_rsrc(vbase + t0 * rowV, clen * rowV);
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int idx = tid + i * NT, r = idx / (DVS / 8), o8 = (idx % (DVS / 8)) * 8;
            pv[i] = P::load8(rv, r * rowV + o8 * ES);
        }
        const rsrc_t rb = make_rsrc(bbase + t0 * rowB, clen * rowB);
        pb = P::load_beta(rb, (tid & (kC - 1)) * rowB);
    };
    if (len > 0) issue_loads(tok0, len < kC ? static_cast<int>(len) : kC, slot0);

    int slot = slot0;
    for (int64_t c0 = 0; c0 < len; c0 += kC, ++slot) {
        const int clen = static_cast<int>(len - c0 < kC ? len - c0 : kC);
        const int64_t t0 = tok0 + c0;

        lds_barrier();  // the previous chunk's readers are done
        // ---- copy the prefetched chunk into LDS ---------------------------------------
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int p = tid + i * NT;
            const int r = p / (DK / 8), c8 = (p % (DK / 8)) * 8;  // Kt/Qt: row r, channel c8
            *reinterpret_cast<uint4*>(&sm.Kt[r][c8]) = pkt[i];
            *reinterpret_cast<uint4*>(&sm.Qt[r][c8]) = pqt[i];
            const int rn = p / (kC / 8), t8 = (p % (kC / 8)) * 8;  // KnT: row channel, token t8
            *reinterpret_cast<uint4*>(&sm.KnT[rn][t8]) = pkn[i];
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int p = tid + i * NT;
            if (p < NTB) {
                const int bi = p / 32, piece = p % 32, row = piece >> 1, half = piece & 1;
                const int a = bi < 1 ? 0 : bi < 3 ? 1 : bi < 6 ? 2 : 3;
                const int b = bi - (a * (a + 1)) / 2;
                *reinterpret_cast<uint4*>(&sm.T[16 * a + row][16 * b + 8 * half]) = ptb[i];
                *reinterpret_cast<uint4*>(&sm.M[16 * a + row][16 * b + 8 * half]) = pmb[i];
            }
        }
        if (tid < NDN) *reinterpret_cast<uint4*>(&sm.decayN[4 * tid]) = pdn;
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int idx = tid + i * NT, r = idx / (DVS / 8), o8 = (idx % (DVS / 8)) * 8;
            *reinterpret_cast<uint4*>(&sm.V[r][o8]) = P::bf16x8(pv[i]);
        }
        if (tid < kC) sm.beta[tid] = pb;
        if (c0 + kC < len) {
            const int64_t rem = len - c0 - kC;
            issue_loads(t0 + kC, rem < kC ? static_cast<int>(rem) : kC, slot + 1);
        }
        lds_barrier();

        // ---- X = K~ S, Y = Q~ S, R = beta (V - X) (wave-local from here on) --------------
        uint4 Sb[KSTEPS];  // bf16 S as B operand: slot e of lane g <-> channel 32s+8g+e
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            Sb[s] = make_uint4(pack_bf16x2(Sacc[2 * s][0], Sacc[2 * s][1]),
                               pack_bf16x2(Sacc[2 * s][2], Sacc[2 * s][3]),
                               pack_bf16x2(Sacc[2 * s + 1][0], Sacc[2 * s + 1][1]),
                               pack_bf16x2(Sacc[2 * s + 1][2], Sacc[2 * s + 1][3]));
        f32x4_t Y[4];
        uint2 Rb[4];
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
            const float4 bb = *reinterpret_cast<const float4*>(&sm.beta[16 * a + 4 * g]);
            const int vc = 16 * w + li;
            f32x4_t R;
            R[0] = bb.x * (bf16_to_f32(sm.V[16 * a + 4 * g + 0][vc]) - X[0]);
            R[1] = bb.y * (bf16_to_f32(sm.V[16 * a + 4 * g + 1][vc]) - X[1]);
            R[2] = bb.z * (bf16_to_f32(sm.V[16 * a + 4 * g + 2][vc]) - X[2]);
            R[3] = bb.w * (bf16_to_f32(sm.V[16 * a + 4 * g + 3][vc]) - X[3]);
            Rb[a] = pack_bf16x4(R);  // B operand: k = token 4g + r of tile a
        }
        // ---- U = T R, O = Y + M R ---------------------------------------------------------
        uint2 Ub[4];
        const rsrc_t ro = make_rsrc(obase + t0 * rowV, clen * rowV);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t U = {0.f, 0.f, 0.f, 0.f};
            f32x4_t O = Y[a];
#pragma unroll
            for (int b = 0; b <= a; ++b) {
                U = mfma16(*reinterpret_cast<const uint2*>(&sm.T[16 * a + li][16 * b + 4 * g]), Rb[b], U);
                O = mfma16(*reinterpret_cast<const uint2*>(&sm.M[16 * a + li][16 * b + 4 * g]), Rb[b], O);
            }
            Ub[a] = pack_bf16x4(U);
            if constexpr (sizeof(TIn) == 2) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.V[16 * a + 4 * g + r][16 * w + li] = f32_to_bf16(O[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    bstore4(ro, (16 * a + 4 * g + r) * rowV + li * 4, __float_as_uint(O[r]));
            }
        }
        if constexpr (sizeof(TIn) == 2) {
            const uint4 o0 = *reinterpret_cast<const uint4*>(&sm.V[lane][16 * w]);
            const uint4 o1 = *reinterpret_cast<const uint4*>(&sm.V[lane][16 * w + 8]);
            bstore16(ro, lane * rowV, o0);
            bstore16(ro, lane * rowV + 16, o1);
        }
        // ---- S = diag(e^{Gamma_n}) S + K^n^T U --------------------------------------------
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
                                 make_uint4(Ub[2 * sp].x, Ub[2 * sp].y, Ub[2 * sp + 1].x, Ub[2 * sp + 1].y),
                                 Sacc[m]);
            }
        }
    }

    if (args.sN) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                args.sN[sbase + static_cast<size_t>(32 * (m >> 1) + 8 * g + 4 * (m & 1) + r) * dv] = Sacc[m][r];
    }
}

// ---- host side --------------------------------------------------------------------------

size_t split_block_bytes(int dk) { return dk == 128 ? Block<128>::BYTES : Block<64>::BYTES; }

int64_t split_max_chunks(int64_t total, int n_seqs) { return (total + kC - 1) / kC + n_seqs; }

size_t split_workspace_bytes(int64_t total, int n_seqs, int H, int dk) {
    const size_t table = ((static_cast<size_t>(n_seqs) + 1) * 4 + 255) / 256 * 256;
    return table + static_cast<size_t>(split_max_chunks(total, n_seqs)) * H * split_block_bytes(dk);
}

template <int DK, int NW, typename TIn>
static hipError_t launch_split_t(const SplitArgs& a0, hipStream_t stream) {
    SplitArgs a = a0;
    if (a.cu) {
        hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, stream, a.cu, a.n_seqs, a.chunk_start);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t slots = a.cu ? split_max_chunks(a.total, a.n_seqs)
                               : static_cast<int64_t>(a.n_seqs) * ((a.T + kC - 1) / kC);
    if (slots > 0) {
        hipLaunchKernelGGL((prefill_intra_kernel<DK, TIn>), dim3(static_cast<unsigned>(slots), a.H), dim3(256), 0,
                           stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    a.nslices = DK / (16 * NW);
    const int groups = (a.npairs + 7) / 8;
    hipLaunchKernelGGL((prefill_state_kernel<DK, NW, TIn>), dim3(static_cast<unsigned>(groups) * 8u * a.nslices),
                       dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill_split(const SplitArgs& a, int dk, bool bf16, int waves, hipStream_t stream) {
    if (dk == 128) {
        if (waves == 8) return bf16 ? launch_split_t<128, 8, bf16_t>(a, stream) : launch_split_t<128, 8, float>(a, stream);
        if (waves == 2) return bf16 ? launch_split_t<128, 2, bf16_t>(a, stream) : launch_split_t<128, 2, float>(a, stream);
        return bf16 ? launch_split_t<128, 4, bf16_t>(a, stream) : launch_split_t<128, 4, float>(a, stream);
    }
    if (waves == 2) return bf16 ? launch_split_t<64, 2, bf16_t>(a, stream) : launch_split_t<64, 2, float>(a, stream);
    return bf16 ? launch_split_t<64, 4, bf16_t>(a, stream) : launch_split_t<64, 4, float>(a, stream);
}

}  // namespace kda
