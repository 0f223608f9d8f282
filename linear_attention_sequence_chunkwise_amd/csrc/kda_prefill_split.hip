// kda_prefill_split.hip -- chunkwise KDA prefill for gfx950, in one of two forms.
// Split form (fewer (sequence, head) chains than compute units, or fp32 inputs), two kernels:
//   K1 (intra): every (chunk, head) in parallel -- gate, decays, the 16-token tile products,
//               T = (I + A_kk)^{-1} and M = A_qk T -- written as one compact factor block
//   K2 (state): per (sequence, head, dv slice), the serial inter-chunk pass
//               X = K~ S, R = beta (V - X), U = T R, O = Q~ S + M R,
//               S <- diag(e^{Gamma_n}) S + K^n^T U
// Only K2's short dependent chain is serial over chunks; everything that does not depend on
// the state runs at full-GPU parallelism in K1.
// Fused form (bf16, a chain per compute unit or more): prefill_fused_kernel, one eight-wave
// workgroup per chain, whose producer waves build the next chunk's factors into LDS with
// K1's phases while its consumer waves run K2's products on the current chunk, so the factor
// blocks never leave the CU (described at the kernel, near the end of this file).
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
// <= 1 off the diagonal and < e^80 on it -- the pages' bound.  Within a tile a decay is the
// exponential of a sum of at most 16 log-decays (bounded by the same -80); across tiles,
// decays are products of tile totals, never exponentials of chunk-long sums.
//
// Factor block of one (chunk, head), bf16 unless noted (offsets in the kernels below):
//   Kt = K~ and Qt = Q~ [64 x DK], KnT = (K e^{Gamma_n - Gamma})^T [DK x 64], each stored as
//   the lane-order image (lane_off, kn_off) that the state pass copies verbatim into LDS,
//   T and M as their 10 lower 16x16 blocks (row-major, block order (a,b) = a(a+1)/2 + b),
//   decayN [DK] fp32 = e^{Gamma_n}; order Qt, M | Kt, KnT, T, decayN (struct Block).
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC = 64;  // chunk

// Factor block layout: the operands of the output products (Q~, M) first, then those of the
// recurrence (K~, K^n, T, e^{Gamma_n}); both parts start on a 1 KiB boundary.
template <int DK>
struct Block {
    static constexpr size_t QT = 0;
    static constexpr size_t MB = QT + size_t(kC) * DK * 2;
    static constexpr size_t KT = MB + 10 * 512;
    static constexpr size_t KN = KT + size_t(kC) * DK * 2;
    static constexpr size_t TB = KN + size_t(DK) * kC * 2;
    static constexpr size_t DN = TB + 10 * 512;
    static constexpr size_t BYTES = DN + size_t(DK) * 4;  // multiple of 256
    static constexpr int NQP = static_cast<int>(KT / 1024);            // 1 KiB pieces of Q~, M
    static constexpr int NBP = static_cast<int>((BYTES + 1023) / 1024);  // pieces of the block
    static_assert(BYTES % 256 == 0 && KT % 1024 == 0, "block alignment");
};

__device__ __forceinline__ int tri_index(int a, int b) { return a * (a + 1) / 2 + b; }

// Lane-order images in a factor block.  K~ and Q~: 1 KiB piece (a, s), a = row tile, s = 32-
// channel step, holds for lane (g, li) the eight channels 32s + 8g .. of row 16a + li -- the 16
// bytes that lane feeds to a 16x16x32 MFMA.  K^n^T: piece (m, sp) holds for lane (g, li) the
// tokens 32sp + 4g .. + 3 and 32sp + 16 + 4g .. + 3 of channel pi(m, li), with the state row
// order pi(m, i) = 32 (m / 2) + 8 (i / 4) + 4 (m % 2) + i % 4 of the state-update product.

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
    __device__ __forceinline__ static float at(const Row8& x, int e) {
        const uint32_t wv = e < 2 ? x.a.x : e < 4 ? x.a.y : e < 6 ? x.a.z : x.a.w;
        return (e & 1) ? hi_bf16(wv) : lo_bf16(wv);
    }
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
    __device__ __forceinline__ static float at(const Row8& x, int e) {
        const uint4& u = e < 4 ? x.a : x.b;
        const int i = e & 3;
        return __uint_as_float(i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w);
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

// ---- chain order for the fused prefill: sequences by decreasing chunk count ---------------
// The fused kernel runs one workgroup per (sequence, head) chain, so a batch of chains of
// mixed lengths finishes sooner when the longest start first.  One workgroup counting-sorts
// the sequences into buckets of their chunk count (floor(log2) and the next two bits: about
// 19% apart), longest bucket first.  The order within a bucket is arbitrary: chains are
// independent, so it affects only when each one runs, never a result.
constexpr int kOrderBuckets = 128;
__device__ __forceinline__ int chain_bucket(const int32_t* cu, int n) {
    const uint32_t c = static_cast<uint32_t>((cu[n + 1] - cu[n] + kC - 1) / kC);
    if (c == 0) return 0;
    const int e = 31 - __builtin_clz(c);
    return 1 + 4 * e + static_cast<int>(((static_cast<uint64_t>(c) << 2) >> e) & 3u);
}
__global__ void __launch_bounds__(1024) chain_order_kernel(const int32_t* cu, int n_seqs, int32_t* order) {
    __shared__ int32_t cnt[kOrderBuckets];
    const int tid = threadIdx.x;
    if (tid < kOrderBuckets) cnt[tid] = 0;
    __syncthreads();
    for (int n = tid; n < n_seqs; n += 1024) atomicAdd(&cnt[chain_bucket(cu, n)], 1);
    __syncthreads();
    if (tid == 0) {  // exclusive prefix over the buckets, longest first
        int run = 0;
        for (int b = kOrderBuckets - 1; b >= 0; --b) {
            const int k = cnt[b];
            cnt[b] = run;
            run += k;
        }
    }
    __syncthreads();
    for (int n = tid; n < n_seqs; n += 1024) order[atomicAdd(&cnt[chain_bucket(cu, n)], 1)] = n;
}

// ---- K1: intra-chunk factors ------------------------------------------------------------
// One workgroup of four waves per (chunk, head).  Wave w owns 16-token tile w and works in
// the MFMA operand layout from the start: lane (g, li) holds token 16w + li and the channels
// 32s + 8g .. 32s + 8g + 7 for every K-step s, exactly the 16 bytes per step it feeds to a
// 16x16x32 product.  The cumulative decays within a tile are therefore an inclusive scan of
// log-decays across the 16 lanes of a DPP row, K~ and Q~ leave registers as linear 1 KiB
// lane-order writes, and only the column operands (read by other waves) and K^n (transposed
// for the state pass) go through LDS.
// Buffers whose lifetimes do not overlap share storage (39.75 KiB at d = 128: four workgroups
// fit a CU's 160 KiB of LDS): the K^n staging gives way to the tile products once it has been
// copied out, and the column operand to T and M once the tile products have read it.
template <int DK>
struct IntraSmem {
    static constexpr int KS = DK / 32;
    static constexpr int NROW = DK + 8;  // K^n staging rows (bf16), 16-byte aligned
    struct Tiles {
        float Ld[4][16][20];        // diagonal blocks of A_kk (fp32), [block][col j][row i]
        bf16_t L[10][16][16];       // A_kk lower blocks (off-diagonal ones used), row-major
        bf16_t Aqk[10][16][16];     // A_qk lower blocks, diagonal included
    };
    struct Out {
        bf16_t T[10][16][16];   // T lower 16x16 blocks, row-major
        bf16_t Tt[10][16][16];  // the same blocks transposed
        bf16_t M[10][16][16];   // M = A_qk T lower blocks, row-major
    };
    union {
        bf16_t kn[kC][NROW];    // K^n = K e^{Gamma_n - Gamma} (token-major), until copied out
        Tiles t;
    } a;
    union {
        uint4 kc[4 * KS * 64];  // k_j e^{rho_{b+1} - Gamma_j} in lane order [b][s][lane]
        Out out;
    } b;
    float ttile[4][DK];         // e^{rho_{a+1} - rho_a}: the product of alpha over tile a
    float pre[4][DK];           // e^{rho_w}: ttile[0] .. ttile[w-1] multiplied in order (1 for w = 0)
    float suf[4][DK];           // e^{Gamma_n - rho_{w+1}}: ttile[w+1] .. ttile[3] in order (1 for w = 3)
    float ae[DK];               // -e^{A} log2(e)
    float beta[kC];
};

// x[lane - n] within the lane's row of 16, or 0 for the first n lanes of the row.
template <int N>
__device__ __forceinline__ float row_shr_or_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xf, 0xf, true));
}

// x[(lane + 8) mod 16] within the lane's row of 16
__device__ __forceinline__ uint32_t row_ror8(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x128, 0xf, 0xf, false));
}

// Half-row loads.  A row piece of 128 bytes that lanes 0-7 and 8-15 of a DPP row would each
// need half of is fetched as one line per row: register a holds, in lanes 0-7, the first half
// of rows 0-7 and, in lanes 8-15, the second half of rows 0-7; register b the same for rows
// 8-15.  Afterwards lane i holds the first half of row i in a and the second half in b.
__device__ __forceinline__ void unswap_halves(uint32_t& a, uint32_t& b, bool lo) {
    const uint32_t ra = row_ror8(a), rb = row_ror8(b);
    const uint32_t first = lo ? a : rb, second = lo ? ra : b;
    a = first;
    b = second;
}
__device__ __forceinline__ void unswap_halves(uint4& a, uint4& b, bool lo) {
    unswap_halves(a.x, b.x, lo);
    unswap_halves(a.y, b.y, lo);
    unswap_halves(a.z, b.z, lo);
    unswap_halves(a.w, b.w, lo);
}

__device__ __forceinline__ float lane8(const uint4& a, const uint4& b, int e) {
    const uint4& u = e < 4 ? a : b;
    const int i = e & 3;
    return __uint_as_float(i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w);
}

// One (chunk, head) of intra-chunk work, phase by phase, for a group of four waves (wave w
// owns 16-token tile w).  The phases are separated by workgroup barriers, which the caller
// places: the intra-chunk kernel runs them back to back, the fused kernel interleaves them
// with its state-pass waves.  Lane (g, li) of wave w holds token 16w + li and the channels
// 32s + 8g .. 32s + 8g + 7 for every K-step s, exactly the 16 bytes per step it feeds to a
// 16x16x32 product.  The cumulative decays within a tile are therefore an inclusive scan of
// log-decays across the 16 lanes of a DPP row, K~ and Q~ leave registers as linear 1 KiB
// lane-order writes, and only the column operands (read by other waves) and K^n (transposed
// for the state pass) go through LDS.
//   load     q, k, z rows into registers (rows past the end read 0), raw beta
//   phase 1  beta -> LDS
//   phase 2  gates, tile-local scans, F = e^{Gamma_i - rho_w}; tile totals -> LDS
//   phase 3  per-channel products of tile totals; e^{Gamma_n} -> block
//   phase 4  operands: K~, Q~ -> block, column operand and K^n staging -> LDS (fused kernel:
//            K^n^T straight into the block, and no phase 5)
//   phase 5  K^n^T -> block in lane order
//   phase 6  the 10 lower 16x16 tiles of A_kk and A_qk (fused kernel: with each wave's own
//            diagonal block of T, phase6_solve)
//   phase 7  diagonal blocks of T (wave 3; intra-chunk kernel)
//   phase 8  off-diagonal blocks of T (waves 0-2)
//   phase 9  M = A_qk T
// The block (K~, Q~, K^n^T, e^{Gamma_n}) is written through `blk`: global memory for the
// intra-chunk kernel, an LDS stage for the fused kernel.  T and M go to the LDS arrays Tb and
// Mb (the fused kernel's stage, or staging that the intra-chunk kernel copies out).
template <int DK, typename TIn, bool HalfRow = false>
struct Producer {
    using Smem = IntraSmem<DK>;
    using P = Pair<TIn>;
    using B = Block<DK>;
    static constexpr int KS = DK / 32;
    static constexpr int MT = DK / 16;
    static constexpr int ES = static_cast<int>(sizeof(TIn));

    int tid, w, lane, g, li, r;
    int clen;
    typename P::Row8 pk[KS], pq[KS];
    uint4 pz[KS][2];
    uint32_t rbeta;
    float F[KS][8];
    uint4 kr[KS], qr[KS];

    __device__ __forceinline__ void init(int thread) {
        tid = thread;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        lane = tid & 63;
        g = lane >> 4;
        li = lane & 15;
        r = 16 * w + li;
    }

    // loads of the chunk of `n_valid` tokens starting at token t0 of head h (rows past the end
    // read 0).  With HalfRow (the fused kernel, whose loads are issued beside its other work)
    // each 128-byte line of a z row is fetched by one instruction (the half-row scheme of
    // unswap_halves, undone by unswap_z before phase 2): the two 16-byte pieces of a lane's 32
    // bytes in K-step s go to pz[s][0] (rows 0-7 of the tile) and pz[s][1] (rows 8-15).  The
    // same scheme for q and k (measured) cost more in phase 4 than it saved.  The intra-chunk
    // kernel, which waits for its loads, fetches each lane's own row pieces.
    static constexpr bool kHalfRowZ = HalfRow;
    __device__ __forceinline__ void load(const SplitArgs& args, int h, int64_t t0, int n_valid) {
        clen = n_valid;
        const int H = args.H;
        const uint32_t rowK = static_cast<uint32_t>(H) * DK * ES;
        const uint32_t rowZ = static_cast<uint32_t>(H) * DK * 4;
        const uint32_t rowB = static_cast<uint32_t>(H) * ES;
        const char* kbase = static_cast<const char*>(args.k) + static_cast<size_t>(h) * DK * ES;
        const char* qbase = static_cast<const char*>(args.q) + static_cast<size_t>(h) * DK * ES;
        const char* bbase = static_cast<const char*>(args.beta) + static_cast<size_t>(h) * ES;
        const char* zbase = reinterpret_cast<const char*>(args.z) + static_cast<size_t>(h) * DK * 4;
        const rsrc_t rk = make_rsrc(kbase + t0 * rowK, clen * rowK);
        const rsrc_t rq = make_rsrc(qbase + t0 * rowK, clen * rowK);
        const rsrc_t rz = make_rsrc(zbase + t0 * rowZ, clen * rowZ);
        const uint32_t lo_row = kHalfRowZ ? 16 * w + (li & 7) : r;
        const uint32_t hi_row = kHalfRowZ ? lo_row + 8 : r;
        const uint32_t zoff0 = kHalfRowZ ? (li < 8 ? 0u : 16u) : 0u, zoff1 = kHalfRowZ ? zoff0 : 16u;
        // The intra-chunk kernel waits for these loads in phase 2 (z) and phase 4 (k, q): z
        // first lets k and q stay in flight through phases 2-3 (B=4 H=32 T=32768: 2.79 ->
        // 2.76 ms).  The fused kernel waits for all of them at the end of phase 6, and there
        // that order is slower (3.88 -> 3.97 ms on the varlen batch): k and q then land beside
        // the gates' VALU work of phase 2.
        constexpr bool kZFirst = !kHalfRowZ;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint32_t ch = 32 * s + 8 * g;
            if constexpr (!kZFirst) {
                pk[s] = P::load8(rk, r * rowK + ch * ES);
                pq[s] = P::load8(rq, r * rowK + ch * ES);
            }
            pz[s][0] = bload16(rz, lo_row * rowZ + ch * 4 + zoff0);
            pz[s][1] = bload16(rz, hi_row * rowZ + ch * 4 + zoff1);
        }
        // (with z first, every thread loads: offsets of threads past the chunk lie beyond the
        // buffer's range and read 0 without a memory access, and a load outside a branch keeps
        // the compiler from waiting for it, and so for every load before it, on the spot)
        if (kZFirst || tid < kC) {
            const rsrc_t rb = make_rsrc(bbase + t0 * rowB, clen * rowB);
            if constexpr (sizeof(TIn) == 2) rbeta = bload2(rb, tid * rowB);
            else rbeta = bload4(rb, tid * rowB);
        }
        if constexpr (kZFirst) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint32_t ch = 32 * s + 8 * g;
                pk[s] = P::load8(rk, r * rowK + ch * ES);
                pq[s] = P::load8(rq, r * rowK + ch * ES);
            }
        }
    }

    // the half-row z loads in place (HalfRow; before phase 2 reads z).  The fused kernel does it
    // at the end of phase 6, where the loads have landed and phase 2's VALU work is not near
    __device__ __forceinline__ void unswap_z() {
        if constexpr (kHalfRowZ) {
#pragma unroll
            for (int s = 0; s < KS; ++s) unswap_halves(pz[s][0], pz[s][1], li < 8);
        }
    }

    __device__ __forceinline__ void phase1(float* beta) {
        if (tid < kC) beta[tid] = __uint_as_float(sizeof(TIn) == 2 ? rbeta << 16 : rbeta);
    }

    // gates, then F = e^{Gamma_i - rho_w}: log2 alpha = g log2(e) (tokens past the end: 0),
    // an inclusive sum over the 16 tokens of the tile (lanes li of one row; a lane with no
    // source adds 0), then one exp2.  The tile-local sum lies in [-80 log2(e), 0], the
    // pages' 16-token bound, so the exponential is finite and normal in fp32.
    __device__ __forceinline__ void phase2(Smem& sm, float gscale) {
        const bool valid = r < clen;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const float4 a0 = *reinterpret_cast<const float4*>(&sm.ae[32 * s + 8 * g]);
            const float4 a1 = *reinterpret_cast<const float4*>(&sm.ae[32 * s + 8 * g + 4]);
            const float ae8[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float sg = fast_rcp(1.f + fast_exp2(ae8[e] * lane8(pz[s][0], pz[s][1], e)));
                F[s][e] = valid ? gscale * sg : 0.f;
            }
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) F[s][e] += row_shr_or_zero<1>(F[s][e]);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) F[s][e] += row_shr_or_zero<2>(F[s][e]);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) F[s][e] += row_shr_or_zero<4>(F[s][e]);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) F[s][e] = fast_exp2(F[s][e] + row_shr_or_zero<8>(F[s][e]));
        if (li == 15) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                *reinterpret_cast<float4*>(&sm.ttile[w][32 * s + 8 * g]) = make_float4(F[s][0], F[s][1], F[s][2], F[s][3]);
                *reinterpret_cast<float4*>(&sm.ttile[w][32 * s + 8 * g + 4]) = make_float4(F[s][4], F[s][5], F[s][6], F[s][7]);
            }
        }
    }

    // per-channel products of tile decays, once per (chunk, head): every wave reads its own
    // row, so no lane selects tiles by the wave index.  e^{Gamma_n} goes to the block.
    __device__ __forceinline__ void phase3(Smem& sm, char* blk) {
        if (tid < DK) {
            const float t0 = sm.ttile[0][tid], t1 = sm.ttile[1][tid], t2 = sm.ttile[2][tid], t3 = sm.ttile[3][tid];
            const float p2 = t0 * t1, p3 = p2 * t2, s12 = t1 * t2;
            sm.pre[0][tid] = 1.f;
            sm.pre[1][tid] = t0;
            sm.pre[2][tid] = p2;
            sm.pre[3][tid] = p3;
            sm.suf[0][tid] = s12 * t3;
            sm.suf[1][tid] = t2 * t3;
            sm.suf[2][tid] = t3;
            sm.suf[3][tid] = 1.f;
            reinterpret_cast<float*>(blk + B::DN)[tid] = p3 * t3;
        }
    }

    // Row operands (registers): Kr = k e^{Gamma_i - rho_w}, Qr likewise.  Column operand (LDS):
    // k e^{rho_{w+1} - Gamma_i}.  Block: K~ = k e^{Gamma_i}, Q~ = q e^{Gamma_i} (lane order,
    // straight from registers); K^n staged for transposition (phase 5), or with KnDirect (the
    // fused kernel, whose block is in LDS) written element by element straight into the
    // transposed lane order of phase 5, which then has nothing left to do.
    template <bool KnDirect = false>
    __device__ __forceinline__ void phase4(Smem& sm, char* blk) {
        // KnDirect: token 16w + li, channel 32s + 8g + e lands in piece
        // (m, sp) = (2s + e / 4, w / 2), lane (li / 4, 4g + e % 4), 2-byte slot
        // 2 (w % 2) + (li % 4) of the piece's eight tokens.  Tokens 2i and 2i + 1 of a channel
        // share a 4-byte word, so lanes li and li ^ 1 swap halves (DPP) and each writes whole
        // words: the even lane channel 2j of both tokens, the odd lane channel 2j + 1.
        const int odd = li & 1;
        char* const kn_lane = blk + B::KN + ((li >> 2) * 16 + 4 * g) * 16 + ((li & 3) >> 1) * 4 +
                              (w >> 1) * 1024 + (w & 1) * 8 + odd * 16;
        const uint32_t kn_sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int ch = 32 * s + 8 * g;
            // two halves of the lane's eight channels (fewer values live at once)
            uint32_t pkr[4], pqr[4], pkc[4], pkt[4], pqt[4], pkn[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                // e^{rho_{w+1} - rho_w}, e^{rho_w} and e^{Gamma_n - rho_{w+1}} of the four channels
                const float4 tw4 = *reinterpret_cast<const float4*>(&sm.ttile[w][ch + 4 * hh]);
                const float4 eR4 = *reinterpret_cast<const float4*>(&sm.pre[w][ch + 4 * hh]);
                const float4 eN4 = *reinterpret_cast<const float4*>(&sm.suf[w][ch + 4 * hh]);
                const float tws[4] = {tw4.x, tw4.y, tw4.z, tw4.w};
                const float eRs[4] = {eR4.x, eR4.y, eR4.z, eR4.w};
                const float eNs[4] = {eN4.x, eN4.y, eN4.z, eN4.w};
                float vkr[4], vqr[4], vkc[4], vkt[4], vqt[4], vkn[4];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int e = 4 * hh + e4;
                    const float tw = tws[e4], eR = eRs[e4], eN = eNs[e4];
                    const float kf = P::at(pk[s], e), qf = P::at(pq[s], e);
                    const float f = F[s][e];
                    const float E = tw * fast_rcp(f);  // e^{rho_{w+1} - Gamma_i}
                    vkr[e4] = kf * f;
                    vqr[e4] = qf * f;
                    vkc[e4] = kf * E;
                    vkt[e4] = vkr[e4] * eR;
                    vqt[e4] = vqr[e4] * eR;
                    vkn[e4] = vkc[e4] * eN;
                }
#pragma unroll
                for (int p2 = 0; p2 < 2; ++p2) {
                    pkr[2 * hh + p2] = pack_bf16x2(vkr[2 * p2], vkr[2 * p2 + 1]);
                    pqr[2 * hh + p2] = pack_bf16x2(vqr[2 * p2], vqr[2 * p2 + 1]);
                    pkc[2 * hh + p2] = pack_bf16x2(vkc[2 * p2], vkc[2 * p2 + 1]);
                    pkt[2 * hh + p2] = pack_bf16x2(vkt[2 * p2], vkt[2 * p2 + 1]);
                    pqt[2 * hh + p2] = pack_bf16x2(vqt[2 * p2], vqt[2 * p2 + 1]);
                    pkn[2 * hh + p2] = pack_bf16x2(vkn[2 * p2], vkn[2 * p2 + 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            kr[s] = make_uint4(pkr[0], pkr[1], pkr[2], pkr[3]);
            qr[s] = make_uint4(pqr[0], pqr[1], pqr[2], pqr[3]);
            const int piece = (w * KS + s) * 64 + lane;
            sm.b.kc[piece] = make_uint4(pkc[0], pkc[1], pkc[2], pkc[3]);
            *reinterpret_cast<uint4*>(blk + B::KT + piece * 16) = make_uint4(pkt[0], pkt[1], pkt[2], pkt[3]);
            *reinterpret_cast<uint4*>(blk + B::QT + piece * 16) = make_uint4(pqt[0], pqt[1], pqt[2], pqt[3]);
            if constexpr (KnDirect) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // channel e = 2j + odd of tokens (li & ~1, li | 1)
                    const uint32_t nb = static_cast<uint32_t>(
                        __builtin_amdgcn_mov_dpp(static_cast<int>(pkn[j]), 0xb1, 0xf, 0xf, true));  // quad_perm [1,0,3,2]
                    const int e = 2 * j;
                    *reinterpret_cast<uint32_t*>(kn_lane + (2 * s + (e >> 2)) * 2048 + (e & 3) * 16) =
                        __builtin_amdgcn_perm(nb, pkn[j], kn_sel);
                }
            } else {
                *reinterpret_cast<uint4*>(&sm.a.kn[r][ch]) = make_uint4(pkn[0], pkn[1], pkn[2], pkn[3]);
            }
        }
    }

    // K^n^T in lane order: piece (m, sp, lane) holds, for lane (g, li), the tokens
    // 32sp + 4g .. and 32sp + 16 + 4g .. of channel pi(m, li)
    __device__ __forceinline__ void phase5(Smem& sm, char* blk) {
        for (int p = tid; p < MT * 2 * 64; p += 256) {
            const int m = p >> 7, sp = (p >> 6) & 1, pl = p & 63, pg = pl >> 4, pli = pl & 15;
            const int c = 32 * (m >> 1) + 8 * (pli >> 2) + 4 * (m & 1) + (pli & 3);
            const int ta = 32 * sp + 4 * pg;
            uint32_t wv[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int t = ta + 16 * hh + 2 * e;
                    wv[2 * hh + e] = static_cast<uint32_t>(sm.a.kn[t][c]) | (static_cast<uint32_t>(sm.a.kn[t + 1][c]) << 16);
                }
            *reinterpret_cast<uint4*>(blk + B::KN + p * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }

    // lower 16x16 tile (w, b), b <= w, of A_kk and A_qk.  The column operand of tile b
    // carries e^{rho_{b+1} - Gamma_j}; it is rescaled per channel by e^{rho_w - rho_{b+1}}
    // (the reciprocal of tile w's own product on the diagonal, at most e^80).  Transposed
    // product: lane ends with four consecutive columns j of one row i.
    __device__ __forceinline__ void tile_products(Smem& sm, int b, f32x4_t& ckk, f32x4_t& cqk) {
        ckk = f32x4_t{0.f, 0.f, 0.f, 0.f};
        cqk = ckk;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int ch = 32 * s + 8 * g;
            uint4 col = sm.b.kc[(b * KS + s) * 64 + lane];
            if (b != w - 1) {
                float4 s0, s1;
                if (b == w) {
                    const float4 t0v = *reinterpret_cast<const float4*>(&sm.ttile[w][ch]);
                    const float4 t1v = *reinterpret_cast<const float4*>(&sm.ttile[w][ch + 4]);
                    s0 = make_float4(fast_rcp(t0v.x), fast_rcp(t0v.y), fast_rcp(t0v.z), fast_rcp(t0v.w));
                    s1 = make_float4(fast_rcp(t1v.x), fast_rcp(t1v.y), fast_rcp(t1v.z), fast_rcp(t1v.w));
                } else {
                    s0 = *reinterpret_cast<const float4*>(&sm.ttile[w - 1][ch]);
                    s1 = *reinterpret_cast<const float4*>(&sm.ttile[w - 1][ch + 4]);
                    if (b == w - 3) {
                        const float4 u0 = *reinterpret_cast<const float4*>(&sm.ttile[w - 2][ch]);
                        const float4 u1 = *reinterpret_cast<const float4*>(&sm.ttile[w - 2][ch + 4]);
                        s0 = make_float4(s0.x * u0.x, s0.y * u0.y, s0.z * u0.z, s0.w * u0.w);
                        s1 = make_float4(s1.x * u1.x, s1.y * u1.y, s1.z * u1.z, s1.w * u1.w);
                    }
                }
                col = scale8(col, s0, s1);
            }
            ckk = mfma32(col, kr[s], ckk);
            cqk = mfma32(col, qr[s], cqk);
        }
    }

    // tile (w, b)'s results: the diagonal A_kk tile (strictly lower, times beta) to fp32
    // scratch Ld for the solve, off-diagonal ones to Lb; A_qk (lower incl. the diagonal) to Ab
    __device__ __forceinline__ void store_tile(Smem& sm, int b, float bi, const f32x4_t& ckk, const f32x4_t& cqk,
                                               bf16_t (*Lb)[16][16], bf16_t (*Ab)[16][16]) {
        const int job = tri_index(w, b);
        if (b == w) {
            float qv[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int jj = 4 * g + rr;
                sm.a.t.Ld[w][jj][li] = jj < li ? bi * ckk[rr] : 0.f;  // strictly lower
                qv[rr] = jj <= li ? cqk[rr] : 0.f;                // lower incl. diagonal
            }
            *reinterpret_cast<uint2*>(&Ab[job][li][4 * g]) =
                make_uint2(pack_bf16x2(qv[0], qv[1]), pack_bf16x2(qv[2], qv[3]));
        } else {
            *reinterpret_cast<uint2*>(&Lb[job][li][4 * g]) =
                make_uint2(pack_bf16x2(bi * ckk[0], bi * ckk[1]), pack_bf16x2(bi * ckk[2], bi * ckk[3]));
            *reinterpret_cast<uint2*>(&Ab[job][li][4 * g]) =
                make_uint2(pack_bf16x2(cqk[0], cqk[1]), pack_bf16x2(cqk[2], cqk[3]));
        }
    }

    // the 10 lower tiles of A_kk and A_qk, row tile w in wave w
    __device__ __forceinline__ void phase6(Smem& sm, const float* beta, bf16_t (*Lb)[16][16],
                                           bf16_t (*Ab)[16][16]) {
        const float bi = beta[r];
        for (int b = 0; b <= w; ++b) {
            f32x4_t ckk, cqk;
            tile_products(sm, b, ckk, cqk);
            store_tile(sm, b, bi, ckk, cqk, Lb, Ab);
        }
    }

    // column j of T_aa = (I + L_aa)^{-1} by fp32 forward substitution from the strictly
    // lower L_aa in Ld[a] (stored column by column)
    __device__ __forceinline__ static void solve_column(const float (*Ld)[20], int j, float (&t)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            float Lm[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 v4 = *reinterpret_cast<const float4*>(&Ld[m][4 * q4]);
                Lm[4 * q4] = v4.x; Lm[4 * q4 + 1] = v4.y; Lm[4 * q4 + 2] = v4.z; Lm[4 * q4 + 3] = v4.w;
            }
            const float tm = t[m];
#pragma unroll
            for (int i = m + 1; i < 16; ++i) t[i] -= Lm[i] * tm;
        }
    }

    // the fused path's phase 6: each wave forms its diagonal tile first and solves its own
    // T_ww right away (the wave reads back only what it wrote, so no barrier), then its
    // off-diagonal tiles, so no later phase waits on one wave solving all four blocks
    __device__ __forceinline__ void phase6_solve(Smem& sm, const float* beta, bf16_t (*Lb)[16][16],
                                                 bf16_t (*Ab)[16][16], bf16_t (*Tb)[16][16]) {
        const float bi = beta[r];
        {
            f32x4_t ckk, cqk;
            tile_products(sm, w, ckk, cqk);
            store_tile(sm, w, bi, ckk, cqk, Lb, Ab);
        }
        // every lane solves column li (the four rows of 16 lanes redundantly); row 0 stores it
        float t[16];
        solve_column(sm.a.t.Ld[w], li, t);
        if (g == 0) {
            const int d = tri_index(w, w);
#pragma unroll
            for (int i = 0; i < 16; ++i) Tb[d][i][li] = f32_to_bf16(t[i]);
        }
        for (int b = 0; b < w; ++b) {
            f32x4_t ckk, cqk;
            tile_products(sm, b, ckk, cqk);
            store_tile(sm, b, bi, ckk, cqk, Lb, Ab);
        }
    }

    // diagonal blocks T_aa = (I + L_aa)^{-1}, fp32 forward substitution (wave 3)
    __device__ __forceinline__ void phase7(Smem& sm, bf16_t (*Tb)[16][16]) {
        if (w != 3) return;
        const int a = lane >> 4, j = lane & 15;
        float t[16];
        solve_column(sm.a.t.Ld[a], j, t);
        // column j of T_aa -> T block (row-major) and its transpose (row j)
        const int d = tri_index(a, a);
#pragma unroll
        for (int i = 0; i < 16; ++i) Tb[d][i][j] = f32_to_bf16(t[i]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<uint2*>(&sm.b.out.Tt[d][j][4 * q4]) =
                make_uint2(pack_bf16x2(t[4 * q4], t[4 * q4 + 1]), pack_bf16x2(t[4 * q4 + 2], t[4 * q4 + 3]));
    }

    // off-diagonal blocks: T_ab = -T_aa sum_{m=b}^{a-1} L_am T_mb, column block b = wave
    __device__ __forceinline__ void phase8(Smem& sm, bf16_t (*Tb)[16][16]) {
        if (w >= 3) return;
        const int b = w;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        for (int a = b + 1; a < 4; ++a) {
            f32x4_t acc = zero;
            for (int m = b; m < a; ++m)
                acc = mfma16(*reinterpret_cast<const uint2*>(&sm.a.t.L[tri_index(a, m)][li][4 * g]),
                             *reinterpret_cast<const uint2*>(&sm.b.out.Tt[tri_index(m, b)][li][4 * g]), acc);
            const f32x4_t tab = mfma16(*reinterpret_cast<const uint2*>(&Tb[tri_index(a, a)][li][4 * g]),
                                       pack_bf16x4(acc), zero);
            // tab[rr] = -T_ab[4g + rr][li]
            const int d = tri_index(a, b);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) Tb[d][4 * g + rr][li] = f32_to_bf16(-tab[rr]);
            *reinterpret_cast<uint2*>(&sm.b.out.Tt[d][li][4 * g]) =
                make_uint2(pack_bf16x2(-tab[0], -tab[1]), pack_bf16x2(-tab[2], -tab[3]));
        }
    }

    // M = A_qk T (lower blocks): M_ab = sum_{m=b}^{a} A_qk[a][m] T_mb
    __device__ __forceinline__ void phase9(Smem& sm, bf16_t (*Mb)[16][16]) {
#pragma unroll
        for (int slot2 = 0; slot2 < 3; ++slot2) {
            const int job = w + slot2 * 4;
            if (job < 10) {
                const int a = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
                const int b = job - (a * (a + 1)) / 2;
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                for (int m = b; m <= a; ++m)
                    acc = mfma16(*reinterpret_cast<const uint2*>(&sm.a.t.Aqk[tri_index(a, m)][li][4 * g]),
                                 *reinterpret_cast<const uint2*>(&sm.b.out.Tt[tri_index(m, b)][li][4 * g]), acc);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Mb[job][4 * g + rr][li] = f32_to_bf16(acc[rr]);
            }
        }
    }
};

// The chunk slot of a (chunk, head) workgroup -> (sequence, first token, valid tokens);
// false for slots past the last chunk.
__device__ __forceinline__ bool slot_chunk(const SplitArgs& args, int slot, int64_t& t0, int& clen) {
    int n;
    int64_t tok0, len, c0;
    if (args.cu) {
        if (slot >= args.chunk_start[args.n_seqs]) return false;
        n = slot_seq(args.chunk_start, args.n_seqs, slot);
        tok0 = args.cu[n];
        len = static_cast<int64_t>(args.cu[n + 1]) - tok0;
        c0 = static_cast<int64_t>(slot - args.chunk_start[n]) * kC;
    } else {
        const int nc = static_cast<int>((args.T + kC - 1) / kC);
        n = slot / nc;
        if (n >= args.n_seqs) return false;
        tok0 = static_cast<int64_t>(n) * args.T;
        len = args.T;
        c0 = static_cast<int64_t>(slot - n * nc) * kC;
    }
    clen = static_cast<int>(len - c0 < kC ? len - c0 : kC);
    t0 = tok0 + c0;
    return true;
}

// One workgroup of four waves per (chunk, head); the factor block goes to global memory.
template <int DK, typename TIn>
__global__ void __launch_bounds__(256, sizeof(TIn) == 2 ? 4 : 2) prefill_intra_kernel(SplitArgs args) {
    using Smem = IntraSmem<DK>;
    // four workgroups per CU (bf16 inputs, see the launch bounds) need their LDS to fit 160 KiB
    static_assert(sizeof(Smem) * (sizeof(TIn) == 2 ? 4 : 2) <= 160 * 1024, "intra-chunk LDS budget");
    using B = Block<DK>;
    __shared__ Smem sm;

    // workgroup -> (chunk slot, head), the head fastest: the workgroups in flight together
    // read the same tokens' rows of every head, which lie next to each other in memory
    const int H = args.H, slot = static_cast<int>(blockIdx.x / H), h = static_cast<int>(blockIdx.x % H);
    int64_t t0;
    int clen;
    if (!slot_chunk(args, slot, t0, clen)) return;
    char* blk = static_cast<char*>(args.blocks) + (static_cast<size_t>(slot) * H + h) * B::BYTES;

    Producer<DK, TIn> pr;
    pr.init(threadIdx.x);
    // the gate constants before the rows, by every thread (past DK they read 0), so the
    // exponential after the row loads waits for them alone
    const uint32_t a_bits = bload4(make_rsrc(args.A + h * DK, DK * 4), pr.tid * 4);
    pr.load(args, h, t0, clen);
    __builtin_amdgcn_sched_barrier(0);
    if (pr.tid < DK) sm.ae[pr.tid] = -expf(__uint_as_float(a_bits)) * kLog2e;
    pr.phase1(sm.beta);
    lds_barrier();
    pr.phase2(sm, args.g_min * kLog2e);
    lds_barrier();
    pr.phase3(sm, blk);
    lds_barrier();
    pr.phase4(sm, blk);
    lds_barrier();
    pr.phase5(sm, blk);
    lds_barrier();  // the tile products below overwrite the K^n staging
    pr.phase6(sm, sm.beta, sm.a.t.L, sm.a.t.Aqk);
    lds_barrier();
    pr.phase7(sm, sm.b.out.T);
    lds_barrier();
    pr.phase8(sm, sm.b.out.T);
    lds_barrier();
    pr.phase9(sm, sm.b.out.M);
    lds_barrier();

    // T and M lower blocks -> factor block (512 bytes per block, 16-byte pieces)
    for (int idx = pr.tid; idx < 2 * 10 * 32; idx += 256) {
        const int which = idx / 320, rem = idx % 320;
        const uint4* src = which == 0 ? reinterpret_cast<const uint4*>(&sm.b.out.T[0][0][0])
                                      : reinterpret_cast<const uint4*>(&sm.b.out.M[0][0][0]);
        *reinterpret_cast<uint4*>(blk + (which == 0 ? B::TB : B::MB) + rem * 16) = src[rem];
    }
}

// ---- K2: serial state pass -----------------------------------------------------------------
// A workgroup runs the chain of one (sequence, head) over a slice of dv columns.  Loader
// waves copy the next chunk's factor block and v slice from global memory straight into the
// other half of a double-buffered LDS stage with LDS-DMA loads (buffer_load_dwordx4 ... lds:
// each instruction writes one contiguous 1 KiB piece, 16 bytes per lane, without passing
// through registers) while the compute waves work on the current half; one workgroup barrier
// per chunk.  The factor block is stored by the intra-chunk kernel in exactly this LDS
// layout, with the operands of the big products in lane order, so every compute read of them
// is a linear, conflict-free ds_read_b128.
//
// A compute wave owns 16 dv columns [col0, col0 + 16) of the state, in registers:
//   S[m][r] = S[pi(m, 4g + r)][col0 + li],
// so that bf16-packing S[2s], S[2s+1] gives, per lane, the eight channels 32 s + 8 g + e,
// which is both the B operand of X = K~ S and the A operand of Y^T = S^T Q~^T.  O is produced
// transposed (O^T = Y^T + R^T M^T), which leaves each lane with four adjacent output columns
// of one token: one 8-byte store per tile, no staging.
//
// Two forms: prefill_state_kernel (NCW compute waves, each running whole chunks for its 16
// columns) and prefill_state_lagged_kernel (one 16-column slice; the output products on a
// second wave, one chunk behind).  Narrower slices shorten the per-chunk critical path and
// make more workgroups read each factor block (from L2).
// Geometry of a chunk's v slice (DVS columns) in LDS: rows of VRB bytes, VRP rows per
// 1 KiB piece, pieces VPS bytes apart.
template <int DVS, typename TIn>
struct VSlice {
    static constexpr int VRB = DVS * static_cast<int>(sizeof(TIn));
    static constexpr int VRP = 1024 / VRB;
    static constexpr int NVP = kC / VRP;
    static constexpr int VPS = 1024 + 32;  // padded piece stride: rows 4 apart fall in other banks
    static constexpr int BYTES = NVP * VPS;
    static_assert(VRP * VRB == 1024 && NVP * VRP == kC, "v pieces");
};

template <int DK, int DVS, typename TIn>
struct StateBuf {
    using V = VSlice<DVS, TIn>;
    static constexpr int VRB = V::VRB, VRP = V::VRP, VPS = V::VPS;
    uint4 blk[Block<DK>::NBP * 64];  // the factor block (the last piece may run past it)
    unsigned char v[V::BYTES];       // v slice, rows of VRB bytes, VRP rows per piece
    float beta[kC];
};

// The (sequence, head, dv slice) chain of one state-pass workgroup.  Consecutive workgroups
// go to different XCDs, and all slices of one (sequence, head) to the same XCD, where they
// share the L2 copy of its factor blocks.
struct ChainPos {
    int n, h, slice, slot0, nchunks;
    int64_t tok0, len;
};
__device__ __forceinline__ bool chain_pos(const SplitArgs& a, ChainPos& p) {
    const int bid = blockIdx.x;
    const int xcd = bid & 7, kq = bid >> 3;
    const int pair = (kq / a.nslices) * 8 + xcd;
    if (pair >= a.npairs) return false;
    p.slice = kq % a.nslices;
    p.n = pair / a.H;
    p.h = pair - p.n * a.H;
    if (a.cu) {
        p.tok0 = a.cu[p.n];
        p.len = static_cast<int64_t>(a.cu[p.n + 1]) - p.tok0;
        p.slot0 = a.chunk_start[p.n];
    } else {
        p.tok0 = static_cast<int64_t>(p.n) * a.T;
        p.len = a.T;
        p.slot0 = p.n * static_cast<int>((a.T + kC - 1) / kC);
    }
    p.nchunks = static_cast<int>((p.len + kC - 1) / kC);
    return true;
}

// Loader waves of the state pass: NLW waves move the NBP pieces (1 KiB) of a chunk's factor
// block and the NVP pieces of its v slice into LDS with LDS-DMA copies (16 bytes per lane,
// not through registers), piece p by wave p mod NLW; block pieces below Block::NQP (Q~, M) go
// to one destination, the rest (K~, K^n, T, e^{Gamma_n}) to another.  With each chunk's copies
// they also pull the next chunk's block lines (this slice's share, line slice + nslices m) and
// v rows into L2, with 4-byte LDS-DMA loads into a dummy area that nothing reads, so nothing
// waits for them: the next copies then find their lines in L2 instead of waiting on the
// farther memory with only one chunk of look-ahead.
template <int DK, int DVS, typename TIn, int NLW, int TL = 1>
struct StageLoader {
    using V = VSlice<DVS, TIn>;
    using B = Block<DK>;
    static constexpr int NBP = B::NBP, NQP = B::NQP, NVP = V::NVP, VRP = V::VRP, VRB = V::VRB;
    static constexpr int LPR = VRB / 16;  // lanes per v row
    static constexpr int PPW = (NBP + NVP + NLW - 1) / NLW;
    static constexpr int LINES = static_cast<int>(B::BYTES / 128);
    static constexpr int TPW = (LINES + 64 * NLW - 1) / (64 * NLW) + 1;  // + 1: v rows
    const char* blocks;   // factor block of chunk 0 of this (sequence, head)
    size_t block_stride;  // bytes from one chunk's block to the next
    const char* v;        // v[tok0][h][first column of the slice]
    const char* beta;     // beta[tok0][h]
    int64_t len;
    uint32_t rowV, rowB;  // bytes per token of v and beta
    int lw, lane, slice, nslices, nchunks;
    uint32_t rbr = 0;     // raw beta bits, converted only when stored (a use here would wait)

    __device__ __forceinline__ int chunk_len(int c) const {
        const int64_t rem = len - static_cast<int64_t>(c) * kC;
        return rem < kC ? static_cast<int>(rem) : kC;
    }
    // Copies of chunk c: block pieces p < NQP to q + 64 p, the others to a + 64 (p - NQP), v
    // pieces to vdst.  Then the L2 warm-up of chunk c + TL: 4-byte LDS-DMA loads of its lines
    // into the dummy words `sink` (64 per wave), which nothing reads, so nothing waits for them.
    __device__ __forceinline__ void fetch(int c, uint4* q, uint4* a, unsigned char* vdst, uint32_t* sink) {
        const int clen = chunk_len(c);
        const rsrc_t rf = make_rsrc(blocks + static_cast<size_t>(c) * block_stride, B::BYTES);
        const rsrc_t rv = make_rsrc(v + static_cast<int64_t>(c) * kC * rowV, clen * rowV);
        if (lw == 0) {
            const rsrc_t rbs = make_rsrc(beta + static_cast<int64_t>(c) * kC * rowB, clen * rowB);
            if constexpr (sizeof(TIn) == 2) rbr = bload2(rbs, lane * rowB);
            else rbr = bload4(rbs, lane * rowB);
        }
#pragma unroll
        for (int i = 0; i < PPW; ++i) {
            const int p = lw + NLW * i;
            if (p < NQP) {
                dma16(rf, q + p * 64, p * 1024 + lane * 16);
            } else if (p < NBP) {
                dma16(rf, a + (p - NQP) * 64, p * 1024 + lane * 16);
            } else if (p < NBP + NVP) {
                const int j = p - NBP;
                dma16(rv, vdst + j * V::VPS, (j * VRP + lane / LPR) * rowV + (lane % LPR) * 16);
            }
        }
        // warm-up (a no-op past the last chunk: empty ranges load nothing)
        const int cn = c + TL;
        const bool live = cn < nchunks;
        const rsrc_t tf = make_rsrc(blocks + static_cast<size_t>(cn) * block_stride, live ? B::BYTES : 0);
        const rsrc_t tv = make_rsrc(v + static_cast<int64_t>(cn) * kC * rowV, live ? chunk_len(cn) * rowV : 0);
#pragma unroll
        for (int i = 0; i + 1 < TPW; ++i)
            dma4(tf, sink, static_cast<uint32_t>(slice + nslices * (lane + 64 * (lw + NLW * i))) * 128);
        dma4(tv, sink, lw == 0 ? lane * rowV : 0x7ffffff0u);
    }
    // wait for the copies (the TPW newest loads, the warm-up, may stay in flight) and store beta
    __device__ __forceinline__ void commit(float* bdst) {
        // s_waitcnt fields: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
        __builtin_amdgcn_s_waitcnt((TPW & 15) | (7 << 4) | (15 << 8) | ((TPW >> 4) << 14));
        if (lw == 0) bdst[lane] = __uint_as_float(sizeof(TIn) == 2 ? rbr << 16 : rbr);
    }
    // The loaders' side of the chunk barrier.  A release fence would wait for every LDS-DMA
    // load, the warm-up included; the copies are already complete (commit), so only the beta
    // store is waited for here.  The empty asm statements keep the compiler from moving LDS
    // accesses across the barrier.
    __device__ __forceinline__ static void barrier() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
};

template <int DK, int DVS, typename TIn, int NLW>
__device__ __forceinline__ StageLoader<DK, DVS, TIn, NLW> make_loader(const SplitArgs& a, const ChainPos& p, int lw) {
    using B = Block<DK>;
    constexpr int ES = static_cast<int>(sizeof(TIn));
    StageLoader<DK, DVS, TIn, NLW> ld;
    const int dv = DK;
    ld.blocks = static_cast<const char*>(a.blocks) + (static_cast<size_t>(p.slot0) * a.H + p.h) * B::BYTES;
    ld.block_stride = static_cast<size_t>(a.H) * B::BYTES;
    ld.v = static_cast<const char*>(a.v) +
           (p.tok0 * a.H * dv + static_cast<int64_t>(p.h) * dv + static_cast<int64_t>(p.slice) * DVS) * ES;
    ld.beta = static_cast<const char*>(a.beta) + (p.tok0 * a.H + p.h) * ES;
    ld.len = p.len;
    ld.rowV = static_cast<uint32_t>(a.H) * dv * ES;
    ld.rowB = static_cast<uint32_t>(a.H) * ES;
    ld.lw = lw;
    ld.lane = threadIdx.x & 63;
    ld.slice = p.slice;
    ld.nslices = a.nslices;
    ld.nchunks = p.nchunks;
    return ld;
}

// x of lane L of this lane's row of 16 lanes: DPP control row_newbcast:L (0x150 + L), a
// CDNA3/CDNA4 broadcast within each row
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + L, 0xf, 0xf, false));
}

template <int DK, int NCW, int NLW, typename TIn>
__global__ void __launch_bounds__(64 * (NCW + NLW)) prefill_state_kernel(SplitArgs args) {
    constexpr int DVS = 16 * NCW;  // columns per workgroup (16 per compute wave)
    using Buf = StateBuf<DK, DVS, TIn>;
    using B = Block<DK>;
    constexpr int KS = DK / 32;
    constexpr int MT = DK / 16;
    constexpr int ES = static_cast<int>(sizeof(TIn));
    constexpr int VRP = Buf::VRP, VRB = Buf::VRB;

    __shared__ Buf sm[2];
    __shared__ uint32_t tsink[64];  // target of the loaders' L2 warm-up loads, never read
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;
    ChainPos cp;
    if (!chain_pos(args, cp)) return;
    const int H = args.H, n = cp.n, h = cp.h, slice = cp.slice, nchunks = cp.nchunks;
    const int64_t tok0 = cp.tok0, len = cp.len;
    const int dv = DK;
    const uint32_t rowV = static_cast<uint32_t>(H) * dv * ES;

    if (w >= NCW) {
        // ================================ loader waves ================================
        auto ld = make_loader<DK, DVS, TIn, NLW>(args, cp, w - NCW);
        if (nchunks > 0) {
            ld.fetch(0, sm[0].blk, sm[0].blk + B::NQP * 64, sm[0].v, tsink);
            ld.commit(sm[0].beta);
        }
        ld.barrier();
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) {
                Buf& b = sm[(c + 1) & 1];
                ld.fetch(c + 1, b.blk, b.blk + B::NQP * 64, b.v, tsink);
                ld.commit(b.beta);
            }
            ld.barrier();
        }
        return;
    }

    // ================================ compute waves ================================
    const int col0 = slice * DVS + 16 * w;
    char* obase = static_cast<char*>(args.o) + (static_cast<size_t>(h) * dv + col0) * ES;

    f32x4_t S[MT];
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * dv + col0 + li;
    if (args.s0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[m][r] = args.s0[sbase + static_cast<size_t>(32 * (m >> 1) + 8 * g + 4 * (m & 1) + r) * dv];
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) S[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // this wave's columns of the state to dst = &S[0][col0 + li] of one (sequence, head)
    auto store_state = [&](float* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[static_cast<size_t>(32 * (m >> 1) + 8 * g + 4 * (m & 1) + r) * dv] = S[m][r];
    };
    lds_barrier();

    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nchunks; ++c) {
        const Buf& b = sm[c & 1];
        const uint4* kt = b.blk + B::KT / 16;
        const uint4* qt = b.blk + B::QT / 16;
        const uint4* kn = b.blk + B::KN / 16;
        const uint2* tb = reinterpret_cast<const uint2*>(b.blk + B::TB / 16);
        const uint2* mb = reinterpret_cast<const uint2*>(b.blk + B::MB / 16);
        const float* dnv = reinterpret_cast<const float*>(b.blk + B::DN / 16);
        const int64_t rem = len - static_cast<int64_t>(c) * kC;
        const int clen = rem < kC ? static_cast<int>(rem) : kC;
        const int64_t t0 = tok0 + static_cast<int64_t>(c) * kC;
        const rsrc_t ro = make_rsrc(obase + t0 * rowV, clen * rowV);

        const int vc = 16 * w + li;  // this lane's v column in the slice
        uint4 Sb[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
            Sb[s] = make_uint4(pack_bf16x2(S[2 * s][0], S[2 * s][1]), pack_bf16x2(S[2 * s][2], S[2 * s][3]),
                               pack_bf16x2(S[2 * s + 1][0], S[2 * s + 1][1]),
                               pack_bf16x2(S[2 * s + 1][2], S[2 * s + 1][3]));
        // The four token tiles are independent until U, so every product below is written as
        // four (or more) interleaved accumulation chains that keep the MFMA pipe busy.  Each
        // phase first issues all its LDS operand reads into registers; a scheduling fence keeps
        // them ahead of the MFMAs, so the waits on them are pipelined instead of one full LDS
        // latency per product.
        uint4 opd[4][KS];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int s = 0; s < KS; ++s) opd[a][s] = kt[(a * KS + s) * 64 + lane];
        float vv[4][4];  // v[16a + 4g + r][col vc]
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * a + 4 * g + r;
                const unsigned char* vp = b.v + (row / VRP) * Buf::VPS + (row % VRP) * VRB + vc * ES;
                if constexpr (sizeof(TIn) == 2) vv[a][r] = bf16_to_f32(*reinterpret_cast<const bf16_t*>(vp));
                else vv[a][r] = *reinterpret_cast<const float*>(vp);
            }
        // beta[16a + 4g + r], read once per row of 16 lanes (lane li holds a = li / 4, r = li % 4)
        // and spread over the row by DPP broadcasts below, instead of a 16-fold broadcast read
        const float bsrc = b.beta[16 * (li >> 2) + 4 * g + (li & 3)];
        __builtin_amdgcn_sched_barrier(0);
        // X = K~ S: X[a][r] = X[16a + 4g + r][col li]
        f32x4_t X[4] = {zero, zero, zero, zero};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int a = 0; a < 4; ++a) X[a] = mfma32(opd[a][s], Sb[s], X[a]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int s = 0; s < KS; ++s) opd[a][s] = qt[(a * KS + s) * 64 + lane];
        uint2 tv[10], mv[10];
#pragma unroll
        for (int t = 0; t < 10; ++t) {
            tv[t] = tb[t * 64 + li * 4 + g];
            mv[t] = mb[t * 64 + li * 4 + g];
        }
        __builtin_amdgcn_sched_barrier(0);
        // Y^T = S^T Q~^T (independent of X; the R arithmetic below fills its MFMA latency)
        f32x4_t Yt[4] = {zero, zero, zero, zero};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int a = 0; a < 4; ++a) Yt[a] = mfma32(Sb[s], opd[a][s], Yt[a]);
        float4 bb[4];
        bb[0] = make_float4(row_bcast<0>(bsrc), row_bcast<1>(bsrc), row_bcast<2>(bsrc), row_bcast<3>(bsrc));
        bb[1] = make_float4(row_bcast<4>(bsrc), row_bcast<5>(bsrc), row_bcast<6>(bsrc), row_bcast<7>(bsrc));
        bb[2] = make_float4(row_bcast<8>(bsrc), row_bcast<9>(bsrc), row_bcast<10>(bsrc), row_bcast<11>(bsrc));
        bb[3] = make_float4(row_bcast<12>(bsrc), row_bcast<13>(bsrc), row_bcast<14>(bsrc), row_bcast<15>(bsrc));
        // R = beta (V - X).  Rows past the chunk's end are zero without a test: the v copy
        // writes zeros there, beta reads as zero, and K~ rows are zero, so X is zero too.
        uint2 Rb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t R;
            R[0] = bb[a].x * (vv[a][0] - X[a][0]);
            R[1] = bb[a].y * (vv[a][1] - X[a][1]);
            R[2] = bb[a].z * (vv[a][2] - X[a][2]);
            R[3] = bb[a].w * (vv[a][3] - X[a][3]);
            Rb[a] = pack_bf16x4(R);  // lane: R[16a + 4g + r][col li]
        }
        // U = T R and O^T = Y^T + R^T M^T, chains over the source tile b.  The M R chain starts
        // from zero and Y^T is added on the VALU: an accumulator is never handed from a
        // 16x16x32 product to a 16x16x16 one, a cross-shape dependency that the generated code
        // did not always space far enough apart.
        f32x4_t U[4] = {zero, zero, zero, zero}, Om[4] = {zero, zero, zero, zero};
#pragma unroll
        for (int bq = 0; bq < 4; ++bq)
#pragma unroll
            for (int a = bq; a < 4; ++a) {
                const int t = tri_index(a, bq);
                U[a] = mfma16(tv[t], Rb[bq], U[a]);
                Om[a] = mfma16(Rb[bq], mv[t], Om[a]);
            }
        uint2 Ub[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) Ub[a] = pack_bf16x4(U[a]);
        __builtin_amdgcn_sched_barrier(0);
        // S = diag(e^{Gamma_n}) S + K^n^T U
        uint4 kk[2][MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            kk[0][m] = kn[(m * 2 + 0) * 64 + lane];
            kk[1][m] = kn[(m * 2 + 1) * 64 + lane];
        }
        // e^{Gamma_n} of state row 32 (j / 8) + 8 g + j % 8 for j = 4 m + r: lane li of a row
        // reads j = 2 li, 2 li + 1 (wrapped inside the DK rows; at DK = 64 lanes 8..15 are
        // unused), then DPP broadcasts spread them over the row
        const float2 dsrc = *reinterpret_cast<const float2*>(
            &dnv[32 * ((li >> 2) & (DK / 32 - 1)) + 8 * g + 2 * (li & 3)]);
        __builtin_amdgcn_sched_barrier(0);
        float4 dn[MT];
        auto dj = [&](auto J) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            return row_bcast<j / 2>((j & 1) ? dsrc.y : dsrc.x);
        };
        auto dn4 = [&](auto M) __attribute__((always_inline)) {
            constexpr int m = decltype(M)::value;
            return make_float4(dj(std::integral_constant<int, 4 * m>{}), dj(std::integral_constant<int, 4 * m + 1>{}),
                               dj(std::integral_constant<int, 4 * m + 2>{}), dj(std::integral_constant<int, 4 * m + 3>{}));
        };
        dn[0] = dn4(std::integral_constant<int, 0>{});
        dn[1] = dn4(std::integral_constant<int, 1>{});
        dn[2] = dn4(std::integral_constant<int, 2>{});
        dn[3] = dn4(std::integral_constant<int, 3>{});
        if constexpr (MT > 4) {
            dn[4] = dn4(std::integral_constant<int, 4>{});
            dn[5] = dn4(std::integral_constant<int, 5>{});
            dn[6] = dn4(std::integral_constant<int, 6>{});
            dn[7] = dn4(std::integral_constant<int, 7>{});
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            S[m][0] *= dn[m].x;
            S[m][1] *= dn[m].y;
            S[m][2] *= dn[m].z;
            S[m][3] *= dn[m].w;
        }
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                S[m] = mfma32(kk[sp][m], make_uint4(Ub[2 * sp].x, Ub[2 * sp].y, Ub[2 * sp + 1].x, Ub[2 * sp + 1].y), S[m]);
        // O: Ot[r] = O[16a + li][col0 + 4g + r]
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4_t Ot = Om[a] + Yt[a];
            const uint32_t off = static_cast<uint32_t>(16 * a + li) * rowV + 4 * g * ES;
            if constexpr (sizeof(TIn) == 2) {
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(Ot[0], Ot[1]), pack_bf16x2(Ot[2], Ot[3])},
                                                      ro, off, 0, 0);
            } else {
                bstore16(ro, off, make_uint4(__float_as_uint(Ot[0]), __float_as_uint(Ot[1]),
                                             __float_as_uint(Ot[2]), __float_as_uint(Ot[3])));
            }
        }
        // prefix-cache checkpoint: the state after every ckpt_chunks full chunks
        if (args.ckpt && (c + 1) % args.ckpt_chunks == 0 && static_cast<int64_t>(c + 1) * kC <= len) {
            const int j = (c + 1) / args.ckpt_chunks - 1;
            const int64_t first = args.ckpt_off ? args.ckpt_off[n] : static_cast<int64_t>(n) * args.ckpt_per_seq;
            store_state(args.ckpt + ((first + j) * H + h) * DK * dv + col0 + li);
        }
        lds_barrier();
    }

    if (args.sN) store_state(args.sN + sbase);
}

// Lagged state pass for 16-column slices: the outputs leave the serial chain.  Wave 0 (chain)
// runs the recurrence X = K~ S, R = beta (V - X), U = T R, S' = diag(e^{Gamma_n}) S + K^n^T U
// over chunk c while wave 1 (output) forms O = Q~ S + M R of chunk c - 1 from the chain's
// packed S and R of that chunk, handed over in LDS -- the output products run on another SIMD
// one chunk behind, and one barrier per chunk still orders everything.  Buffers live as long
// as that needs: the recurrence part of the factor block, v and beta in two stages (chunk
// c + 1 lands while c runs), the Q~/M part and the packed S in three (chunk c - 1 is read while
// c + 1 lands / S(c + 1) is written), R in two.
template <int DK, typename TIn>
struct LagBuf {
    using V = VSlice<16, TIn>;
    using B = Block<DK>;
    static constexpr int NAP = B::NBP - B::NQP;  // pieces of K~, K^n, T, e^{Gamma_n}
    struct Stage {
        uint4 a[NAP * 64];
        unsigned char v[V::BYTES];
        float beta[kC];
    };
    Stage st[2];
    uint4 q[3][B::NQP * 64];   // Q~, M
    uint4 xs[3][DK / 32 * 64]; // packed S of a chunk start, in the chain wave's lane order
    uint2 xr[2][4 * 64];       // packed R, in the chain wave's lane order
    uint32_t tsink[64];        // target of the loaders' L2 warm-up loads, never read
};

template <int DK, int NLW, typename TIn>
__global__ void __launch_bounds__(64 * (2 + NLW)) prefill_state_lagged_kernel(SplitArgs args) {
    using L = LagBuf<DK, TIn>;
    using V = VSlice<16, TIn>;
    using B = Block<DK>;
    constexpr int KS = DK / 32;
    constexpr int MT = DK / 16;
    constexpr int ES = static_cast<int>(sizeof(TIn));
    // piece offsets (uint4 units) of the recurrence operands inside a stage's a[]
    constexpr int OKT = 0, OKN = (B::KN - B::KT) / 16, OTB = (B::TB - B::KT) / 16, ODN = (B::DN - B::KT) / 16;

    __shared__ L sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;
    ChainPos cp;
    if (!chain_pos(args, cp)) return;
    const int H = args.H, n = cp.n, h = cp.h, nchunks = cp.nchunks;
    const int64_t tok0 = cp.tok0, len = cp.len;
    const int dv = DK;
    const uint32_t rowV = static_cast<uint32_t>(H) * dv * ES;
    const int col0 = cp.slice * 16;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

    if (w >= 2) {
        // ================================ loader waves ================================
        auto ld = make_loader<DK, 16, TIn, NLW>(args, cp, w - 2);
        if (nchunks > 0) {
            ld.fetch(0, sm.q[0], sm.st[0].a, sm.st[0].v, sm.tsink);
            ld.commit(sm.st[0].beta);
        }
        ld.barrier();
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) {
                typename L::Stage& b = sm.st[(c + 1) & 1];
                ld.fetch(c + 1, sm.q[(c + 1) % 3], b.a, b.v, sm.tsink);
                ld.commit(b.beta);
            }
            ld.barrier();
        }
        return;
    }

    if (w == 1) {
        // ================================ output wave ================================
        char* obase = static_cast<char*>(args.o) + (static_cast<size_t>(h) * dv + col0) * ES;
        // O of chunk e: O^T = S^T Q~^T + R^T M^T
        auto out = [&](int e) __attribute__((always_inline)) {
            const uint4* qt = sm.q[e % 3] + B::QT / 16;
            const uint2* mb = reinterpret_cast<const uint2*>(sm.q[e % 3] + B::MB / 16);
            const int64_t rem = len - static_cast<int64_t>(e) * kC;
            const int clen = rem < kC ? static_cast<int>(rem) : kC;
            const rsrc_t ro = make_rsrc(obase + (tok0 + static_cast<int64_t>(e) * kC) * rowV, clen * rowV);
            uint4 Sb[KS], opd[4][KS];
            uint2 Rb[4], mv[10];
#pragma unroll
            for (int s = 0; s < KS; ++s) Sb[s] = sm.xs[e % 3][s * 64 + lane];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int s = 0; s < KS; ++s) opd[a][s] = qt[(a * KS + s) * 64 + lane];
#pragma unroll
            for (int a = 0; a < 4; ++a) Rb[a] = sm.xr[e & 1][a * 64 + lane];
#pragma unroll
            for (int t = 0; t < 10; ++t) mv[t] = mb[t * 64 + li * 4 + g];
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t Yt[4] = {zero, zero, zero, zero}, Om[4] = {zero, zero, zero, zero};
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int a = 0; a < 4; ++a) Yt[a] = mfma32(Sb[s], opd[a][s], Yt[a]);
            // the M R chain starts from zero and Y^T is added on the VALU, so no accumulator
            // passes from a 16x16x32 product to a 16x16x16 one
#pragma unroll
            for (int bq = 0; bq < 4; ++bq)
#pragma unroll
                for (int a = bq; a < 4; ++a) Om[a] = mfma16(Rb[bq], mv[tri_index(a, bq)], Om[a]);
            // Ot[r] = O[16a + li][col0 + 4g + r]
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4_t Ot = Om[a] + Yt[a];
                const uint32_t off = static_cast<uint32_t>(16 * a + li) * rowV + 4 * g * ES;
                if constexpr (sizeof(TIn) == 2) {
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2_t{pack_bf16x2(Ot[0], Ot[1]), pack_bf16x2(Ot[2], Ot[3])}, ro, off, 0, 0);
                } else {
                    bstore16(ro, off, make_uint4(__float_as_uint(Ot[0]), __float_as_uint(Ot[1]),
                                                 __float_as_uint(Ot[2]), __float_as_uint(Ot[3])));
                }
            }
        };
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            if (c > 0) out(c - 1);
            lds_barrier();
        }
        if (nchunks > 0) out(nchunks - 1);
        return;
    }

    // ================================ chain wave ================================
    f32x4_t S[MT];
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * dv + col0 + li;
    // state row of accumulator element (m, r): 32 (m / 2) + 8 g + 4 (m % 2) + r
    if (args.s0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[m][r] = args.s0[sbase + static_cast<size_t>(32 * (m >> 1) + 8 * g + 4 * (m & 1) + r) * dv];
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) S[m] = zero;
    }
    auto store_state = [&](float* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[static_cast<size_t>(32 * (m >> 1) + 8 * g + 4 * (m & 1) + r) * dv] = S[m][r];
    };
    // packed bf16 state: the B operand of X = K~ S here, the A operand of Y^T in the output wave
    uint4 Sb[KS];
    auto pack_state = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            Sb[s] = make_uint4(pack_bf16x2(S[2 * s][0], S[2 * s][1]), pack_bf16x2(S[2 * s][2], S[2 * s][3]),
                               pack_bf16x2(S[2 * s + 1][0], S[2 * s + 1][1]),
                               pack_bf16x2(S[2 * s + 1][2], S[2 * s + 1][3]));
            sm.xs[slot][s * 64 + lane] = Sb[s];
        }
    };
    pack_state(0);
    lds_barrier();

    for (int c = 0; c < nchunks; ++c) {
        const typename L::Stage& b = sm.st[c & 1];
        const uint4* kt = b.a + OKT;
        const uint4* kn = b.a + OKN;
        const uint2* tb = reinterpret_cast<const uint2*>(b.a + OTB);
        const float* dnv = reinterpret_cast<const float*>(b.a + ODN);
        uint4 opd[4][KS];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int s = 0; s < KS; ++s) opd[a][s] = kt[(a * KS + s) * 64 + lane];
        float vv[4][4];  // v[16a + 4g + r][col li]
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * a + 4 * g + r;
                const unsigned char* vp = b.v + (row / V::VRP) * V::VPS + (row % V::VRP) * V::VRB + li * ES;
                if constexpr (sizeof(TIn) == 2) vv[a][r] = bf16_to_f32(*reinterpret_cast<const bf16_t*>(vp));
                else vv[a][r] = *reinterpret_cast<const float*>(vp);
            }
        float4 bb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) bb[a] = *reinterpret_cast<const float4*>(&b.beta[16 * a + 4 * g]);
        uint2 tv[10];
#pragma unroll
        for (int t = 0; t < 10; ++t) tv[t] = tb[t * 64 + li * 4 + g];
        __builtin_amdgcn_sched_barrier(0);
        // X = K~ S: X[a][r] = X[16a + 4g + r][col li], four interleaved chains
        f32x4_t X[4] = {zero, zero, zero, zero};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int a = 0; a < 4; ++a) X[a] = mfma32(opd[a][s], Sb[s], X[a]);
        __builtin_amdgcn_sched_barrier(0);
        uint4 kk[2][MT];
        float4 dn[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            kk[0][m] = kn[(m * 2 + 0) * 64 + lane];
            kk[1][m] = kn[(m * 2 + 1) * 64 + lane];
            dn[m] = *reinterpret_cast<const float4*>(&dnv[32 * (m >> 1) + 8 * g + 4 * (m & 1)]);
        }
        // R = beta (V - X).  Rows past the chunk's end are zero without a test: the v copy
        // writes zeros there, beta reads as zero, and K~ rows are zero, so X is zero too.
        uint2 Rb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t R;
            R[0] = bb[a].x * (vv[a][0] - X[a][0]);
            R[1] = bb[a].y * (vv[a][1] - X[a][1]);
            R[2] = bb[a].z * (vv[a][2] - X[a][2]);
            R[3] = bb[a].w * (vv[a][3] - X[a][3]);
            Rb[a] = pack_bf16x4(R);  // lane: R[16a + 4g + r][col li]
            sm.xr[c & 1][a * 64 + lane] = Rb[a];
        }
        // U = T R, chains over the source tile
        f32x4_t U[4] = {zero, zero, zero, zero};
#pragma unroll
        for (int bq = 0; bq < 4; ++bq)
#pragma unroll
            for (int a = bq; a < 4; ++a) U[a] = mfma16(tv[tri_index(a, bq)], Rb[bq], U[a]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            S[m][0] *= dn[m].x;
            S[m][1] *= dn[m].y;
            S[m][2] *= dn[m].z;
            S[m][3] *= dn[m].w;
        }
        uint2 Ub[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) Ub[a] = pack_bf16x4(U[a]);
        // S = diag(e^{Gamma_n}) S + K^n^T U
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                S[m] = mfma32(kk[sp][m], make_uint4(Ub[2 * sp].x, Ub[2 * sp].y, Ub[2 * sp + 1].x, Ub[2 * sp + 1].y), S[m]);
        // prefix-cache checkpoint: the state after every ckpt_chunks full chunks
        if (args.ckpt && (c + 1) % args.ckpt_chunks == 0 && static_cast<int64_t>(c + 1) * kC <= len) {
            const int jc = (c + 1) / args.ckpt_chunks - 1;
            const int64_t first = args.ckpt_off ? args.ckpt_off[n] : static_cast<int64_t>(n) * args.ckpt_per_seq;
            store_state(args.ckpt + ((first + jc) * H + h) * DK * dv + col0 + li);
        }
        pack_state((c + 1) % 3);
        lds_barrier();
    }

    if (args.sN) store_state(args.sN + sbase);
}

// ---- fused prefill: intra-chunk factors and the state pass in one workgroup -------------
// One workgroup of eight waves per (sequence, head) chain.  Waves 0-3 (producers) build
// the factor block of chunk c + 1 into one LDS stage with intra-chunk phases 1-4 and 6 above
// (phase 4 writing K^n^T itself, phase 6 in the form that also solves the diagonal blocks of
// T), while
// waves 4-7 (consumers) run the state pass over chunk c from the other stage, each owning
// DK / 4 columns of the dk x dv state in MFMA accumulators.  The factor block never leaves
// the CU, so the call moves only the method's own bytes through HBM: q, k, v, beta, z in, o
// out, and the states.  The two groups share the workgroup barrier: every iteration runs the
// producers' five phase barriers, and the consumers place their phases between them.
// Unlike the split path, the stage holds the diagonal blocks T_aa of T = (I + A_kk)^{-1}, the
// strictly lower blocks L of A_kk and the blocks of A_qk: the consumers apply T by block
// forward substitution, which takes the off-diagonal T blocks and M = A_qk T (phases 8-9)
// off the producers' serial path.
// Producers load chunk c + 1's q, k, z and beta into the registers that chunk c's operands
// have released, at the start of phase 6: issued beside the LDS-heavy phases 4 and 5, the same
// loads stalled those phases for thousands of cycles.  The consumers load the next chunk's v
// after phase C, for the same reason.
template <int DK>
struct FusedSmem {
    struct Stage {
        uint4 blk[Block<DK>::BYTES / 16];  // factor block in the state pass's LDS layout
        float beta[kC];
    };
    IntraSmem<DK> p;  // producer scratch
    Stage st[2];
};

// Consumer wave: NH halves of 16 state columns, [col0 + 16 h, col0 + 16 h + 16).  The state
// rows are kept in the permuted order pi(m, i) of the state pass, so bf16-packing two
// accumulator tiles gives each lane eight consecutive key channels.
template <int DK, typename TIn>
struct Consumer {
    static constexpr int NH = DK / 64;
    static constexpr int KS = DK / 32;
    static constexpr int MT = DK / 16;
    static constexpr int ES = static_cast<int>(sizeof(TIn));
    using B = Block<DK>;
    using Stage = typename FusedSmem<DK>::Stage;

    int lane, g, li, col0;
    f32x4_t S[NH][MT];
    uint32_t vr[NH][4][4];  // v[16a + 4g + r][col0 + 16h + li] of the next chunk, as fp32 bits
    uint2 Rb[NH][4];
    uint2 Ub[NH][4];
    f32x4_t Yt[NH][4];      // Y^T = S^T Q~^T of the chunk, from phase Y to phase B

    // bf16-packed state, half h, K-step s: the eight key channels 32 s + 8 g .. of the lane
    __device__ __forceinline__ uint4 packed_state(int h, int s) const {
        return make_uint4(pack_bf16x2(S[h][2 * s][0], S[h][2 * s][1]),
                          pack_bf16x2(S[h][2 * s][2], S[h][2 * s][3]),
                          pack_bf16x2(S[h][2 * s + 1][0], S[h][2 * s + 1][1]),
                          pack_bf16x2(S[h][2 * s + 1][2], S[h][2 * s + 1][3]));
    }

    // v rows of the chunk at token t0 with n_valid tokens (rows past the end read 0)
    // (the lane's part of each offset is one VGPR; the row and half parts are wave-uniform and
    // go in the instruction's scalar offset)
    __device__ __forceinline__ void load_v(const char* vbase, uint32_t rowV, int64_t t0, int n_valid) {
        const rsrc_t rv = make_rsrc(vbase + t0 * rowV, n_valid * rowV);
        const uint32_t voff = static_cast<uint32_t>(4 * g) * rowV + static_cast<uint32_t>(col0 + li) * ES;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t soff = static_cast<uint32_t>(16 * a + r) * rowV + 16 * h * ES;
                    if constexpr (sizeof(TIn) == 2)
                        vr[h][a][r] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rv, voff, soff, 0)) << 16;
                    else
                        vr[h][a][r] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff, soff, 0);
                }
    }

    // X = K~ S, R = beta (V - X).  Rows past the chunk's end are zero without a test: v and
    // beta read as zero there and K~ rows are zero.  The chunk's v was loaded after the
    // previous chunk's last phase.
    __device__ __forceinline__ void phaseA(const Stage& b) {
        const uint4* kt = b.blk + B::KT / 16;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        f32x4_t X[NH][4];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int a = 0; a < 4; ++a) X[h][a] = zero;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 opd[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) opd[a] = kt[(a * KS + s) * 64 + lane];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const uint4 sb = packed_state(h, s);
#pragma unroll
                for (int a = 0; a < 4; ++a) X[h][a] = mfma32(opd[a], sb, X[h][a]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // beta[16a + 4g + r], read once per row of 16 lanes and spread by DPP row broadcasts
        const float bsrc = b.beta[16 * (li >> 2) + 4 * g + (li & 3)];
        float4 bb[4];
        bb[0] = make_float4(row_bcast<0>(bsrc), row_bcast<1>(bsrc), row_bcast<2>(bsrc), row_bcast<3>(bsrc));
        bb[1] = make_float4(row_bcast<4>(bsrc), row_bcast<5>(bsrc), row_bcast<6>(bsrc), row_bcast<7>(bsrc));
        bb[2] = make_float4(row_bcast<8>(bsrc), row_bcast<9>(bsrc), row_bcast<10>(bsrc), row_bcast<11>(bsrc));
        bb[3] = make_float4(row_bcast<12>(bsrc), row_bcast<13>(bsrc), row_bcast<14>(bsrc), row_bcast<15>(bsrc));
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4_t R;
                R[0] = bb[a].x * (__uint_as_float(vr[h][a][0]) - X[h][a][0]);
                R[1] = bb[a].y * (__uint_as_float(vr[h][a][1]) - X[h][a][1]);
                R[2] = bb[a].z * (__uint_as_float(vr[h][a][2]) - X[h][a][2]);
                R[3] = bb[a].w * (__uint_as_float(vr[h][a][3]) - X[h][a][3]);
                Rb[h][a] = pack_bf16x4(R);  // lane: R[16a + 4g + r][col li of half h]
            }
    }

    // U by block forward substitution over the four token tiles,
    //   U_a = T_aa (R_a - sum_{m<a} L_am U_m),   L = the strictly lower A_kk blocks,
    // which equals (I + A_kk)^{-1} R tile by tile; then the outputs
    //   O_a = Q~_a S + sum_{m<=a} A_qk[a][m] U_m,
    // formed transposed (O^T = S^T Q~^T + U^T A_qk^T) so each lane holds four adjacent output
    // columns of one token, and stored.  Every 16x16x16 chain starts from zero and Y^T is added
    // on the VALU, so no accumulator passes from a 16x16x32 product to a 16x16x16 one.
    // Y^T = S^T Q~^T (S before this chunk's update)
    __device__ __forceinline__ void phaseY(const Stage& b) {
        const uint4* qt = b.blk + B::QT / 16;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int a = 0; a < 4; ++a) Yt[h][a] = zero;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 opd[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) opd[a] = qt[(a * KS + s) * 64 + lane];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const uint4 sb = packed_state(h, s);
#pragma unroll
                for (int a = 0; a < 4; ++a) Yt[h][a] = mfma32(sb, opd[a], Yt[h][a]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    __device__ __forceinline__ void phaseB(const Stage& b, char* obase, uint32_t rowV, int64_t t0, int n_valid) {
        const uint2* lb = reinterpret_cast<const uint2*>(b.blk + B::TB / 16);
        const uint2* ab = reinterpret_cast<const uint2*>(b.blk + B::MB / 16);
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        {
            uint2 lv[10];  // block (a, m), row li, columns 4g .. 4g + 3
#pragma unroll
            for (int t = 0; t < 10; ++t) lv[t] = lb[t * 64 + li * 4 + g];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    f32x4_t acc = zero;
#pragma unroll
                    for (int m = 0; m < a; ++m) acc = mfma16(lv[tri_index(a, m)], Ub[h][m], acc);
                    const uint2 rb = Rb[h][a];
                    const f32x4_t y = {lo_bf16(rb.x) - acc[0], hi_bf16(rb.x) - acc[1],
                                       lo_bf16(rb.y) - acc[2], hi_bf16(rb.y) - acc[3]};
                    Ub[h][a] = pack_bf16x4(mfma16(lv[tri_index(a, a)], pack_bf16x4(y), zero));
                }
        }
        __builtin_amdgcn_sched_barrier(0);
        uint2 av[10];
#pragma unroll
        for (int t = 0; t < 10; ++t) av[t] = ab[t * 64 + li * 4 + g];
        const rsrc_t ro = make_rsrc(obase + t0 * rowV, n_valid * rowV);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            f32x4_t Om[4] = {zero, zero, zero, zero};
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int a = m; a < 4; ++a) Om[a] = mfma16(Ub[h][m], av[tri_index(a, m)], Om[a]);
            const uint32_t voff = static_cast<uint32_t>(li) * rowV + static_cast<uint32_t>(col0 + 4 * g) * ES;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                // Ot[r] = O[16a + li][col0 + 16h + 4g + r]
                const f32x4_t Ot = Om[a] + Yt[h][a];
                const uint32_t soff = static_cast<uint32_t>(16 * a) * rowV + 16 * h * ES;
                if constexpr (sizeof(TIn) == 2) {
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2_t{pack_bf16x2(Ot[0], Ot[1]), pack_bf16x2(Ot[2], Ot[3])}, ro, voff, soff, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4_t{__float_as_uint(Ot[0]), __float_as_uint(Ot[1]), __float_as_uint(Ot[2]),
                                __float_as_uint(Ot[3])}, ro, voff, soff, 0);
                }
            }
        }
    }

    // S = diag(e^{Gamma_n}) S + K^n^T U
    __device__ __forceinline__ void phaseC(const Stage& b) {
        const uint4* kn = b.blk + B::KN / 16;
        const float* dnv = reinterpret_cast<const float*>(b.blk + B::DN / 16);
        // e^{Gamma_n} of state row 32 (j / 8) + 8 g + j % 8 for j = 4 m + r: lane li of a row
        // reads j = 2 li, 2 li + 1 (wrapped inside the DK rows), DPP broadcasts spread them
        const float2 dsrc = *reinterpret_cast<const float2*>(
            &dnv[32 * ((li >> 2) & (DK / 32 - 1)) + 8 * g + 2 * (li & 3)]);
        auto dj = [&](auto J) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
            return row_bcast<j / 2>((j & 1) ? dsrc.y : dsrc.x);
        };
        auto scale = [&](auto M) __attribute__((always_inline)) {
            constexpr int m = decltype(M)::value;
            const float d0 = dj(std::integral_constant<int, 4 * m>{});
            const float d1 = dj(std::integral_constant<int, 4 * m + 1>{});
            const float d2 = dj(std::integral_constant<int, 4 * m + 2>{});
            const float d3 = dj(std::integral_constant<int, 4 * m + 3>{});
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                S[h][m][0] *= d0;
                S[h][m][1] *= d1;
                S[h][m][2] *= d2;
                S[h][m][3] *= d3;
            }
        };
        scale(std::integral_constant<int, 0>{});
        scale(std::integral_constant<int, 1>{});
        scale(std::integral_constant<int, 2>{});
        scale(std::integral_constant<int, 3>{});
        if constexpr (MT > 4) {
            scale(std::integral_constant<int, 4>{});
            scale(std::integral_constant<int, 5>{});
            scale(std::integral_constant<int, 6>{});
            scale(std::integral_constant<int, 7>{});
        }
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4 kk = kn[(m * 2 + sp) * 64 + lane];
#pragma unroll
                for (int h = 0; h < NH; ++h)
                    S[h][m] = mfma32(kk, make_uint4(Ub[h][2 * sp].x, Ub[h][2 * sp].y, Ub[h][2 * sp + 1].x,
                                                    Ub[h][2 * sp + 1].y), S[h][m]);
            }
    }

    // The state to / from one (sequence, head)'s dk x dv matrix at `base` (row stride dv = DK),
    // this wave's columns.  Buffer accesses: one VGPR of lane offset, the row and half parts
    // in the scalar offset, so no per-element 64-bit addresses stay live in the chunk loop.
    __device__ __forceinline__ uint32_t state_voff() const {
        return static_cast<uint32_t>(8 * g * DK + col0 + li) * 4;
    }
    __device__ __forceinline__ static uint32_t state_soff(int h, int m, int r) {
        return static_cast<uint32_t>((32 * (m >> 1) + 4 * (m & 1) + r) * DK + 16 * h) * 4;
    }
    __device__ __forceinline__ void store_state(float* base) const {
        const rsrc_t rs = make_rsrc(base, DK * DK * 4);
        const uint32_t voff = state_voff();
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[h][m][r]), rs, voff,
                                                          state_soff(h, m, r), 0);
    }
    __device__ __forceinline__ void load_state(const float* base) {
        const rsrc_t rs = make_rsrc(base, base ? DK * DK * 4 : 0);  // no state: reads 0
        const uint32_t voff = state_voff();
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[h][m][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, state_soff(h, m, r), 0));
    }
};

// The fused path's barrier slots per chunk: producer phases 1, 2, 3, 4 (which writes K^n^T
// itself, so there is no phase 5) and 6 (with the diagonal solves); the consumers run A, B
// and C beside phases 2, 4 and 6
constexpr int kFusedPhases = 5;
constexpr int kSlotA = 2, kSlotB = 4, kSlotC = 5;
// The slot of phase Y (Y^T = S^T Q~^T): up to kSlotB it runs for the chunk in hand; from
// kSlotC on it runs for the next chunk (after phase C has updated S; that chunk's Q~ is
// complete after producer phase 4)
constexpr int kSlotY = 5;
static_assert(kSlotY <= kSlotB || (kSlotY >= kSlotC && kSlotY <= kFusedPhases), "phase Y slot");

template <int DK, typename TIn>
__global__ void __launch_bounds__(512) prefill_fused_kernel(SplitArgs args) {
    using Sm = FusedSmem<DK>;
    static_assert(sizeof(Sm) <= 160 * 1024, "fused prefill LDS budget");
    constexpr int ES = static_cast<int>(sizeof(TIn));
    __shared__ Sm sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> (chain rank, head), the head fastest; varlen chains run longest first
    const int H = args.H;
    if (static_cast<int>(blockIdx.x) >= args.npairs) return;
    const int rank = static_cast<int>(blockIdx.x) / H, h = static_cast<int>(blockIdx.x) - rank * H;
    const int n = args.cu ? args.chunk_start[rank] : rank;
    const int64_t tok0 = seq_start(args.cu, args.T, n);
    const int64_t len = (args.cu ? static_cast<int64_t>(args.cu[n + 1]) : tok0 + args.T) - tok0;
    const int nchunks = static_cast<int>((len + kC - 1) / kC);
    auto chunk_len = [&](int c) {
        const int64_t rem = len - static_cast<int64_t>(c) * kC;
        return rem < kC ? static_cast<int>(rem) : kC;
    };

    if (w < 4) {
        // ================================ producers ================================
        Producer<DK, TIn, true> pr;
        pr.init(tid);
        if (tid < DK) sm.p.ae[tid] = -expf(args.A[h * DK + tid]) * kLog2e;
        const float gscale = args.g_min * kLog2e;
        if (nchunks > 0) {
            pr.load(args, h, tok0, chunk_len(0));
            pr.unswap_z();
        }
        for (int c = 0; c <= nchunks; ++c) {
            // iteration c builds chunk c's block in stage c % 2 (the consumers read the other)
            const bool live = c < nchunks;
            typename Sm::Stage& st = sm.st[c & 1];
            char* blk = reinterpret_cast<char*>(st.blk);
            // the stage's 16x16 block areas: T_aa and L_am (a > m) in one, A_qk in the other
            bf16_t(*Tb)[16][16] = reinterpret_cast<bf16_t(*)[16][16]>(blk + Block<DK>::TB);
            bf16_t(*Ab)[16][16] = reinterpret_cast<bf16_t(*)[16][16]>(blk + Block<DK>::MB);
            if (live) pr.phase1(st.beta);
            lds_barrier();
            if (live) pr.phase2(sm.p, gscale);
            lds_barrier();
            if (live) pr.phase3(sm.p, blk);
            lds_barrier();
            if (live) pr.template phase4<true>(sm.p, blk);  // K^n^T straight into the stage
            lds_barrier();
            // chunk c's q, k, z registers are free: load chunk c + 1 into them
            if (c + 1 < nchunks) pr.load(args, h, tok0 + static_cast<int64_t>(c + 1) * kC, chunk_len(c + 1));
            if (live) pr.phase6_solve(sm.p, st.beta, Tb, Ab, Tb);
            if (c + 1 < nchunks) pr.unswap_z();
            lds_barrier();
        }
        return;
    }

    // ================================ consumers ================================
    Consumer<DK, TIn> cs;
    cs.lane = tid & 63;
    cs.g = cs.lane >> 4;
    cs.li = cs.lane & 15;
    cs.col0 = (w - 4) * (DK / 4);
    const int dv = DK;
    const uint32_t rowV = static_cast<uint32_t>(H) * dv * ES;
    const char* vbase = static_cast<const char*>(args.v) + (static_cast<size_t>(h) * dv) * ES;
    char* obase = static_cast<char*>(args.o) + (static_cast<size_t>(h) * dv) * ES;
    const size_t sbase = (static_cast<size_t>(n) * H + h) * DK * dv;
    cs.load_state(args.s0 ? args.s0 + sbase : nullptr);
    if (nchunks > 0) cs.load_v(vbase, rowV, tok0, chunk_len(0));
    for (int c = 0; c <= nchunks; ++c) {
        // iteration c runs the state pass over chunk c - 1 from stage (c - 1) % 2
        const int e = c - 1;
        const bool live = e >= 0;
        const typename Sm::Stage& st = sm.st[e & 1];
        const int64_t t0 = tok0 + static_cast<int64_t>(e) * kC;
        // one consumer phase beside producer phases kSlotA, kSlotB and kSlotC (1-based), as
        // many barriers per iteration as the producers
#pragma unroll
        for (int k = 1; k <= kFusedPhases; ++k) {
            if (live && k == kSlotA) cs.phaseA(st);
            if constexpr (kSlotY <= kSlotB) {
                if (live && k == kSlotY) cs.phaseY(st);
            }
            if (live && k == kSlotB) cs.phaseB(st, obase, rowV, t0, chunk_len(e));
            if (live && k == kSlotC) {
                cs.phaseC(st);
                if (c < nchunks) cs.load_v(vbase, rowV, tok0 + static_cast<int64_t>(c) * kC, chunk_len(c));
                // prefix-cache checkpoint: the state after every ckpt_chunks full chunks
                if (args.ckpt && (e + 1) % args.ckpt_chunks == 0 && static_cast<int64_t>(e + 1) * kC <= len) {
                    const int j = (e + 1) / args.ckpt_chunks - 1;
                    const int64_t first = args.ckpt_off ? args.ckpt_off[n] : static_cast<int64_t>(n) * args.ckpt_per_seq;
                    cs.store_state(args.ckpt + ((first + j) * H + h) * DK * dv);
                }
            }
            if constexpr (kSlotY >= kSlotC) {
                if (k == kSlotY && c < nchunks) cs.phaseY(sm.st[c & 1]);
            }
            lds_barrier();
        }
    }
    if (args.sN) cs.store_state(args.sN + sbase);
}

// ---- host side --------------------------------------------------------------------------

size_t split_block_bytes(int dk) { return dk == 128 ? Block<128>::BYTES : Block<64>::BYTES; }

int64_t split_max_chunks(int64_t total, int n_seqs) { return (total + kC - 1) / kC + n_seqs; }

size_t fused_workspace_bytes(int n_seqs) { return ((static_cast<size_t>(n_seqs) + 1) * 4 + 255) / 256 * 256; }

size_t split_workspace_bytes(int64_t total, int n_seqs, int H, int dk) {
    return fused_workspace_bytes(n_seqs) + static_cast<size_t>(split_max_chunks(total, n_seqs)) * H * split_block_bytes(dk);
}

// K1 then K2 (the lagged 16-column state pass, or NCW compute waves of 16 columns)
template <int DK, int NCW, typename TIn, bool LAG = false>
static hipError_t launch_split_t(const SplitArgs& a0, hipStream_t stream) {
    constexpr int NLW = 4;  // loader waves
    SplitArgs a = a0;
    if (a.cu) {
        hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, stream, a.cu, a.n_seqs, a.chunk_start);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t slots = a.cu ? split_max_chunks(a.total, a.n_seqs)
                               : static_cast<int64_t>(a.n_seqs) * ((a.T + kC - 1) / kC);
    if (slots > 0) {
        hipLaunchKernelGGL((prefill_intra_kernel<DK, TIn>), dim3(static_cast<unsigned>(slots * a.H)), dim3(256), 0,
                           stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    a.nslices = DK / (16 * NCW);
    const int groups = (a.npairs + 7) / 8;
    const dim3 grid(static_cast<unsigned>(groups) * 8u * a.nslices);
    if constexpr (LAG)
        hipLaunchKernelGGL((prefill_state_lagged_kernel<DK, NLW, TIn>), grid, dim3(64 * (2 + NLW)), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_state_kernel<DK, NCW, NLW, TIn>), grid, dim3(64 * (NCW + NLW)), 0, stream, a);
    return hipGetLastError();
}

// one fused workgroup of eight waves per (sequence, head); a varlen call first orders the
// sequences (into the workspace's table, which the fused kernel reads as chain order)
template <int DK, typename TIn>
static hipError_t launch_fused_t(const SplitArgs& a, hipStream_t stream) {
    if (a.cu) {
        hipLaunchKernelGGL(chain_order_kernel, dim3(1), dim3(1024), 0, stream, a.cu, a.n_seqs, a.chunk_start);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.npairs > 0)
        hipLaunchKernelGGL((prefill_fused_kernel<DK, TIn>), dim3(static_cast<unsigned>(a.npairs)), dim3(512), 0,
                           stream, a);
    return hipGetLastError();
}

template <int DK, typename TIn>
static hipError_t launch_split_d(const SplitArgs& a, int ncw, hipStream_t stream) {
    // the fused kernel exists for bf16 inputs only (fp32 operands need more registers)
    if constexpr (sizeof(TIn) == 2) {
        if (ncw == 0) return launch_fused_t<DK, TIn>(a, stream);
    } else {
        if (ncw == 0) return hipErrorInvalidValue;
    }
    // the lagged pass holds three Q~/M stages, which leave no LDS for fp32 v rows at d = 128
    if constexpr (DK == 64 || sizeof(TIn) == 2)
        if (ncw == 1) return launch_split_t<DK, 1, TIn, true>(a, stream);
    if (ncw == 1) return launch_split_t<DK, 1, TIn>(a, stream);
    if (ncw == 2) return launch_split_t<DK, 2, TIn>(a, stream);
    return launch_split_t<DK, 4, TIn>(a, stream);
}

hipError_t launch_prefill_split(const SplitArgs& a, int dk, bool bf16, int ncw, hipStream_t stream) {
    if (dk == 128) return bf16 ? launch_split_d<128, bf16_t>(a, ncw, stream) : launch_split_d<128, float>(a, ncw, stream);
    return bf16 ? launch_split_d<64, bf16_t>(a, ncw, stream) : launch_split_d<64, float>(a, ncw, stream);
}

}  // namespace kda
