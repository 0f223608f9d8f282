// kda_api.cpp -- the C ABI declared in include/kda.h: argument checks, then kernel launch.
//
// Every check runs on the host before any HIP call, so an invalid call launches nothing
// and writes nothing.  The library allocates nothing and keeps no state between calls
// except a per-device cache of the compute-unit count used to size launches and, for
// kda_prefill_fwd_noalloc, the per-device address of its static scratch array.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "kda_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// beta is read one element at a time: element alignment suffices.
bool beta_aligned(const void* p, kda_dtype dt) {
    return (reinterpret_cast<uintptr_t>(p) & (dt == KDA_BF16 ? 1u : 3u)) == 0;
}

bool supported_d(int dk, int dv) { return dk == dv && (dk == 64 || dk == 128); }

constexpr int64_t kMaxElems = int64_t(1) << 46;  // far beyond any device memory

// CU count of the calling thread's current device, queried once per device.  Atomic entries:
// calls from several host threads may fill the same entry at once (with the same value).
int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// The prefill's form for np (sequence, head) chains on the current device: 0 for the fused
// kernel, else the state pass's compute waves per workgroup (1, 2 or 4).
int prefill_form(kda_dtype dt, int64_t np, int dk) {
    const int cus = compute_units();
    // With a chain for every compute unit, one fused workgroup per (sequence, head) keeps the
    // factor blocks on chip (bf16 inputs; the fp32 form needs more registers than it has).
    if (dt == KDA_BF16 && np >= cus) return 0;
    // Each state-pass workgroup copies the whole factor block of every chunk, so narrow dv
    // slices cost block re-reads (from L2: the slices of one head run on one XCD) but shorten
    // the per-chunk critical path.  Halve the compute waves per workgroup (64 columns at
    // most) while the chains still fit the compute units.
    int ncw = 4;
    while (ncw > 1 && np * (dk / (8 * ncw)) <= cus) ncw /= 2;
    return ncw;
}

}  // namespace

extern "C" {

const char* kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: invalid or inconsistent size";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head size, dtype or g_min not supported";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: pointer not 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed";
        case KDA_ERR_SCRATCH:
            return "KDA_ERR_SCRATCH: the call needs more than KDA_NOALLOC_SCRATCH_BYTES of scratch";
    }
    return "unknown kda_status";
}

kda_status kda_gate(const float* z, const float* A, float* g, float* gcum, int64_t total_tokens,
                    int H, int dk, const int32_t* cu_seqlens, int n_seqs, int chunk, float g_min,
                    hipStream_t stream) {
    if (total_tokens < 0 || H <= 0 || dk <= 0 || n_seqs <= 0) return KDA_ERR_SHAPE;
    if (!A || (total_tokens > 0 && (!z || (!g && !gcum)))) return KDA_ERR_NULL;
    if (dk % 4 != 0) return KDA_ERR_UNSUPPORTED;
    if (chunk < 1 || chunk > KDA_GATE_MAX_CHUNK) return KDA_ERR_SHAPE;
    if (!std::isfinite(g_min) || !(g_min < 0.f)) return KDA_ERR_UNSUPPORTED;
    if (!cu_seqlens && total_tokens % n_seqs != 0) return KDA_ERR_SHAPE;
    if (total_tokens > kMaxElems / (static_cast<int64_t>(H) * dk)) return KDA_ERR_SHAPE;
    if (static_cast<int64_t>(H) * dk / 4 > int64_t(65535) * 256) return KDA_ERR_SHAPE;
    if ((total_tokens + chunk - 1) / chunk > int64_t(0x7fffffff)) return KDA_ERR_SHAPE;
    // one workgroup of 256 threads per (token window, 1024-channel block) in a 1-D grid
    if ((total_tokens + chunk - 1) / chunk * ((static_cast<int64_t>(H) * dk / 4 + 255) / 256) >
        int64_t(0xffffffff) / 256)
        return KDA_ERR_SHAPE;
    if (!aligned16(z) || !aligned16(A) || (g && !aligned16(g)) || (gcum && !aligned16(gcum)) ||
        (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)))
        return KDA_ERR_ALIGN;
    if (total_tokens == 0) return KDA_OK;
    kda::GateArgs a{};
    a.z = z; a.A = A; a.g = g; a.gcum = gcum; a.total = total_tokens; a.H = H; a.dk = dk;
    a.cu = cu_seqlens; a.n_seqs = n_seqs;
    a.T = cu_seqlens ? 0 : total_tokens / n_seqs;
    a.chunk = chunk; a.g_min = g_min;
    return kda::launch_gate(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_prefill_workspace_size(int64_t total_tokens, int n_seqs, int H, int dk, int dv,
                                  kda_dtype dt) {
    if (total_tokens < 0 || n_seqs <= 0 || H <= 0 || !supported_d(dk, dv)) return 0;
    if (total_tokens > kMaxElems / (static_cast<int64_t>(H) * dk)) return 0;
    // the fused kernel keeps its factors in LDS and needs only the sequence-order table
    if (prefill_form(dt, static_cast<int64_t>(n_seqs) * H, dk) == 0) return kda::fused_workspace_bytes(n_seqs);
    return kda::split_workspace_bytes(total_tokens, n_seqs, H, dk);
}

namespace {

struct Checkpoints {
    float* states;           // NULL: none
    const int32_t* offsets;  // varlen: first checkpoint of each sequence
    int interval;            // tokens, a positive multiple of 64
};

// Where the workspace comes from: the caller's buffer, or the device's static scratch array
// (kda_prefill_fwd_noalloc).
enum class WorkspaceSource { kCaller, kStaticScratch };

kda_status prefill_impl(kda_dtype dt, const void* q, const void* k, const void* v,
                        const void* beta, const float* z, const float* A, float g_min,
                        const float* initial_state, float* final_state,
                        const int32_t* cu_seqlens, int n_seqs, int64_t T_or_total, int H,
                        int dk, int dv, void* o, const Checkpoints& ck, void* workspace,
                        size_t workspace_bytes, hipStream_t stream,
                        WorkspaceSource wsrc = WorkspaceSource::kCaller) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (n_seqs <= 0 || T_or_total < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    const int64_t total = cu_seqlens ? T_or_total : static_cast<int64_t>(n_seqs) * T_or_total;
    // per-token tensors may be NULL only when there are no tokens
    if (!A || (total > 0 && (!q || !k || !v || !beta || !z || !o))) return KDA_ERR_NULL;
    if (!supported_d(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(g_min) || g_min < -5.f || !(g_min < 0.f)) return KDA_ERR_UNSUPPORTED;
    if (!cu_seqlens && n_seqs > 0 && T_or_total > kMaxElems / n_seqs) return KDA_ERR_SHAPE;
    if (total > kMaxElems / (static_cast<int64_t>(H) * dk)) return KDA_ERR_SHAPE;
    if (static_cast<int64_t>(n_seqs) * H > int64_t(0x7fffffff) / 16 || H > 65535) return KDA_ERR_SHAPE;
    // one intra-chunk workgroup per (chunk slot, head) in a 1-D grid
    if (kda::split_max_chunks(total, n_seqs) > int64_t(0x7fffffff) / H) return KDA_ERR_SHAPE;
    // 64 token rows of one chunk must span < 2^31 bytes (32-bit buffer offsets)
    if (static_cast<int64_t>(H) * dk * 4 * 64 >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !beta_aligned(beta, dt) ||
        !aligned16(z) || !aligned16(A) || !aligned16(o) || (initial_state && !aligned16(initial_state)) ||
        (final_state && !aligned16(final_state)) ||
        (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)))
        return KDA_ERR_ALIGN;
    if (initial_state && final_state && initial_state != final_state) {
        const uintptr_t bytes = static_cast<uintptr_t>(n_seqs) * H * dk * dv * sizeof(float);
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(initial_state);
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(final_state);
        if (a0 < b0 + bytes && b0 < a0 + bytes) return KDA_ERR_SHAPE;  // partial overlap
    }
    if (ck.states) {
        if (ck.interval <= 0 || ck.interval % 64 != 0) return KDA_ERR_SHAPE;
        if (cu_seqlens && !ck.offsets) return KDA_ERR_NULL;
        if (!aligned16(ck.states) || (ck.offsets && (reinterpret_cast<uintptr_t>(ck.offsets) & 3u)))
            return KDA_ERR_ALIGN;
    }
    const size_t need = kda_prefill_workspace_size(total, n_seqs, H, dk, dv, dt);
    if (wsrc == WorkspaceSource::kStaticScratch && need > KDA_NOALLOC_SCRATCH_BYTES)
        return KDA_ERR_SCRATCH;
    if (total == 0 && !final_state) return KDA_OK;  // nothing to compute or write
    if (wsrc == WorkspaceSource::kStaticScratch) {
        if (kda::noalloc_scratch(&workspace) != hipSuccess) return KDA_ERR_HIP;
        workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KDA_ERR_WORKSPACE;

    kda::SplitArgs a{};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.z = z; a.A = A; a.g_min = g_min;
    a.s0 = initial_state; a.sN = final_state; a.cu = cu_seqlens; a.n_seqs = n_seqs;
    a.T = cu_seqlens ? 0 : T_or_total; a.H = H; a.o = o; a.npairs = n_seqs * H;
    a.total = total;
    if (ck.states) {
        a.ckpt = ck.states;
        a.ckpt_off = cu_seqlens ? ck.offsets : nullptr;
        a.ckpt_chunks = ck.interval / 64;
        a.ckpt_per_seq = cu_seqlens ? 0 : static_cast<int>(T_or_total / ck.interval);
    }
    // the form the workspace was sized for (kda_prefill_workspace_size); the fused form has
    // no factor blocks in memory
    const int ncw = prefill_form(dt, a.npairs, dk);
    a.chunk_start = static_cast<int32_t*>(workspace);
    a.blocks = ncw == 0 ? nullptr : static_cast<char*>(workspace) + kda::fused_workspace_bytes(n_seqs);
    return kda::launch_prefill_split(a, dk, dt == KDA_BF16, ncw, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

kda_status kda_prefill_fwd(kda_dtype dt, const void* q, const void* k, const void* v,
                           const void* beta, const float* z, const float* A, float g_min,
                           const float* initial_state, float* final_state,
                           const int32_t* cu_seqlens, int n_seqs, int64_t T_or_total, int H,
                           int dk, int dv, void* o, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    return prefill_impl(dt, q, k, v, beta, z, A, g_min, initial_state, final_state, cu_seqlens,
                        n_seqs, T_or_total, H, dk, dv, o, Checkpoints{nullptr, nullptr, 0},
                        workspace, workspace_bytes, stream);
}

kda_status kda_prefill_fwd_noalloc(kda_dtype dt, const void* q, const void* k, const void* v,
                                   const void* beta, const float* z, const float* A,
                                   float g_min, const float* initial_state, float* final_state,
                                   const int32_t* cu_seqlens, int n_seqs, int64_t T_or_total,
                                   int H, int dk, int dv, void* o, hipStream_t stream) {
    return prefill_impl(dt, q, k, v, beta, z, A, g_min, initial_state, final_state, cu_seqlens,
                        n_seqs, T_or_total, H, dk, dv, o, Checkpoints{nullptr, nullptr, 0},
                        nullptr, 0, stream, WorkspaceSource::kStaticScratch);
}

kda_status kda_prefill_fwd_checkpointed(kda_dtype dt, const void* q, const void* k,
                                        const void* v, const void* beta, const float* z,
                                        const float* A, float g_min, const float* initial_state,
                                        float* final_state, const int32_t* cu_seqlens,
                                        int n_seqs, int64_t T_or_total, int H, int dk, int dv,
                                        void* o, float* checkpoints,
                                        const int32_t* checkpoint_offsets,
                                        int checkpoint_interval, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    if (!checkpoints) return KDA_ERR_NULL;
    return prefill_impl(dt, q, k, v, beta, z, A, g_min, initial_state, final_state, cu_seqlens,
                        n_seqs, T_or_total, H, dk, dv, o,
                        Checkpoints{checkpoints, checkpoint_offsets, checkpoint_interval},
                        workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(kda_dtype dt, const void* q, const void* k, const void* v,
                           const void* beta, const float* z, const float* A, float g_min,
                           float* state, int N, int H, int dk, int dv, void* o,
                           hipStream_t stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (N > 0 && (!q || !k || !v || !beta || !z || !A || !state || !o)) return KDA_ERR_NULL;
    if (!supported_d(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(g_min) || !(g_min < 0.f)) return KDA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(N) * H > int64_t(0x7fffffff)) return KDA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !beta_aligned(beta, dt) ||
        !aligned16(z) || !aligned16(A) || !aligned16(state) || !aligned16(o))
        return KDA_ERR_ALIGN;
    if (N == 0) return KDA_OK;
    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.z = z; a.A = A; a.g_min = g_min;
    a.state = state; a.N = N; a.H = H; a.o = o;
    return kda::launch_decode(a, dk, dt == KDA_BF16, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_verify(kda_dtype dt, const void* q, const void* k, const void* v,
                             const void* beta, const float* z, const float* A, float g_min,
                             const float* state, int N, int K, int H, int dk, int dv, void* o,
                             hipStream_t stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || K < 1 || K > KDA_DECODE_MAX_DRAFT) return KDA_ERR_SHAPE;
    if (N > 0 && (!q || !k || !v || !beta || !z || !A || !state || !o)) return KDA_ERR_NULL;
    if (!supported_d(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(g_min) || !(g_min < 0.f)) return KDA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(N) * H > int64_t(0x7fffffff)) return KDA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !beta_aligned(beta, dt) ||
        !aligned16(z) || !aligned16(A) || !aligned16(state) || !aligned16(o))
        return KDA_ERR_ALIGN;
    if (N == 0) return KDA_OK;
    kda::DecodeMultiArgs a{};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.z = z; a.A = A; a.g_min = g_min;
    a.state_in = state; a.N = N; a.K = K; a.H = H; a.o = o;
    return kda::launch_decode_multi(a, dk, dt == KDA_BF16, false, stream) == hipSuccess ? KDA_OK
                                                                                          : KDA_ERR_HIP;
}

kda_status kda_decode_commit(kda_dtype dt, const void* k, const void* v, const void* beta,
                             const float* z, const float* A, float g_min, float* state, int N,
                             int K, int H, int dk, int dv, const int32_t* accepted,
                             hipStream_t stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || K < 1 || K > KDA_DECODE_MAX_DRAFT) return KDA_ERR_SHAPE;
    if (N > 0 && (!k || !v || !beta || !z || !A || !state || !accepted)) return KDA_ERR_NULL;
    if (!supported_d(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(g_min) || !(g_min < 0.f)) return KDA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(N) * H > int64_t(0x7fffffff)) return KDA_ERR_SHAPE;
    if (!aligned16(k) || !aligned16(v) || !beta_aligned(beta, dt) || !aligned16(z) ||
        !aligned16(A) || !aligned16(state) || (reinterpret_cast<uintptr_t>(accepted) & 3u))
        return KDA_ERR_ALIGN;
    if (N == 0) return KDA_OK;
    kda::DecodeMultiArgs a{};
    a.k = k; a.v = v; a.beta = beta; a.z = z; a.A = A; a.g_min = g_min;
    a.state = state; a.accepted = accepted; a.N = N; a.K = K; a.H = H;
    return kda::launch_decode_multi(a, dk, dt == KDA_BF16, true, stream) == hipSuccess ? KDA_OK
                                                                                         : KDA_ERR_HIP;
}

kda_status kda_output_gate(kda_dtype dt, const void* o, const void* gate, const float* weight,
                           float eps, int64_t rows, int dv, void* y, hipStream_t stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (rows < 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (dv != 64 && dv != 128) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(eps) || eps < 0.f) return KDA_ERR_UNSUPPORTED;
    if (!weight || (rows > 0 && (!o || !gate || !y))) return KDA_ERR_NULL;
    if (rows > kMaxElems / dv) return KDA_ERR_SHAPE;
    if (!aligned16(o) || !aligned16(gate) || !aligned16(weight) || !aligned16(y)) return KDA_ERR_ALIGN;
    if (rows == 0) return KDA_OK;
    kda::OutputGateArgs a{};
    a.o = o; a.gate = gate; a.w = weight; a.eps = eps; a.rows = rows; a.y = y;
    return kda::launch_output_gate(a, dv, dt == KDA_BF16, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_short_conv(kda_dtype dt, const void* x, const float* weight, int width,
                          const float* cache_in, float* cache_out, const int32_t* cu_seqlens,
                          int n_seqs, int64_t T_or_total, int C, int l2_group, void* y,
                          hipStream_t stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (n_seqs <= 0 || T_or_total < 0 || C <= 0) return KDA_ERR_SHAPE;
    if (width < 1 || width > KDA_SHORT_CONV_MAX_WIDTH) return KDA_ERR_UNSUPPORTED;
    if (C % 8 != 0 || (l2_group != 0 && l2_group != 64 && l2_group != 128) ||
        (l2_group && C % l2_group != 0))
        return KDA_ERR_UNSUPPORTED;
    if (C > 65535 * 2048) return KDA_ERR_SHAPE;
    if (!cu_seqlens && T_or_total > kMaxElems / n_seqs) return KDA_ERR_SHAPE;
    const int64_t total = cu_seqlens ? T_or_total : static_cast<int64_t>(n_seqs) * T_or_total;
    if (total > kMaxElems / C) return KDA_ERR_SHAPE;
    // one workgroup of 256 threads per (64-token segment, 2048-channel block) in a 1-D grid
    if ((total + 63) / 64 * ((C + 2047) / 2048) > int64_t(0xffffffff) / 256) return KDA_ERR_SHAPE;
    if (!weight || (total > 0 && (!x || !y))) return KDA_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || (reinterpret_cast<uintptr_t>(weight) & 3u) ||
        (reinterpret_cast<uintptr_t>(cache_in) & 3u) || (reinterpret_cast<uintptr_t>(cache_out) & 3u) ||
        (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)))
        return KDA_ERR_ALIGN;
    if (total > 0 && x == y) return KDA_ERR_SHAPE;  // the window reads earlier rows of x
    kda::ShortConvArgs a{};
    a.x = x; a.w = weight; a.W = width; a.cache_in = width > 1 ? cache_in : nullptr;
    a.cache_out = width > 1 ? cache_out : nullptr; a.cu = cu_seqlens; a.n_seqs = n_seqs;
    a.T = cu_seqlens ? 0 : T_or_total; a.total = total; a.C = C; a.l2 = l2_group; a.y = y;
    if (total == 0 && !a.cache_out) return KDA_OK;
    return kda::launch_short_conv(a, dt == KDA_BF16, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
