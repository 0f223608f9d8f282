/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) forward pass.
 *
 * Sources, by page title and section:
 *   [K3 note]  "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
 *              (Awesome-LLM-Research-Collections note on the K3 technical report)
 *   [K3 hood]  "Kimi K3 Under the Hood: A 2.8T MoE Built for Million-Token Agents"
 *
 * The operator, per (sequence, head), with state S in R^{dk x dv} (rows = key channels):
 *   g_t = g_min * Sigmoid(e^{A} z_t),  alpha_t = e^{g_t},  g_min = -5      [K3 note] §3.3
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T  [K3 note] §3.1
 *   o_t = S_t^T q_t   (read after the update; no scale is applied to q)   [K3 note] §3.2
 * Prefill evaluates it chunk by chunk (64-token chunks of 16-token tiles); decode advances
 * the state by one token ([K3 note] §3.3, recurrent decoding and chunked prefill).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates or frees device memory and keeps no state between calls.  The one
 *     exception is the fixed scratch array of kda_prefill_fwd_noalloc, a static device
 *     variable that each device holds from the library's load until the process ends.
 *   - Layouts are row-major with the last dimension contiguous:
 *       q, k, z  [tokens, H, dk]      v, o  [tokens, H, dv]      beta  [tokens, H]
 *       A        [H, dk]              states [N, H, dk, dv] (dv fastest, rows = key channels)
 *     q, k, v, beta and o have the element type given by `dt`; z, A and all states are fp32.
 *   - Pointers must be 16-byte aligned, except beta (element-aligned) and cu_seqlens
 *     (4-byte aligned); KDA_ERR_ALIGN otherwise.  Pointers to per-token
 *     tensors (q, k, v, beta, z, g, gcum, o) may be NULL only when the call has no tokens
 *     (then nothing is read or written through them); otherwise NULL is KDA_ERR_NULL.
 *   - Work is enqueued on `stream` (NULL = the default stream); calls return before it
 *     finishes.  Argument checks run on the host before anything is enqueued; on an error
 *     nothing is launched and nothing is written.  Device-side faults surface at the
 *     caller's next synchronisation.  The contents of cu_seqlens are not validated (that
 *     would need a synchronisation): they must start at 0, be non-decreasing and end at
 *     the token count.  NaN/Inf inputs propagate.
 *   - Calls are thread-safe; calls that overlap on the same output memory race.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL                                 */
    KDA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or too big  */
    KDA_ERR_UNSUPPORTED = -3, /* head size, element type or g_min outside what is compiled  */
    KDA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                           */
    KDA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than kda_prefill_workspace_size */
    KDA_ERR_HIP = -6,         /* the HIP runtime rejected a launch                          */
    KDA_ERR_SCRATCH = -7      /* kda_prefill_fwd_noalloc: the call needs more than          */
                              /* KDA_NOALLOC_SCRATCH_BYTES of scratch                       */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0, /* q, k, v, beta, o are fp32 (contractions still run on bf16 MFMA)   */
    KDA_BF16 = 1 /* q, k, v, beta, o are bf16; o is rounded to nearest even           */
} kda_dtype;

/* Largest chunk length accepted by kda_gate. */
#define KDA_GATE_MAX_CHUNK 1024
/* widest ShortConv kda_short_conv supports */
#define KDA_SHORT_CONV_MAX_WIDTH 4
/* most draft tokens kda_decode_verify / kda_decode_commit take per call */
#define KDA_DECODE_MAX_DRAFT 16

/*
 * kda_gate -- lower-bounded decay gate and chunk-local cumulative log-decay.
 * [K3 note] §3.3 (lower-bounded decay; reciprocal cumulative decay in chunked prefill);
 * [K3 hood] "Sequence mixing" (the retention parameterisation).
 *
 *   g[t,h,c]    = g_min * Sigmoid(exp(A[h,c]) * z[t,h,c])          (fp32)
 *   gcum[t,h,c] = sum of g[t',h,c] over t' from the start of t's chunk up to t inclusive
 * Chunks are `chunk` tokens long and restart at every sequence start; a sequence's last
 * chunk may be shorter.
 *
 *   z, A        input, fp32 ([total_tokens, H, dk], [H, dk])
 *   g, gcum     outputs, fp32 [total_tokens, H, dk]; either may be NULL, not both
 *   cu_seqlens  device int32 [n_seqs + 1] sequence starts, or NULL for n_seqs sequences of
 *               total_tokens / n_seqs tokens each (then total_tokens % n_seqs must be 0)
 *   chunk       1 .. KDA_GATE_MAX_CHUNK (the prefill uses 64)
 *   g_min       finite and < 0 (the pages fix -5)
 *   dk          a multiple of 4; total_tokens >= 0; H >= 1; n_seqs >= 1
 * KDA_ERR_SHAPE also when ceil(total_tokens / chunk) * ceil(H * dk / 1024) exceeds 2^24 - 1
 * (one 256-thread workgroup per window of chunk tokens and 1024 channels).
 */
kda_status kda_gate(const float* z, const float* A, float* g, float* gcum,
                    int64_t total_tokens, int H, int dk, const int32_t* cu_seqlens,
                    int n_seqs, int chunk, float g_min, hipStream_t stream);

/*
 * kda_prefill_workspace_size -- bytes of device workspace kda_prefill_fwd needs for this
 * problem on the current device (a multiple of 256).  With bf16 inputs and at least one
 * (sequence, head) chain per compute unit of the current device, the prefill is one fused
 * kernel that keeps each chunk's factors on chip: the workspace then holds only a table of
 * n_seqs + 1 int32 (the varlen chain order), 256 bytes per 64 sequences.  Otherwise the
 * prefill runs in two kernels: the first computes every (chunk, head)'s intra-chunk factors
 * in parallel into the workspace (58.5 KiB per chunk and head at d = 128, 34.25 KiB at d = 64,
 * for at most ceil(total/64) + n_seqs chunks, after the same table); the second runs the
 * serial inter-chunk state pass over them.  The form follows the device current at the
 * call, so query with the device current that the prefill will run on (a size taken for a
 * device with more compute units may be too small: KDA_ERR_WORKSPACE).  Returns 0 for
 * invalid sizes; the prefill call reports those.
 */
size_t kda_prefill_workspace_size(int64_t total_tokens, int n_seqs, int H, int dk, int dv,
                                  kda_dtype dt);

/*
 * kda_prefill_fwd -- chunkwise KDA prefill over a packed batch.
 * [K3 note] §3.3 (chunked prefill: (X_[c], S_in) -> (Y_[c], S_out), S_in[c+1] = S_out[c];
 * 16-token tiles whose cumulative log-decay stays in (-80, 0) so every tile, diagonal or
 * not, is a dense bf16 matrix product); §3.1-§3.2 (the recurrence it evaluates);
 * [K3 hood] "Serving two incompatible cache types" (a prefix hit restores the state at
 * the hit boundary and resumes prefill from it; cached checkpoints are read-only).
 *
 *   dt             element type of q, k, v, beta and o
 *   q, k           [total, H, dk];  v [total, H, dv];  beta [total, H]
 *   z, A           decay logits [total, H, dk] and per-(head, channel) A [H, dk], fp32;
 *                  the gate above is applied inside the kernel
 *   g_min          in [-5, 0): the 16-token bound needs g >= -5 (KDA_ERR_UNSUPPORTED else)
 *   initial_state  fp32 [N, H, dk, dv], read only, or NULL for zero states
 *   final_state    fp32 [N, H, dk, dv] written with each sequence's last state, or NULL;
 *                  may alias initial_state only as the very same pointer
 *   cu_seqlens     device int32 [N + 1], or NULL for N sequences of T_or_total tokens each
 *   n_seqs         N >= 1
 *   T_or_total     tokens per sequence when cu_seqlens is NULL, else the packed total
 *   dk, dv         64 or 128 each, dk == dv
 *   o              [total, H, dv] output of type dt
 *   workspace      device scratch of at least kda_prefill_workspace_size(...) bytes,
 *                  16-byte aligned (KDA_ERR_WORKSPACE otherwise); may be NULL only when
 *                  there is nothing to compute; contents on return are undefined
 * Size limits (KDA_ERR_SHAPE beyond them): H <= 65535; 64 token rows of one head's z span
 * less than 2^31 bytes (H * dk * 256 < 2^31); (ceil(total / 64) + N) * H <= 2^31 - 1, one
 * intra-chunk workgroup per (chunk, head).
 * A zero-length sequence writes no output rows and copies its initial state (or zeros) to
 * final_state.  Results equal the token recurrence up to floating-point association.
 */
kda_status kda_prefill_fwd(kda_dtype dt, const void* q, const void* k, const void* v,
                           const void* beta, const float* z, const float* A, float g_min,
                           const float* initial_state, float* final_state,
                           const int32_t* cu_seqlens, int n_seqs, int64_t T_or_total, int H,
                           int dk, int dv, void* o, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * kda_prefill_fwd_noalloc -- kda_prefill_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, with the workspace taken from a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES per device instead of a caller buffer.
 *
 * All arguments of kda_prefill_fwd keep their meaning; there is no workspace argument.
 *   - The call is accepted only when kda_prefill_workspace_size(...) of the same sizes is at
 *     most KDA_NOALLOC_SCRATCH_BYTES (64 MiB).  In the two-kernel form that is about 1,100
 *     (chunk, head) pairs at d = 128 (e.g. 4096 tokens x 16 heads); the fused form (bf16,
 *     a chain per compute unit) needs only the chain-order table, so any bf16 batch with
 *     that many chains fits.  KDA_ERR_SCRATCH otherwise, checked on the host before
 *     anything else happens.
 *   - The array's device address is looked up once per device (hipGetSymbolAddress, on the
 *     first call with that device current); a failed lookup returns KDA_ERR_HIP.  The call
 *     itself allocates nothing (no hipMalloc, no library allocation).
 *   - Every call on a device shares that device's array and leaves its contents undefined:
 *     calls that overlap in time on one device (several streams, several host threads)
 *     race on it and must be ordered by the caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_prefill_fwd_noalloc(kda_dtype dt, const void* q, const void* k, const void* v,
                                   const void* beta, const float* z, const float* A,
                                   float g_min, const float* initial_state, float* final_state,
                                   const int32_t* cu_seqlens, int n_seqs, int64_t T_or_total,
                                   int H, int dk, int dv, void* o, hipStream_t stream);

/*
 * kda_prefill_fwd_checkpointed -- kda_prefill_fwd that also writes prefix-cache checkpoints:
 * the recurrent state at every checkpoint_interval tokens of each sequence.
 * [K3 note] §9 (KDA keeps one large state per sequence, so checkpoints are affordable only
 * at sparse, 512-token hash boundaries; a prefix hit restores the state at the boundary and
 * resumes prefill); [K3 hood] "Serving two incompatible cache types" (checkpoints at
 * selected hash boundaries, copied read-only into the request's running state).
 *
 * All arguments of kda_prefill_fwd keep their meaning, plus:
 *   checkpoint_interval  tokens between checkpoints, a positive multiple of 64
 *                        (KDA_ERR_SHAPE otherwise)
 *   checkpoints          fp32 [n_ckpt, H, dk, dv], 16-byte aligned (NULL: KDA_ERR_NULL).
 *                        Checkpoint j (0-based) of sequence n is the state after its first
 *                        (j + 1) * checkpoint_interval tokens, initial_state included, for
 *                        j < floor(L_n / checkpoint_interval).  It is stored at index
 *                        first_n + j, where first_n = n * floor(T / checkpoint_interval) for
 *                        equal-length batches, else checkpoint_offsets[n].
 *   checkpoint_offsets   device int32 [N + 1]: required (KDA_ERR_NULL) with cu_seqlens, ignored
 *                        without; the exclusive prefix sum of floor(L_n / checkpoint_interval),
 *                        which the caller computes from the lengths it packed.  Its contents
 *                        are not validated.
 * A checkpoint that falls on a sequence's last token equals that sequence's final state.
 * Resuming kda_prefill_fwd from checkpoint j (as initial_state) over the remaining tokens
 * reproduces the original outputs of those tokens exactly (same chunk boundaries).
 */
kda_status kda_prefill_fwd_checkpointed(kda_dtype dt, const void* q, const void* k,
                                        const void* v, const void* beta, const float* z,
                                        const float* A, float g_min, const float* initial_state,
                                        float* final_state, const int32_t* cu_seqlens,
                                        int n_seqs, int64_t T_or_total, int H, int dk, int dv,
                                        void* o, float* checkpoints,
                                        const int32_t* checkpoint_offsets,
                                        int checkpoint_interval, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/*
 * kda_decode_step -- one recurrent decode step for N sequences x H heads, state in place.
 * [K3 note] §3.2 (the per-token map (x_t, S_{t-1}) -> (y_t, S_t) and its order: decay
 * Sbar = Diag(alpha) S, predict vhat = Sbar^T k, write S = Sbar + beta k (v - vhat)^T,
 * read o = S^T q after the write); §3.3 (recurrent decoding, one token at a time).
 *
 *   q, k, z        [N, H, dk] (one token per sequence);  v [N, H, dv];  beta [N, H]
 *   A              [H, dk] fp32;  g_min finite and < 0
 *   state          fp32 [N, H, dk, dv], read and overwritten with S_t
 *   o              [N, H, dv] output of type dt
 *   dk, dv         64 or 128 each, dk == dv
 */
kda_status kda_decode_step(kda_dtype dt, const void* q, const void* k, const void* v,
                           const void* beta, const float* z, const float* A, float g_min,
                           float* state, int N, int H, int dk, int dv, void* o,
                           hipStream_t stream);

/*
 * kda_decode_verify -- outputs of K draft tokens per sequence from the committed state,
 * which is only read.  [K3 hood] "Serving two incompatible cache types" (rejected draft
 * tokens must not advance the recurrent state; the small projected inputs are kept and the
 * accepted ones replayed on chip); [K3 note] §3.2 (each token's output is read after its
 * own write).  o[n, t] equals what t + 1 consecutive kda_decode_step calls on draft tokens
 * 0..t would return for token t; the state is read once for all K tokens.
 *
 *   q, k, z        [N, K, H, dk];  v [N, K, H, dv];  beta [N, K, H];  A [H, dk] fp32
 *   state          fp32 [N, H, dk, dv], read only
 *   K              1 .. KDA_DECODE_MAX_DRAFT draft tokens per sequence (KDA_ERR_SHAPE else)
 *   o              [N, K, H, dv] output of type dt
 *   dk, dv         64 or 128 each, dk == dv
 */
kda_status kda_decode_verify(kda_dtype dt, const void* q, const void* k, const void* v,
                             const void* beta, const float* z, const float* A, float g_min,
                             const float* state, int N, int K, int H, int dk, int dv, void* o,
                             hipStream_t stream);

/*
 * kda_decode_commit -- advance each sequence's state in place by its accepted draft tokens:
 * replays the first accepted[n] of the K tokens given to kda_decode_verify (same k, v, beta,
 * z; q is not needed), reading and writing the state once.  Same sources as above.
 *
 *   accepted       device int32 [N]; values are clamped to [0, K]; 0 leaves the state as is
 *   other arguments as for kda_decode_verify; state fp32 [N, H, dk, dv] read and written
 * The result equals accepted[n] consecutive kda_decode_step calls.
 */
kda_status kda_decode_commit(kda_dtype dt, const void* k, const void* v, const void* beta,
                             const float* z, const float* A, float g_min, float* state, int N,
                             int K, int H, int dk, int dv, const int32_t* accepted,
                             hipStream_t stream);

/*
 * kda_output_gate -- fused output epilogue y = Sigmoid(gate) * RMSNorm(o), per row.
 * [K3 note] §3.2 (the K3 output path W_o[Sigmoid(W_g x_t) (.) RMSNorm(o~_t)]; the projections
 * need trained weights, so this entry takes the readout o~ and the gate logits W_g x_t).
 * RMSNorm(o) = o / sqrt(mean(o^2) + eps) * weight, over the d_v channels of one row.
 *
 *   dt        element type of o, gate and y
 *   o, gate   [rows, dv] (a row is one token of one head, e.g. rows = tokens * H)
 *   weight    fp32 [dv];  eps finite and >= 0
 *   y         [rows, dv] output of type dt; may be o itself (in place)
 *   dv        64 or 128
 */
kda_status kda_output_gate(kda_dtype dt, const void* o, const void* gate, const float* weight,
                           float eps, int64_t rows, int dv, void* y, hipStream_t stream);

/*
 * kda_short_conv -- KDA input prologue: y = Swish(ShortConv(x)), then L2Norm per head when
 * l2_group > 0 (the q and k branches; 0 for v).  [K3 note] §3.2 (q, k = L2Norm(Swish(
 * ShortConv(W x))), v = Swish(ShortConv(W_v x)); during decoding ShortConv also reads and
 * updates the layer's short-convolution cache C^conv).  The projections need trained
 * weights, so x is the projected input.  ShortConv is a causal depthwise convolution over
 * the tokens of each sequence: y_t[c] = sum_i weight[c][i] * x_{t-width+1+i}[c] (the last tap
 * on the current token); Swish(u) = u Sigmoid(u); L2Norm divides each group of l2_group
 * channels by sqrt(sum u^2 + 1e-6).  A decode step is a call with one token per sequence.
 *
 *   dt          element type of x and y
 *   x           [total, C] packed tokens (C = heads x head dim, a multiple of 8)
 *   weight      fp32 [C, width], width 1 .. KDA_SHORT_CONV_MAX_WIDTH
 *   cache_in    fp32 [N, C, width-1] or NULL (zeros): the width-1 inputs that precede each
 *               sequence, oldest first
 *   cache_out   fp32 [N, C, width-1] or NULL: receives the last width-1 inputs of each
 *               sequence (reaching into cache_in for shorter sequences); may be cache_in
 *   cu_seqlens  device int32 [N + 1], or NULL for N sequences of T_or_total tokens
 *   l2_group    0, 64 or 128 (C a multiple of it)
 *   y           [total, C] of type dt; must not be x
 * KDA_ERR_SHAPE also when ceil(total / 64) * ceil(C / 2048) exceeds 2^24 - 1 (one 256-thread
 * workgroup per 64-token segment and 2048 channels).
 */
kda_status kda_short_conv(kda_dtype dt, const void* x, const float* weight, int width,
                          const float* cache_in, float* cache_out, const int32_t* cu_seqlens,
                          int n_seqs, int64_t T_or_total, int C, int l2_group, void* y,
                          hipStream_t stream);

/* kda_status_str -- a static, human-readable name for a status code. */
const char* kda_status_str(kda_status status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
