// kda_launch.h -- internal launch interface between the C ABI (kda_api.cpp) and the kernels.
// Arguments here have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct GateArgs {
    const float* z;
    const float* A;
    float* g;        // nullable
    float* gcum;     // nullable
    int64_t total;
    int H, dk;
    const int32_t* cu;  // nullable => n_seqs sequences of T tokens
    int n_seqs;
    int64_t T;
    int chunk;
    float g_min;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const float* z;
    const float* A;
    float g_min;
    const float* s0;    // nullable
    float* sN;          // nullable
    const int32_t* cu;  // nullable => N sequences of T tokens
    int n_seqs;
    int64_t T;
    int H;
    void* o;
    int npairs;         // n_seqs * H
    int nslices;        // set by the launcher
};

// Two-kernel prefill (intra-chunk factors, then the serial state pass) over a workspace
// holding the varlen chunk table and one factor block per (chunk, head).
struct SplitArgs : PrefillArgs {
    int64_t total;           // packed token count
    int32_t* chunk_start;    // [n_seqs + 1] in the workspace (varlen only); the fused kernel
                             // keeps its chain order there instead
    void* blocks;            // factor blocks in the workspace
    float* ckpt;             // nullable: states at every ckpt_chunks-th chunk boundary
    const int32_t* ckpt_off; // [n_seqs + 1] first checkpoint of each sequence (varlen)
    int ckpt_chunks;         // checkpoint interval in chunks
    int ckpt_per_seq;        // checkpoints per sequence when ckpt_off is NULL
};

size_t split_block_bytes(int dk);
int64_t split_max_chunks(int64_t total, int n_seqs);
// Sequence-order table alone (what the fused form needs), and table plus factor blocks.
size_t fused_workspace_bytes(int n_seqs);
size_t split_workspace_bytes(int64_t total, int n_seqs, int H, int dk);
// State-pass workgroup shape: ncw (1, 2 or 4) compute waves of 16 dv columns each, or 0 for
// the fused single-kernel prefill (one eight-wave workgroup per (sequence, head)).
hipError_t launch_prefill_split(const SplitArgs& a, int dk, bool bf16, int ncw, hipStream_t stream);

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const float* z;
    const float* A;
    float g_min;
    float* state;
    int N, H;
    void* o;
};

// Several consecutive tokens per sequence with the state held on chip: verify (outputs of
// every draft token, state read only) or commit (state advanced by accepted[n] tokens).
struct DecodeMultiArgs {
    const void* q;          // [N, K, H, dk] (verify only)
    const void* k;
    const void* v;          // [N, K, H, dv]
    const void* beta;       // [N, K, H]
    const float* z;         // [N, K, H, dk]
    const float* A;
    float g_min;
    const float* state_in;  // verify
    float* state;           // commit (in place)
    const int32_t* accepted;  // commit: tokens to replay per sequence, clamped to [0, K]
    int N, K, H;
    void* o;                // verify: [N, K, H, dv]
};
constexpr int kDecodeMaxDraft = 16;

struct OutputGateArgs {
    const void* o;      // [rows, dv]
    const void* gate;   // [rows, dv] gate logits
    const float* w;     // [dv] RMSNorm weight
    float eps;
    int64_t rows;
    void* y;            // [rows, dv]
};

struct ShortConvArgs {
    const void* x;          // [total, C] projected inputs
    const float* w;         // [C, W] taps, the last on the current token
    int W;                  // 1 .. 4
    const float* cache_in;  // nullable, [N, C, W-1]
    float* cache_out;       // nullable, [N, C, W-1]; may be cache_in
    const int32_t* cu;      // nullable => n_seqs sequences of T tokens
    int n_seqs;
    int64_t T;
    int64_t total;
    int C;
    int l2;                 // 0, or the channels of one head for L2Norm
    void* y;                // [total, C]
};

// Device address of the calling thread's current device's static scratch array
// (KDA_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_gate(const GateArgs& a, hipStream_t stream);
hipError_t launch_short_conv(const ShortConvArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_output_gate(const OutputGateArgs& a, int dv, bool bf16, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, hipStream_t stream);
hipError_t launch_decode_multi(const DecodeMultiArgs& a, int d, bool bf16, bool commit, hipStream_t stream);

}  // namespace kda
