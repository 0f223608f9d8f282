// kda_device.h -- device-side helpers shared by the gfx950 KDA kernels.
//
// bf16 values are kept as raw 16-bit patterns (uint16_t) in memory; conversion from fp32
// uses the hardware round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950).
// Matrix products use the CDNA4 bf16 MFMA instructions with fp32 accumulation:
//   mfma32: v_mfma_f32_16x16x32_bf16   A 16x32, B 32x16, 8 bf16 per lane per operand
//   mfma16: v_mfma_f32_16x16x16_bf16   A 16x16, B 16x16, 4 bf16 per lane per operand
// Lane layout of a 16x16 fp32 result (wave64, lane l, g = l/16, r = 0..3): row 4g+r,
// column l%16.  Operand lanes supply row (A) or column (B) l%16; the K positions a lane
// supplies are indexed by (g, slot) identically for A and B, so any consistent
// assignment of logical K indices to (g, slot) yields the same contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 -> two bf16 packed into 32 bits (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x and 1/x on the hardware transcendental unit (about 1 ulp in fp32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint2 pack_bf16x4(f32x4_t v) {
    return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// --- buffer (SGPR-descriptor) memory access ----------------------------------------------
// A raw buffer covers [base, base + nbytes).  Loads at byte offsets >= nbytes return zero
// and stores there are dropped, so a descriptor rebased at a chunk's first token with
// nbytes = (valid rows) x (row bytes) masks the rows past a sequence's end without any
// per-lane test, and addressing needs no 64-bit per-lane arithmetic.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(nbytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload2(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, off, 0, 0);
}

// Streaming 16-byte global accesses for data that one kernel touches exactly once (inputs
// read once, outputs written once): the nontemporal hint keeps them from displacing lines
// that other accesses reuse.
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream16(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, static_cast<u32x4_t*>(p));
}
__device__ __forceinline__ float4 ld_stream_f4(const void* p) {
    const uint4 u = ld_stream16(p);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
}
__device__ __forceinline__ void st_stream_f4(void* p, float4 v) {
    st_stream16(p, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                              __float_as_uint(v.w)));
}

// LDS-DMA: the 64 lanes' 16-byte pieces at byte offsets voff of r are written, in lane
// order, to the contiguous 1 KiB at lds (a workgroup-uniform LDS address), without passing
// through registers.  Out-of-range lanes write zeros.  Completion is tracked by vmcnt.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}
// The same with 4-byte pieces (256 bytes at lds).
__device__ __forceinline__ void dma4(rsrc_t r, void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voff, 0, 0, 0);
}

// --- element loads of the caller's tensor type -------------------------------------------

template <typename T> struct Elem;

template <> struct Elem<bf16_t> {
    // 8 consecutive elements -> 8 bf16 (16 bytes)
    __device__ __forceinline__ static uint4 load8(const bf16_t* p) {
        return *reinterpret_cast<const uint4*>(p);
    }
    __device__ __forceinline__ static float load1(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store1(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

template <> struct Elem<float> {
    __device__ __forceinline__ static uint4 load8(const float* p) {
        float4 a = reinterpret_cast<const float4*>(p)[0];
        float4 b = reinterpret_cast<const float4*>(p)[1];
        return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                          pack_bf16x2(b.z, b.w));
    }
    __device__ __forceinline__ static float load1(const float* p) { return *p; }
    __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

// Workgroup barrier that orders LDS accesses only.  A full __syncthreads() also waits for
// every outstanding global load and store of the thread (s_waitcnt vmcnt(0)), which would
// stall on in-flight prefetches and output stores; LDS is the only memory the workgroup's
// threads exchange through.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Start token of sequence n: cu_seqlens[n] when given, else n * T (equal-length batch).
__device__ __forceinline__ int64_t seq_start(const int32_t* cu, int64_t T, int n) {
    return cu ? static_cast<int64_t>(cu[n]) : static_cast<int64_t>(n) * T;
}

}  // namespace kda
