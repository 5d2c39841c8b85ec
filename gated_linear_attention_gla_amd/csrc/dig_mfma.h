// dig_mfma.h -- gfx950 device helpers shared by the bf16 GLA kernels:
// v_mfma_f32_16x16x32_bf16 operands, LDS reads (plain and transposing), raw
// buffer loads/stores with out-of-range zeroing, and an LDS-only barrier.
//
// MFMA 16x16x32 operand layout: lane l supplies row (A) / column (B) l % 16
// and the 8-element K slice l / 16; the accumulator holds rows 4*(l/16) + e,
// e = 0..3, of column l % 16.  The K order inside one product is free as long
// as A and B agree.
#pragma once

#include "dig_internal.h"

namespace dig {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// A 16-wide K block on the 32-wide instruction, upper half zero.  (Kept on
// one MFMA shape: a 16x16x16 result feeding a 16x16x32 accumulator in
// another register was issued without the wait states it needs.)
__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
  return mfma32(make_uint4(a.x, a.y, 0u, 0u), make_uint4(b.x, b.y, 0u, 0u), c);
}
__device__ __forceinline__ uint2 pack4(f32x4_t x) {
  return make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}
__device__ __forceinline__ uint4 cat(uint2 lo, uint2 hi) { return make_uint4(lo.x, lo.y, hi.x, hi.y); }
__device__ __forceinline__ uint2 lds2(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
// Global memory accesses through address-space-1 pointers, so they compile to
// global_load/global_store (vmcnt only) rather than FLAT instructions, which
// would also count in lgkmcnt and be waited on by every LDS barrier.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gload16(const uint16_t *p) {
  const u32x4_t v = *(__attribute__((address_space(1))) const u32x4_t *)(size_t)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Raw buffer loads: 48-bit base (one (batch, head) slice, wave-uniform) plus
// a 32-bit byte offset per lane.  Offsets at or beyond num_records return
// zeros, which serves both the ragged tail and the channel padding without
// predication.  Word 3 = untyped 32-bit data format (CDNA).
constexpr unsigned kOOB = 0x80000000u;   // an offset past every valid span
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Raw buffer store of 8 bytes; out-of-range offsets are dropped, so stores
// need no branch (which would split the surrounding MFMA code into blocks).
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, unsigned off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, unsigned off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)off, 0, 0);
}
__device__ __forceinline__ uint4 lds4(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane j
// receives element (j % 4) of the 8-byte read addressed by lane 4e + j/4,
// e = 0..3.  If lane s of the group addresses row t0 + s/4, column
// c0 + 4*(s%4) of a token-major tile, lane j receives column c0 + j of rows
// t0 .. t0+3.
__device__ __forceinline__ uint2 lds_tr(const uint16_t *p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_t *)(__attribute__((address_space(3))) char *)(size_t)(p));
  return __builtin_bit_cast(uint2, r);
}

// 2^x on the transcendental unit (v_exp_f32); results below 2^-126 flush to 0.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Device-coherent 16-byte accesses for the state hand-off between
// workgroups: cache-policy bit sc1 (what the compiler emits for agent-scope
// atomics) writes through to the coherence point and reads from it, so no L2
// writeback/invalidate fence is needed.
constexpr int kCohPolicy = 16;
__device__ __forceinline__ float4 bload_coh(__amdgpu_buffer_rsrc_t r, unsigned off) {
  const f32x4_t v = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCohPolicy));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void bstore_coh(__amdgpu_buffer_rsrc_t r, unsigned off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                                 __float_as_uint(v.w)},
                                         r, (int)off, 0, kCohPolicy);
}
// Wait until all of this wave's vector-memory operations (loads and stores)
// have completed.
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS-only workgroup barrier: waits for this wave's LDS traffic, not for its
// global loads, so prefetches stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace
}  // namespace dig
