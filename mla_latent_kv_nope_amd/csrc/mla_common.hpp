// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int v2i32;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWave = 64;

// ---- bf16 <-> fp32 --------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite and infinite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair, round to nearest even (the compiler emits the
// gfx950 packed conversion for this pattern).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---- MFMA wrappers (layouts verified on gfx950) ---------------------------
// 32x32x16 bf16: A lane l holds row l%32, k = 8*(l/32)+[0,8); B lane l holds
// column l%32, same k; C element i of lane l is C[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16: A lane l holds row l%16, k = 8*(l/16)+[0,8); B lane l holds
// column l%16, same k; C element i of lane l is C[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- LDS transpose read ---------------------------------------------------
// Within each group of 16 lanes, destination lane i receives element (i%4) of
// the 8 bytes read by source lane 4*e + i/4, for e = 0..3.  With source lane
// 4r+q pointing at row r, columns [4q, 4q+4) of a row-major 16-bit tile, lane i
// receives column i of rows 0..3.
// The pointer must point into a __shared__ array; it is converted with an
// address-space cast (not through an integer), so the compiler still knows
// which object is read: a read whose object is unknown makes it wait for every
// in-flight global->LDS copy first.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* lds_ptr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<void*>(lds_ptr)));
  return __builtin_bit_cast(bf16x4, v);
}

// 8-bit transpose read: in each 16-lane group, lane j receives byte j % 8 of
// the 8 bytes addressed by lane 2k + j / 8 as its byte k (k = 0 .. 7): the
// group's lanes address 8 rows of 16 bytes (two lanes per row) and each lane
// gets one column of them.
__device__ __forceinline__ v2i32 lds_read_tr8(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i32*)(const_cast<void*>(lds_ptr)));
}

// ---- fp8 ------------------------------------------------------------------
// Two OCP e4m3 codes (byte pair 0-1, or 2-3 with HI) as two bf16, exactly:
// every e4m3 value (3 mantissa bits, exponents -9..8) is a bf16 value.  The
// gfx950 conversion instruction runs at scale 1 (its scale operand only
// takes the power-of-two part).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, HI));
}
// Two e4m3 codes times an fp32 scale, rounded to two bf16: the codes are
// converted exactly to fp32 (scale 1), multiplied by the scale in fp32 and
// rounded to nearest even.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2_scaled(uint32_t codes, float scale) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
  const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, 1.0f, HI);
  return pack_bf16x2(v[0] * scale, v[1] * scale);
}

// ---- raw buffer access -----------------------------------------------------
// A buffer resource over [p, p + bytes) in the gfx9 raw (unswizzled) format.
// Loads and stores through it take a per-lane 32-bit offset plus a uniform
// offset, so a run of accesses at constant distances needs no 64-bit address
// per access.  Out-of-range accesses read 0 and drop writes.
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void buffer_store_f32x4(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, static_cast<int>(voff),
                                         static_cast<int>(soff), 0);
}
__device__ __forceinline__ f32x4 buffer_load_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
// four fp32 <-> four bf16 (round to nearest even) through an 8-byte access
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
__device__ __forceinline__ void buffer_store_bf16x4(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                    uint32_t soff) {
  const i32x2 p = {static_cast<int>(pack_bf16x2(v[0], v[1])), static_cast<int>(pack_bf16x2(v[2], v[3]))};
  __builtin_amdgcn_raw_buffer_store_b64(p, r, static_cast<int>(voff), static_cast<int>(soff), 0);
}
__device__ __forceinline__ f32x4 buffer_load_bf16x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const i32x2 p = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voff), static_cast<int>(soff), 0);
  const uint32_t lo = static_cast<uint32_t>(p[0]), hi = static_cast<uint32_t>(p[1]);
  return f32x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u), __uint_as_float(hi << 16),
               __uint_as_float(hi & 0xffff0000u)};
}

// ---- global -> LDS copies -------------------------------------------------
// 16 bytes per lane from global memory straight into LDS: lane l writes LDS
// bytes [lds + 16l, +16).  Issued through inline assembly so that the
// compiler does not track them: it would otherwise make transpose reads wait
// for every copy in flight.  The caller orders them with wait_vmcnt and a
// workgroup barrier before the data is read.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
// (wave-uniform operands are passed through readfirstlane so that they are
// scalar registers)
__device__ __forceinline__ uint64_t uniform_u64(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// source = sbase (wave-uniform) + voff (per lane)
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  __asm__ __volatile__("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                       :
                       : "v"(voff), "s"(uniform_u64(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                       : "memory", "m0");
}
// source = per-lane address
__device__ __forceinline__ void lds_dma16_v(const void* src, uint32_t lds) {
  __asm__ __volatile__("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                       :
                       : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
                       : "memory", "m0");
}

// ---- waits and barriers ---------------------------------------------------
// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that also stops the compiler moving memory operations across it.
__device__ __forceinline__ void block_barrier() {
  __asm__ __volatile__("s_barrier" ::: "memory");
}

// ---- cross-lane helpers ---------------------------------------------------
__device__ __forceinline__ float max_across_half_waves(float x) {
  // {x[l], x[l ^ 32]} as a pair on every lane
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_half_waves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// {x[l], x[l ^ 16]} as a pair on every lane
__device__ __forceinline__ float max_across_quarter_pairs(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_quarter_pairs(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane index recomputed at each use (two VALU ops).  The volatile asm keeps the
// compiler from hoisting values derived from it out of loops, which trades a
// few instructions for registers that would otherwise stay occupied.
__device__ __forceinline__ int lane_id_fresh() {
  int l;
  __asm__ __volatile__("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ float shfl_f32(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

}  // namespace mla
