// Device helpers shared by the gfx950 kernels: bf16 packing, 16-byte
// loads and stores, MFMA operand types, wavefront reductions and the
// workgroup-to-XCD remapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hswa {

typedef uint16_t bf16_t;                                     // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));   // MFMA operand
typedef float f32x4 __attribute__((ext_vector_type(4)));     // 16x16 MFMA accumulator
typedef float f32x16 __attribute__((ext_vector_type(16)));   // 32x32 MFMA accumulator
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Status codes mirrored from hswa.h for the internal launchers.
enum { ST_OK = 0, ST_INVALID = 1, ST_UNSUPPORTED = 2, ST_HIP = 3 };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Low / high bfloat16 of a packed dword, widened exactly to fp32.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values rounded to nearest-even bfloat16 and packed (lo, hi).
// On gfx950 this is the hardware v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Element e (0..7) of eight packed bfloat16 values, widened to fp32.
__device__ __forceinline__ float elem_bf16(const uint4& v, int e) {
  uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return (e & 1) ? hi_bf16(w) : lo_bf16(w);
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = lo_bf16(v.x); f[1] = hi_bf16(v.x);
  f[2] = lo_bf16(v.y); f[3] = hi_bf16(v.y);
  f[4] = lo_bf16(v.z); f[5] = hi_bf16(v.z);
  f[6] = lo_bf16(v.w); f[7] = hi_bf16(v.w);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

// D = A * B + C on the 16x16x32 bf16 matrix core.  With lane l = 16*g + c:
// A holds row c, k-block g (8 values); B holds column c, k-block g; D holds
// rows 4*g .. 4*g+3 of column c.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A * B + C on the 32x32x16 bf16 matrix core.  With lane l = 32*h + i:
// A holds row i, k = 8h .. 8h+7; B holds column i, k = 8h .. 8h+7; element
// v of D is row 8*(v/4) + 4*h + v%4 of column i.  On gfx950 it sustains
// twice the flops per cycle of the 16x16x32 form.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// c + lo + hi of a packed bf16 pair, in fp32 (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float c) {
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// gfx950 transposed LDS read of 4 x 16-bit values (ds_read_b64_tr_b16).
// Within each group of 16 lanes, lane i receives element i % 4 of the 8
// bytes addressed by lane 4k + i / 4, for k = 0..3.  With a row-major matrix
// in LDS and lane j addressing M[r0 + j/4][c0 + 4 * (j % 4)], lane i gets the
// column M[r0 + k][c0 + i], k = 0..3: the k-major operand layout of an MFMA.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr4(const void* p) {
  typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p);
  return __builtin_bit_cast(uint2, r);
}

// Decode lazy-rescaling threshold (log2 units): a running max moves only when
// a tile's max passes it by more than this, so the probabilities stay
// below 2^kDecLazy.
constexpr float kDecLazy = 8.f;

// Workgroup barrier without the release fence of __syncthreads(), which
// would wait for every copy in flight; the caller waits with an explicit
// vmcnt for the copies it needs, and its LDS writes that other wavefronts
// read must be complete (lgkmcnt) before it.  The empty asm statements keep
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS reads of global_load_lds targets, written as inline asm with their own
// lgkmcnt(0) wait.  The compiler's wait analysis would otherwise see a plain
// read as one of memory that copies in flight may write and wait for every
// copy (vmcnt(0)), also those issued for later tiles; the caller waits for
// the copies of the tile it reads (s_waitcnt vmcnt) and a barrier.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_b128x2(uint4& r0, uint4& r1, uint32_t a0, uint32_t a1) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(a0), "v"(a1)
      : "memory");
}
__device__ __forceinline__ void lds_b64x6(uint2 (&r)[6], const uint32_t (&a)[6]) {
  asm volatile(
      "ds_read_b64 %0, %6\n\t"
      "ds_read_b64 %1, %7\n\t"
      "ds_read_b64 %2, %8\n\t"
      "ds_read_b64 %3, %9\n\t"
      "ds_read_b64 %4, %10\n\t"
      "ds_read_b64 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
      : "memory");
}
__device__ __forceinline__ void lds_b128x6(uint4 (&r)[6], const uint32_t (&a)[6]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b128 %4, %10\n\t"
      "ds_read_b128 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
      : "memory");
}
// Eight transposed 4 x 16-bit reads (as lds_tr4).
__device__ __forceinline__ void lds_tr4x8(uint2 (&r)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// Codes 2w, 2w + 1 of the 4 E4M3 codes in v (w = 0 or 1) as a packed bf16
// pair, by gfx950's direct E4M3 -> bf16 conversion with a unit scale: every
// E4M3 value is a bf16 value, so the conversion is exact (the same bits as
// the exact conversion to fp32 with the lower halves dropped).
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}

// 8 E4M3 codes -> 8 bf16 (element e from byte e).
__device__ __forceinline__ uint4 widen8(uint2 w) {
  return make_uint4(e4m3_pair<false>(w.x), e4m3_pair<true>(w.x), e4m3_pair<false>(w.y),
                    e4m3_pair<true>(w.y));
}

// Max / sum across the four lanes l, l^16, l^32, l^48 (same column c), with
// gfx950's row-swapping moves instead of LDS-routed lane shuffles:
// v_permlane16_swap on two copies of v leaves rows (0, 0, 2, 2) in one and
// (1, 1, 3, 3) in the other, v_permlane32_swap the lower half twice in one
// and the upper half twice in the other; both lanes of a pair combine the
// same two operands in the same order.
__device__ __forceinline__ float max_across_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  This maps the
// hardware id to a logical id such that each XCD receives one contiguous
// range of logical ids, so neighbouring tiles share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int q = nwg >> 3, rem = nwg & 7;
  const int x = bid & 7, slot = bid >> 3;
  return (x < rem) ? x * (q + 1) + slot : rem * (q + 1) + (x - rem) * q + slot;
}

// Heavy / light interleave for causal work: 0 -> nb-1, 1 -> 0, 2 -> nb-2, ...
// Any contiguous run of indices then carries a balanced amount of work.
__device__ __forceinline__ int zigzag(int k, int nb) {
  return (k & 1) ? (k >> 1) : (nb - 1 - (k >> 1));
}

}  // namespace hswa
