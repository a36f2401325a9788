// Shared pieces of the token-selection kernels (select_tokens.hip and
// select_lse.hip): the K tile geometry, LDS addressing, the exchange
// across wavefront halves and the twelve K operand reads of a key row.
#pragma once

#include "common.h"

namespace hswa {
namespace {

constexpr int D = 192;
constexpr int KS = D / 16;              // k-steps of the 32x32x16 MFMA
constexpr int GQ = 16;                   // query heads per kv head (one MFMA column block)
constexpr int BK = 32;                   // keys per LDS tile
constexpr int KROW = D * 2;              // 384 B per key row
constexpr int KTILE = BK * KROW;         // 12 KB
constexpr int KINSTR = KTILE / 1024;     // 12 copies of 1 KB

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The partner of v across the wavefront halves: v_permlane32_swap on two
// copies of v leaves the lower half twice in one and the upper half twice
// in the other, a VALU move (no LDS round trip); both lanes of a pair see
// the operands in the same order.
struct Pair {
  float a, b;
};
__device__ __forceinline__ Pair halves32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// The twelve K operands of one key row: k-step 4 u + b sits 128 u bytes on
// from ad[b].  In asm: for a plain read the compiler would also wait for the
// next tile's copies in flight; the copies of this tile have been waited for
// before the barrier.  The block waits for its own reads before it returns.
__device__ __forceinline__ void lds_k12(bf16x8 (&f)[KS], const uint32_t (&ad)[4]) {
  uint4 r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11;
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b128 %4, %12 offset:128\n\t"
      "ds_read_b128 %5, %13 offset:128\n\t"
      "ds_read_b128 %6, %14 offset:128\n\t"
      "ds_read_b128 %7, %15 offset:128\n\t"
      "ds_read_b128 %8, %12 offset:256\n\t"
      "ds_read_b128 %9, %13 offset:256\n\t"
      "ds_read_b128 %10, %14 offset:256\n\t"
      "ds_read_b128 %11, %15 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
        "=&v"(r7), "=&v"(r8), "=&v"(r9), "=&v"(r10), "=&v"(r11)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
  f[0] = as_bf16x8(r0);
  f[1] = as_bf16x8(r1);
  f[2] = as_bf16x8(r2);
  f[3] = as_bf16x8(r3);
  f[4] = as_bf16x8(r4);
  f[5] = as_bf16x8(r5);
  f[6] = as_bf16x8(r6);
  f[7] = as_bf16x8(r7);
  f[8] = as_bf16x8(r8);
  f[9] = as_bf16x8(r9);
  f[10] = as_bf16x8(r10);
  f[11] = as_bf16x8(r11);
}
static_assert(KS == 12, "twelve k-steps of 16 dims");

}  // namespace
}  // namespace hswa
