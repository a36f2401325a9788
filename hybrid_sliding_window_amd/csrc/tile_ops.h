// Tile-level building blocks shared by the matrix-core prefill kernels
// (d_qk = 192, d_v = 128, bf16): the 32-key K/V tile geometry and its LDS
// layout, the global-to-LDS copies, the explicit vector-memory waits, the
// LDS operand reads written as inline asm that wait for their own data, and
// the in-register RoPE of q.
//
// LDS layout of a tile (unpadded rows, XOR swizzles applied on the global
// side of the copies so that the MFMA operand reads hit distinct banks):
//   K (and q)  rows of 384 B   16-byte chunk c of row r at c ^ ((r >> 1) & 7)
//   V          rows of 256 B   64-byte unit u of row r at u ^ (r & 3)
#pragma once

#include "common.h"

namespace hswa {
namespace {

constexpr int D = 192;
constexpr int DV = 128;
constexpr int KS = D / 16;             // 12 k-steps of the 32x32x16 MFMA
constexpr int MT = DV / 32;            // 4 output tiles of 32 dims
constexpr int BK = 32;                 // keys per tile
constexpr int KROW = D * 2;            // 384 B
constexpr int VROW = DV * 2;           // 256 B
constexpr int KTILE = BK * KROW;       // 12 KB = 12 load instructions
constexpr int VTILE = BK * VROW;       // 8 KB = 8
constexpr int MAX_HALF = 32;           // rotary pairs handled
constexpr int MAX_HQ = 256;            // sinks kept in LDS

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void g2lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_base, 16, 0, 0);
}
// The same with the non-temporal hint, for data read exactly once (q): it
// should not push the K/V rows that the next items read again out of L2.
__device__ __forceinline__ void g2lds16_nt(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_base, 16, 0, 2);
}


// The two matrix-core prefill kernels sum a tile's P (per lane, 16 keys)
// against the current reference and move the reference only when that sum
// passes kLazySum: every P is then at most 2^12, well inside bf16 and fp32.
constexpr float kLazySum = 4096.f;

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
#define VMCNT(n) (0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// Wait until the copy that has `younger` vector-memory operations issued
// after it has completed: vmcnt(k) for the largest listed k <= younger.
// The counter saturates at 63, so at 63 younger operations the copy is done.
__device__ __forceinline__ void wait_copy(int younger) {
  if (younger <= 0) { __builtin_amdgcn_s_waitcnt(VMCNT(0)); return; }
  if (younger >= 63) return;
  if (younger >= 48) __builtin_amdgcn_s_waitcnt(VMCNT(48));
  else if (younger >= 40) __builtin_amdgcn_s_waitcnt(VMCNT(40));
  else if (younger >= 32) __builtin_amdgcn_s_waitcnt(VMCNT(32));
  else if (younger >= 24) __builtin_amdgcn_s_waitcnt(VMCNT(24));
  else if (younger >= 21) __builtin_amdgcn_s_waitcnt(VMCNT(21));
  else if (younger >= 20) __builtin_amdgcn_s_waitcnt(VMCNT(20));
  else if (younger >= 16) __builtin_amdgcn_s_waitcnt(VMCNT(16));
  else if (younger >= 13) __builtin_amdgcn_s_waitcnt(VMCNT(13));
  else if (younger >= 12) __builtin_amdgcn_s_waitcnt(VMCNT(12));
  else if (younger >= 8) __builtin_amdgcn_s_waitcnt(VMCNT(8));
  else if (younger >= 5) __builtin_amdgcn_s_waitcnt(VMCNT(5));
  else if (younger >= 3) __builtin_amdgcn_s_waitcnt(VMCNT(3));
  else if (younger >= 2) __builtin_amdgcn_s_waitcnt(VMCNT(2));
  else __builtin_amdgcn_s_waitcnt(VMCNT(1));
}

// LDS reads of the copy targets.  They are written as inline asm, each
// block ending with its own lgkmcnt(0) wait, so the compiler does not see
// them as reads of memory that copies in flight may write: its wait
// analysis cannot follow the copy stream across items and would otherwise
// wait for every copy in flight.  The explicit vmcnt waits above, followed
// by a workgroup barrier, are what order each read after its copy.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Operand k-steps 0..5 / 6..11 of a 384-byte row: k-step 4q + r at a[r] + 128 q.
__device__ __forceinline__ void lds_ksteps_lo(u32x4 (&f)[KS], uint32_t a0, uint32_t a1, uint32_t a2,
                                              uint32_t a3) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b128 %4, %6 offset:128\n\t"
      "ds_read_b128 %5, %7 offset:128\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}
__device__ __forceinline__ void lds_ksteps_hi(u32x4 (&f)[KS], uint32_t a0, uint32_t a1, uint32_t a2,
                                              uint32_t a3) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:128\n\t"
      "ds_read_b128 %1, %9 offset:128\n\t"
      "ds_read_b128 %2, %6 offset:256\n\t"
      "ds_read_b128 %3, %7 offset:256\n\t"
      "ds_read_b128 %4, %8 offset:256\n\t"
      "ds_read_b128 %5, %9 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[6]), "=&v"(f[7]), "=&v"(f[8]), "=&v"(f[9]), "=&v"(f[10]), "=&v"(f[11])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// V^T operand pieces of key step KK of a 32-key tile: for output tile mt,
// the rows 16 KK + 0..7 piece at a[mt] + 4096 KK and the rows 16 KK + 8..15
// piece 2048 bytes further (ds_read_b64_tr_b16, see lds_tr4).
template <int KK>
__device__ __forceinline__ void lds_vhalf(u32x2 (&f)[8], uint32_t a0, uint32_t a1, uint32_t a2,
                                          uint32_t a3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
        "=&v"(f[6]), "=&v"(f[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "i"(4096 * KK), "i"(4096 * KK + 2048)
      : "memory");
}

// Rotate the rotary k-steps of q (pair (ka, ka + PK): dims 16 ka + 8 h + e
// and + R/2) by pos * theta^(-p/half) for pair p = 16 ka + 8 h + e; other
// k-steps keep their exact bf16 values.  rev[p] = theta^(-p/half) / (2 pi)
// in fp64: the angle in revolutions is formed in fp64 (positions reach
// 2^18 and beyond), reduced to [0, 1) and only then evaluated in fp32 with
// the hardware sine and cosine, which take revolutions.
template <int PK>
__device__ __forceinline__ void rotate_q(u32x4 (&qf)[KS], const double* rev, double pos, int h) {
#pragma unroll
  for (int ka = 0; ka < PK; ++ka) {
    float x0[8], x1[8];
    unpack8(__builtin_bit_cast(uint4, qf[ka]), x0);
    unpack8(__builtin_bit_cast(uint4, qf[ka + PK]), x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double turns = pos * rev[16 * ka + 8 * h + e];
      const float f = (float)(turns - floor(turns));
      const float c = __builtin_amdgcn_cosf(f);
      const float sn = __builtin_amdgcn_sinf(f);
      const float y0 = x0[e] * c - x1[e] * sn;
      const float y1 = x1[e] * c + x0[e] * sn;
      x0[e] = y0;
      x1[e] = y1;
    }
    qf[ka] = __builtin_bit_cast(u32x4, pack8(x0));
    qf[ka + PK] = __builtin_bit_cast(u32x4, pack8(x1));
  }
}

// Per-lane LDS byte offsets of the MFMA operand reads from a tile, for lane
// (i = lane & 31, h = lane >> 5).  K (A operand of S^T = K . Q^T): row r of
// the tile holds logical 16-byte chunk c at physical chunk c ^ ((r >> 1) & 7),
// and for k-step ks = 4q + j this lane (row i, half h) reads chunk
// 8q + 2 (j ^ s1) + h1, i.e. krd[j] + 128 q (see lds_ksteps_lo / _hi).
// V^T (A operand of O^T += V^T . P^T, read transposed): key row 4h + jv/4
// (+ 16 kk, + 8), 8-byte piece jv % 4 at dim 16 (p & 1) + 4 (p >> 1) + 8 ihi
// of the 32-dim output tile, so that lane (i, h) receives dims 16h + 0..15
// of each tile in its 16 outputs; the 64-byte unit of output tile mt in that
// row is mt ^ (row & 3) = mt ^ (jv / 4).
__device__ __forceinline__ void operand_offsets(int lane, uint32_t (&krd)[4], uint32_t (&vrd)[4]) {
  const int i = lane & 31, h = lane >> 5;
  const int sw = (i >> 1) & 7;
  const int s1 = sw >> 1, h1 = h ^ (sw & 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) krd[j] = i * KROW + 16 * (2 * (j ^ s1) + h1);
  const int jv = lane & 15, ihi = (lane >> 4) & 1;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    vrd[mt] = (4 * h + (jv >> 2)) * VROW + 32 * (jv & 1) + 8 * ((jv >> 1) & 1) + 16 * ihi +
              64 * (mt ^ (jv >> 2));
}

}  // namespace
}  // namespace hswa
