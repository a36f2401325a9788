// Log-sum-exp rows for token selection on the gfx950 matrix cores.
//
// "MiMo-V3 HySparse2" (aideepthink.cn), section 4: the importance of token j
// for query i and kv head g is the full-attention layer's softmax
// probability summed over the group's query heads, which needs each head's
// normaliser lse_hi over the keys 0 .. i (no sink).  This kernel computes
// those rows; select_tokens_kernel (select_tokens.hip) ranks the candidates
// with them.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "select_ops.h"

namespace hswa {
namespace {

constexpr float kLazyCap = 0x1p60f;              // tile sums past this move the reference

// sum over the lane's 16 scores of 2^(c2 x - ref), in four partial sums
__device__ __forceinline__ float tile_sum(const f32x16& x, float c2, float ref) {
  float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 16; ++e) part[e & 3] += fast_exp2(fmaf(x[e], c2, -ref));
  return (part[0] + part[1]) + (part[2] + part[3]);
}

}  // namespace

// lse_hi = log2 sum_{j <= i} 2^(c2 s_hij) for every (row, head) of the rows
// that rank their candidates (i - recent + 1 > max_sel > 0).  A workgroup of
// four wavefronts owns 16 consecutive rows of one (sequence, kv head), four
// rows per wavefront: two blocks of 32 (row, head) columns, row 2 nb + c / 16
// of the wavefront and head c % 16 in column c of block nb.  Each block's
// product is K . Q^T with the 32 keys of a tile on M, so lane (column c,
// half h) holds 16 keys of one (row, head), and each score costs an fma, one
// exponential and an add.  The sum is
// taken against a reference that moves lazily: a tile is summed against the
// current reference and only if that sum passes kLazyCap (a key more than
// ~2^60 above it, or no reference yet) is the tile's max taken and the
// reference moved to it, so a tile costs no max tree on the common path.
// Any reference at or below the true max gives the same lse up to rounding
// (the sum holds at most 2^16 terms of at most 2^60: no overflow).  The two
// lane halves hold different keys of the same column and are merged at the
// end.  Two
// workgroups share a compute unit, one wavefront of each per SIMD, so that
// the matrix products of one overlap the exponentials of the other.
constexpr int LNW = 4;                           // wavefronts per workgroup
constexpr int LRW = 4;                           // rows per wavefront
constexpr int LROWS = LNW * LRW;                 // 16 rows per workgroup
constexpr int LCP = KINSTR / LNW;                // 1 KB tile copies per wavefront
static_assert(KINSTR % LNW == 0, "copies split evenly over the wavefronts");
constexpr int LNS = 4;                           // K tile stages: copies run three tiles ahead
static_assert(LCP == 3, "the waits below count three copies per tile");
__global__ __launch_bounds__(LNW * 64, 2) void select_lse_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char kst[LNS][KTILE];
  constexpr int RW = LRW;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 31, hi = lane >> 5;
  const int n = a.n, hkv = a.hkv, K = a.max_sel, recent = a.recent;
  const int nblk = (n + LROWS - 1) / LROWS;
  const int ngrp = a.B * hkv;
  const int items = ngrp * nblk;
  const int nwg = (int)gridDim.x, wg = (int)blockIdx.x;
  const float c2 = a.scale * kLog2e;
  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.half > 0 ? a.krot : a.k);
  const int kstride = hkv * KROW;

  // K tile copies (layout as in the selection kernel; wavefront w issues
  // copies w, w + 4, w + 8) and operand addresses
  int drow[LCP], doff[LCP];
#pragma unroll
  for (int u = 0; u < LCP; ++u) {
    const int sl = 64 * (wave + LNW * u) + lane;
    const int row = sl / 24, pc = sl - row * 24;
    drow[u] = row;
    doff[u] = 16 * (pc ^ ((row >> 1) & 7));
  }
  uint32_t koff[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) koff[bb] = c * KROW + 16 * ((2 * bb + hi) ^ ((c >> 1) & 7));

  // heaviest items first, alternating direction per round (as the selection kernel)
  for (int r = 0; r * nwg < items; ++r) {
    const int item = r * nwg + ((r & 1) ? nwg - 1 - wg : wg);
    if (item >= items) continue;
    const int blk = nblk - 1 - item / ngrp;
    const int bg = item - (item / ngrp) * ngrp;
    const int b = bg / hkv, g = bg - b * hkv;
    const int i0 = blk * LROWS;
    const int ilast = min(n - 1, i0 + LROWS - 1);
    // the block's last row has the most candidates: nothing to rank if it keeps them all
    if (K <= 0 || ilast - recent + 1 <= K) continue;
    const long long tokbase = (long long)b * n;
    const int r0 = i0 + RW * wave;               // the wavefront's first row

    int myrow[2];
    bf16x8 qf[2][KS];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      myrow[nb] = r0 + 2 * nb + (c >> 4);
      const bf16_t* qrow =
          Qp + ((tokbase + min(myrow[nb], n - 1)) * a.hq + g * GQ + (c & 15)) * D + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[nb][ks] = as_bf16x8(ld16(qrow + 16 * ks));
    }
    const unsigned char* kbase =
        reinterpret_cast<const unsigned char*>(Kp + (tokbase * hkv + g) * D);
    auto issue = [&](int k0, int kend, unsigned char* kd) {
#pragma unroll
      for (int u = 0; u < LCP; ++u) {
        const int key = min(k0 + drow[u], kend - 1);
        __builtin_amdgcn_global_load_lds(
            (glb_void_t*)(kbase + ((long long)key * kstride + doff[u])),
            (lds_void_t*)(kd + 1024 * (wave + LNW * u)), 16, 0, 0);
      }
    };

    // running (reference, sum) of the lane's column in each block over its
    // keys: l = sum 2^(c2 s - m).  The reference starts finite, so a masked
    // key (-inf) needs no special case, and at -FLT_MAX the first visible
    // key overflows the tile sum, which sets it
    float m[2] = {-__FLT_MAX__, -__FLT_MAX__}, l[2] = {0.f, 0.f};
    const int nkeys = ilast + 1;
    const int ntile = (nkeys + BK - 1) / BK;
    __syncthreads();                             // the previous item's tiles are consumed
    for (int t = 0; t < LNS - 1 && t < ntile; ++t) issue(t * BK, nkeys, kst[t]);
    for (int t = 0; t < ntile; ++t) {
      unsigned char* cur = kst[t % LNS];
      // this wavefront's copies of tile t have landed once at most those of
      // the (up to two) tiles issued after it are outstanding
      const int ahead = min(ntile - 1 - t, LNS - 2);
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0F76);        // vmcnt(6)
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F73);   // vmcnt(3)
      else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
      __syncthreads();                           // everyone's copies landed; tile t - 1 consumed
      if (t + LNS - 1 < ntile) issue((t + LNS - 1) * BK, nkeys, kst[(t + LNS - 1) % LNS]);
      const int k0 = t * BK;
      if (k0 > r0 + RW - 1) continue;            // keys past all of the wavefront's rows
      const uint32_t base = lds_addr(cur);
      uint32_t ad[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) ad[bb] = base + koff[bb];
      bf16x8 kf[KS];
      lds_k12(kf, ad);
      f32x16 sc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[nb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sc[nb] = mfma32(kf[ks], qf[nb][ks], sc[nb]);
      // element e is key k0 + 8 (e / 4) + 4 hi + e % 4
      const bool diag = k0 + BK - 1 > r0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x16 x = sc[nb];
        if (diag) {
          // key k0 + kk (kk = 8 (e / 4) + 4 hi + e % 4) is visible iff kk <= dhi
          const int dhi = myrow[nb] - (k0 + 4 * hi);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int kk = 8 * (e >> 2) + (e & 3);
            x[e] = (kk > dhi) ? kNegInf : x[e];
          }
        }
        float ps = tile_sum(x, c2, m[nb]);
        if (!(ps <= kLazyCap)) {
          // the reference is unset, or a key beats it by more than ~2^60:
          // move it to the running max and sum the tile again
          float mx = fmaxf(x[0], x[1]);
#pragma unroll
          for (int e = 2; e < 16; ++e) mx = fmaxf(mx, x[e]);
          const float mn = fmaxf(m[nb], mx * c2);
          l[nb] *= fast_exp2(m[nb] - mn);
          m[nb] = mn;
          ps = tile_sum(x, c2, mn);
        }
        l[nb] += ps;
      }
    }
    // merge the two halves' keys; lane (c, h) writes column c of block h
    float out[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const Pair pm = halves32(m[nb]), pl = halves32(l[nb]);
      const float M = fmaxf(pm.a, pm.b);
      const float L = pl.a * fast_exp2(pm.a - M) + pl.b * fast_exp2(pm.b - M);
      out[nb] = M + __log2f(L);
    }
    const int row = r0 + 2 * hi + (c >> 4);
    if (row < n) a.sel_lse[(tokbase + row) * a.hq + g * GQ + (c & 15)] = hi ? out[1] : out[0];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);            // no copy into LDS outlives the workgroup
}

hipError_t launch_select_lse(const AttnArgs& a, int cus, hipStream_t stream) {
  const long long lse_items = (long long)a.B * a.hkv * ((a.n + LROWS - 1) / LROWS);
  if (lse_items == 0) return hipSuccess;
  const unsigned lse_grid = (unsigned)(lse_items < 2 * cus ? lse_items : 2 * cus);
  hipLaunchKernelGGL(select_lse_kernel, dim3(lse_grid), dim3(LNW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hswa
