// bf16 prefill on the gfx950 matrix cores: sliding-window attention with a
// sink, and (window 0, no sink) the full-causal GA sibling.
//
// Operation: "MiMo-V2-Flash: Hybrid Sliding Window Attention Architecture"
// (rslog.cc) section 2.1 (window), 2.3 (scores), 4.4 (sink-seeded max and
// denominator, output), 5 (GA rows have no sink).  Head shapes from
// "MiMo-V2.6-Flash hybrid SWA" (pwwt.cn) sections 3-4: d_qk 192, d_v 128,
// 64 query heads over 8 (SWA) or 4 (GA) kv heads.
//
// Work decomposition.  A workgroup (4 wavefronts) owns one kv head g and a
// block of T = 128 / G consecutive query tokens; its 128 rows are those T
// tokens times the G query heads of group g, so every K/V tile staged in
// LDS serves all of them.  Each wavefront holds 32 rows as two 16-column
// MFMA operands.
//
// Orientation.  Scores are computed transposed, S^T = K . Q^T, so a lane
// owns one query row (column c) and four keys per 16-key sub-tile.  Two
// sub-tiles of that output are, lane for lane, the B operand of the next
// product O^T += V^T . P^T, so P never leaves registers.  The row max needs
// only two cross-lane steps (lanes c, c+16, c+32, c+48); the row sum stays
// per lane until the end.
//
// Softmax runs in base 2: the fp32 scores are multiplied by scale * log2(e)
// inside the exp2 argument (one FMA), so q is rounded to bf16 only where
// RoPE changed it; the sink is multiplied by log2(e) only.  The state starts at m = sink, l = 1 (one lane per row), which is
// the sink's exp(sink - m) term of the denominator.
//
// RoPE.  q is rotated in registers (pairs r, r + R/2 sit in the same lane
// when R/2 is a multiple of 32); K is rotated while it is staged into LDS.
// The cos/sin values come from a table built in fp64 for the call.
#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

constexpr int D = 192;                 // q/k head dim
constexpr int DV = 128;                // v head dim
constexpr int KS = D / 32;             // k-steps of the 16x16x32 MFMA
constexpr int NT = DV / 16;            // 16-wide output tiles
constexpr int BK = 32;                 // keys per staged tile
constexpr int ROWS = 128;              // query rows per workgroup
constexpr int NTHREADS = 256;
constexpr int KSTR = D + 8;            // K row pitch in LDS (elements): 400 B
constexpr int VSTR = BK + 8;           // V^T row pitch in LDS (elements): 80 B
constexpr int KUNITS = BK * 12;        // 12 two-chunk units per K row

// Rotate q held as KS k-steps of 8 values: pair (ka, ka + PK) in lane.
template <int PK>
__device__ __forceinline__ void rotate_q(float (&f)[KS][8], const float2* __restrict__ trow,
                                         int grp) {
#pragma unroll
  for (int ka = 0; ka < PK; ++ka) {
    const float2* t = trow + 32 * ka + 8 * grp;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = t[e];
      const float x0 = f[ka][e], x1 = f[ka + PK][e];
      f[ka][e] = x0 * cs.x - x1 * cs.y;
      f[ka + PK][e] = x1 * cs.x + x0 * cs.y;
    }
  }
}

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

}  // namespace

__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(AttnArgs a, int log2g,
                                                                   int nblk, int balance) {
  __shared__ __attribute__((aligned(16))) bf16_t sk[BK * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t svt[DV * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, grp = lane >> 4;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bg = logical / nblk;
  const int kb = logical - bg * nblk;
  const int blk = balance ? zigzag(kb, nblk) : kb;
  const int b = bg / a.hkv, g = bg - b * a.hkv;
  const int G = 1 << log2g;
  const int T = ROWS >> log2g;
  const int n = a.n;
  const int i0 = blk * T;
  const long long tokbase = (long long)b * n;

  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ Vp = static_cast<const bf16_t*>(a.v);
  bf16_t* __restrict__ Op = static_cast<bf16_t*>(a.o);

  // ---- the two query rows of this lane ---------------------------------
  int tok[2], head[2];
  bool rv[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int r = wave * 32 + cb * 16 + c;
    tok[cb] = i0 + (r >> log2g);
    head[cb] = g * G + (r & (G - 1));
    rv[cb] = tok[cb] < n;
  }

  // ---- q: load, rotate, round to bf16 -----------------------------------
  bf16x8 qf[2][KS];
  const float c2 = a.scale * kLog2e;   // raw score -> base-2 units
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    float f[KS][8];
    if (rv[cb]) {
      const bf16_t* qrow = Qp + ((tokbase + tok[cb]) * a.hq + head[cb]) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) unpack8(ld16(qrow + 32 * ks), f[ks]);
      if (a.half > 0) {
        const float2* trow = a.rope + (long long)tok[cb] * a.half;
        switch (a.half >> 5) {
          case 1: rotate_q<1>(f, trow, grp); break;
          case 2: rotate_q<2>(f, trow, grp); break;
          default: rotate_q<3>(f, trow, grp); break;
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) f[ks][e] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[cb][ks] = as_bf16x8(pack8(f[ks]));
  }

  // ---- softmax state seeded with the sink -------------------------------
  float m[2], l[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float s2 = a.sink ? a.sink[head[cb]] * kLog2e : kNegInf;
    m[cb] = s2;
    l[cb] = (grp == 0 && s2 > kNegInf) ? 1.f : 0.f;
  }
  f32x4 acc[2][NT];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[cb][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- key range of the workgroup and of this wavefront ----------------
  const int W = a.window;
  const int kstart = (W > 0) ? max(0, i0 - W + 1) : 0;
  const int kend = min(n, i0 + T);
  const int tw0 = i0 + ((wave * 32) >> log2g);
  const int tw1 = min(n - 1, i0 + ((wave * 32 + 31) >> log2g));
  const bool wave_live = tw0 < n;
  const int npair = a.half >> 3;       // rotary 8-dim chunk pairs per K row

  for (int j0 = kstart; j0 < kend; j0 += BK) {
    __syncthreads();  // the previous tile is no longer read

    // -- stage K (rotated) into LDS: [key][dim], 16-byte chunks --------
    for (int u = tid; u < KUNITS; u += NTHREADS) {
      const int kk = u / 12, slot = u - (u / 12) * 12;
      const int j = j0 + kk;
      const bool rot = slot < npair;
      const int c0 = rot ? slot : 2 * npair + 2 * (slot - npair);
      const int c1 = rot ? slot + npair : c0 + 1;
      uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
      if (j < kend) {
        const bf16_t* kp = Kp + ((tokbase + j) * a.hkv + g) * D;
        x0 = ld16(kp + 8 * c0);
        x1 = ld16(kp + 8 * c1);
        if (rot) {
          const float2* tr = a.rope + (long long)j * a.half + 8 * c0;
          float f0[8], f1[8];
          unpack8(x0, f0);
          unpack8(x1, f1);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float2 cs = tr[e];
            const float y0 = f0[e] * cs.x - f1[e] * cs.y;
            const float y1 = f1[e] * cs.x + f0[e] * cs.y;
            f0[e] = y0;
            f1[e] = y1;
          }
          x0 = pack8(f0);
          x1 = pack8(f1);
        }
      }
      st16(&sk[kk * KSTR + 8 * c0], x0);
      st16(&sk[kk * KSTR + 8 * c1], x1);
    }

    // -- stage V transposed into LDS: [dv][key slot] ---------------------
    // Key kk of the tile goes to slot 8*((kk>>2)&3) + 4*(kk>>4) + (kk&3):
    // the 8 keys one lane feeds the PV product become one 16-byte read.
    if (tid < 128) {
      const int kq = tid & 7, dc = tid >> 3;
      uint4 rr[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = j0 + 4 * kq + q4;
        rr[q4] = (j < kend) ? ld16(Vp + ((tokbase + j) * a.hkv + g) * DV + 8 * dc)
                            : make_uint4(0, 0, 0, 0);
      }
      const int pos0 = 8 * (kq & 3) + 4 * (kq >> 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = half16(rr[0], e) | (half16(rr[1], e) << 16);
        const uint32_t w1 = half16(rr[2], e) | (half16(rr[3], e) << 16);
        st8(&svt[(8 * dc + e) * VSTR + pos0], make_uint2(w0, w1));
      }
    }
    __syncthreads();

    if (!wave_live || j0 > tw1) continue;
    if (W > 0 && j0 + BK - 1 < tw0 - W + 1) continue;
    const bool need_mask = (j0 + BK - 1 > tw0) || (W > 0 && j0 < tw1 - W + 1);

    // -- S^T = K . Q^T for two 16-key sub-tiles ---------------------------
    f32x4 s[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      s[sub][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[sub][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 kf = as_bf16x8(ld16(&sk[(sub * 16 + c) * KSTR + 32 * ks + 8 * grp]));
        s[sub][0] = mfma16(kf, qf[0][ks], s[sub][0]);
        s[sub][1] = mfma16(kf, qf[1][ks], s[sub][1]);
      }
    }

    if (need_mask) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int ti = tok[cb];
        const int lo = (W > 0) ? ti - W + 1 : -0x7fffffff;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + sub * 16 + 4 * grp + r;
            if (j > ti || j < lo) s[sub][cb][r] = kNegInf;
          }
      }
    }

    // -- online softmax (base 2) and P in bf16 ----------------------------
    bf16x8 pb[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float mx = fmaxf(fmaxf(fmaxf(s[0][cb][0], s[0][cb][1]), fmaxf(s[0][cb][2], s[0][cb][3])),
                       fmaxf(fmaxf(s[1][cb][0], s[1][cb][1]), fmaxf(s[1][cb][2], s[1][cb][3])));
      mx = max_across_groups(mx) * c2;   // base-2 units
      const float mn = fmaxf(m[cb], mx);
      const float ms = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[cb] - ms);
      float p[8];
      float ps = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[sub * 4 + r] = fast_exp2(fmaf(s[sub][cb][r], c2, -ms));
          ps += p[sub * 4 + r];
        }
      l[cb] = l[cb] * alpha + ps;
      m[cb] = mn;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[cb][t] *= alpha;
      pb[cb] = as_bf16x8(pack8(p));
    }

    // -- O^T += V^T . P^T --------------------------------------------------
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 vf = as_bf16x8(ld16(&svt[(16 * t + c) * VSTR + 8 * grp]));
      acc[0][t] = mfma16(vf, pb[0], acc[0][t]);
      acc[1][t] = mfma16(vf, pb[1], acc[1][t]);
    }
  }

  // ---- epilogue: o = O / l, rounded to bf16 -----------------------------
  float lt[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) lt[cb] = sum_across_groups(l[cb]);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    if (!rv[cb]) continue;
    const float inv = (lt[cb] > 0.f) ? 1.f / lt[cb] : 0.f;
    bf16_t* orow = Op + ((tokbase + tok[cb]) * a.hq + head[cb]) * DV + 4 * grp;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint2 w = make_uint2(pack_bf16x2(acc[cb][t][0] * inv, acc[cb][t][1] * inv),
                                 pack_bf16x2(acc[cb][t][2] * inv, acc[cb][t][3] * inv));
      st8(orow + 16 * t, w);
    }
  }
}

bool prefill_bf16_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && G >= 1 && G <= ROWS && (G & (G - 1)) == 0 &&
         (a.half % 32) == 0 && 2 * a.half <= D;
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  int log2g = 0;
  while ((1 << log2g) < G) ++log2g;
  const int T = ROWS >> log2g;
  const int nblk = (a.n + T - 1) / T;
  const long long total = (long long)a.B * a.hkv * nblk;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int balance = (a.window <= 0 || a.window >= a.n) ? 1 : 0;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)total), dim3(NTHREADS), 0, stream, a,
                     log2g, nblk, balance);
  return hipGetLastError();
}

}  // namespace hswa
