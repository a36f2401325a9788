// bf16 token-level sparse attention with a sink on the gfx950 matrix cores.
//
// "MiMo-V3 HySparse2" (aideepthink.cn), section 4: a forced-recent window
// of the latest tokens (128) plus up to 1024 tokens selected outside it,
// merged into one sparse attention over a single shared KV cache.  The
// softmax is the sink form of "MiMo-V2-Flash: Hybrid Sliding Window
// Attention Architecture" (rslog.cc) section 4.4.
//
// A wavefront owns one (batch b, query i, kv head g): its G <= 16 query
// heads are the N side of 16x16x32 MFMAs over the gathered keys.  The key
// list is the selected indices followed by the recent window; lanes 0..31
// resolve the 32 key rows of a tile and hand them to the other lanes with
// cross-lane reads.  K rows are gathered straight into A-operand registers
// (their rotated dims from the copy rotated once per call), V rows through a
// small LDS transpose.
// Workgroups are remapped so that consecutive queries of one kv head run on
// one XCD and share the recent window in its L2.
//
// The FP8 instantiation reads K/V as E4M3 codes (8 codes per operand slot,
// widened exactly to bf16 in registers); the rotated dims come from the copy
// rotated once per call from the codes' values.  k_scale multiplies the
// score, v_scale the output.
#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

constexpr int D = 192;
constexpr int DV = 128;
constexpr int KS = D / 32;
constexpr int NT = DV / 16;
constexpr int BK = 32;
constexpr int VSTR = BK + 8;

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Rotate KS k-steps of 8 values held by one lane (pair (ka, ka + PK)).
template <int PK>
__device__ __forceinline__ void rotate_frag(float (&f)[KS][8], const float2* __restrict__ trow,
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

__device__ __forceinline__ void rotate_any(float (&f)[KS][8], const float2* trow, int half,
                                           int grp) {
  switch (half >> 5) {
    case 0: break;
    case 1: rotate_frag<1>(f, trow, grp); break;
    case 2: rotate_frag<2>(f, trow, grp); break;
    default: rotate_frag<3>(f, trow, grp); break;
  }
}

}  // namespace

// FP8: K/V are E4M3 codes; NR (FP8 only): k-steps inside the rotated dims
// (R / 32, a compile-time constant so that every gather of a tile is issued
// before the first is used).
template <bool FP8, int NR>
__device__ __forceinline__ void sparse_attn(const AttnArgs& a, bf16_t* svt) {
  const int lane = threadIdx.x, c = lane & 15, grp = lane >> 4;
  const int n = a.n;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int i = logical % n;
  const int bg = logical / n;
  const int g = bg % a.hkv, b = bg / a.hkv;
  const int G = a.hq / a.hkv;
  const long long tokbase = (long long)b * n;

  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ Vp = static_cast<const bf16_t*>(a.v);
  const uint8_t* __restrict__ Kc = static_cast<const uint8_t*>(a.k);   // E4M3 codes (FP8)
  const uint8_t* __restrict__ Vc = static_cast<const uint8_t*>(a.v);
  const bf16_t* __restrict__ Kr = static_cast<const bf16_t*>(a.krot);
  const int R = 2 * a.half;

  // q of head g*G + c, rotated at position i and rounded once to bf16.
  bf16x8 qf[KS];
  {
    float f[KS][8];
    if (c < G) {
      const bf16_t* qrow =
          static_cast<const bf16_t*>(a.q) + ((tokbase + i) * a.hq + g * G + c) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) unpack8(ld16(qrow + 32 * ks), f[ks]);
      if (a.half > 0) rotate_any(f, a.rope + (long long)i * a.half, a.half, grp);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) f[ks][e] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(pack8(f[ks]));
  }

  const float c2 = a.scale * kLog2e * (FP8 ? a.kscale[g] : 1.f);   // raw score -> base-2 units
  const float s2 = (c < G && a.sink) ? a.sink[g * G + c] * kLog2e : kNegInf;
  float m = s2;
  float l = (grp == 0 && s2 > kNegInf) ? 1.f : 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const long long li = (tokbase + i) * a.hkv + g;
  int cnt = a.sel_count[li];
  cnt = cnt < 0 ? 0 : (cnt > a.max_sel ? a.max_sel : cnt);
  const int* __restrict__ sel = a.sel_idx + li * a.max_sel;
  const int rlo = (i - a.recent + 1 > 0) ? i - a.recent + 1 : 0;
  const int total = cnt + (i - rlo + 1);
  const int sel_hi = i - a.recent;     // largest admissible selected index

  for (int t0 = 0; t0 < total; t0 += BK) {
    // token index of key t0 + (lane & 31); -1 marks no key
    int myj = -1;
    {
      const int t = t0 + (lane & 31);
      if (t < cnt) {
        const int jj = sel[t];
        myj = (jj >= 0 && jj <= sel_hi) ? jj : -1;
      } else if (t < total) {
        myj = rlo + (t - cnt);
      }
    }
    // K rows straight into A-operand registers; k-steps inside the rotated
    // dims come from the rotated copy made once per call.
    uint4 kr[2][KS];
    uint4 vr[2][4];
    if (FP8) {
      // every gather first (codes of the unrotated k-steps, rotated bf16 dims,
      // V codes), then the widening
      uint2 k8[2][KS], v8[2][4];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int j = __shfl(myj, sub * 16 + c);
        const long long row = (tokbase + (j >= 0 ? j : 0)) * a.hkv + g;
        const bf16_t* kq = Kr + row * (32 * NR) + 8 * grp;
        const uint8_t* kp = Kc + row * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks < NR) kr[sub][ks] = (j >= 0) ? ld16(kq + 32 * ks) : make_uint4(0, 0, 0, 0);
          else k8[sub][ks] = (j >= 0) ? *reinterpret_cast<const uint2*>(kp + 32 * ks)
                                      : make_uint2(0, 0);
        }
      }
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int u = lane + 64 * w;
        const int kq = u & 7, dc = u >> 3;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int j = __shfl(myj, 4 * kq + q4);
          const long long vo = ((tokbase + (j >= 0 ? j : 0)) * a.hkv + g) * DV + 8 * dc;
          v8[w][q4] = (j >= 0) ? *reinterpret_cast<const uint2*>(Vc + vo) : make_uint2(0, 0);
        }
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int ks = NR; ks < KS; ++ks) kr[sub][ks] = widen8(k8[sub][ks]);
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) vr[w][q4] = widen8(v8[w][q4]);
    } else {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int j = __shfl(myj, sub * 16 + c);
        if (j >= 0) {
          const long long row = (tokbase + j) * a.hkv + g;
          const bf16_t* kq = Kr + row * R + 8 * grp;
          const bf16_t* kp = Kp + row * D + 8 * grp;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kr[sub][ks] = ld16((32 * ks < R) ? kq + 32 * ks : kp + 32 * ks);
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) kr[sub][ks] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int u = lane + 64 * w;
        const int kq = u & 7, dc = u >> 3;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int j = __shfl(myj, 4 * kq + q4);
          vr[w][q4] = (j >= 0) ? ld16(Vp + ((tokbase + j) * a.hkv + g) * DV + 8 * dc)
                               : make_uint4(0, 0, 0, 0);
        }
      }
    }

    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc[0] = mfma16(as_bf16x8(kr[0][ks]), qf[ks], sc[0]);
      sc[1] = mfma16(as_bf16x8(kr[1][ks]), qf[ks], sc[1]);
    }
    // keys without a row: the lane holding key (sub, 4*grp + r) asks its owner
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jr = __shfl(myj, sub * 16 + 4 * grp + r);
        if (jr < 0) sc[sub][r] = kNegInf;
      }

    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = max_across_groups(mx) * c2;   // base-2 units
    const float mn = fmaxf(m, mx);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    float pv[8];
    float ps = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[sub * 4 + r] = fast_exp2(fmaf(sc[sub][r], c2, -ms));
        ps += pv[sub * 4 + r];
      }
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] *= alpha;
    const bf16x8 pb = as_bf16x8(pack8(pv));

    __syncthreads();
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int u = lane + 64 * w;
      const int kq = u & 7, dc = u >> 3;
      const int pos0 = 8 * (kq & 3) + 4 * (kq >> 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = half16(vr[w][0], e) | (half16(vr[w][1], e) << 16);
        const uint32_t w1 = half16(vr[w][2], e) | (half16(vr[w][3], e) << 16);
        st8(&svt[(8 * dc + e) * VSTR + pos0], make_uint2(w0, w1));
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 vf = as_bf16x8(ld16(&svt[(16 * t + c) * VSTR + 8 * grp]));
      acc[t] = mfma16(vf, pb, acc[t]);
    }
  }

  const float lt = sum_across_groups(l);
  if (c < G) {
    const float inv = (lt > 0.f) ? (FP8 ? a.vscale[g] : 1.f) / lt : 0.f;
    bf16_t* orow = static_cast<bf16_t*>(a.o) + ((tokbase + i) * a.hq + g * G + c) * DV + 4 * grp;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint2 w = make_uint2(pack_bf16x2(acc[t][0] * inv, acc[t][1] * inv),
                                 pack_bf16x2(acc[t][2] * inv, acc[t][3] * inv));
      st8(orow + 16 * t, w);
    }
  }
}

__global__ __launch_bounds__(64) void sparse_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t svt[DV * VSTR];
  sparse_attn<false, 0>(a, svt);
}

// NR: rotated k-steps (rotary half-width 0 or 32)
template <int NR>
__global__ __launch_bounds__(64) void sparse_fp8_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t svt[DV * VSTR];
  sparse_attn<true, NR>(a, svt);
}

bool sparse_bf16_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && G >= 1 && G <= 16 && (a.half % 32) == 0 &&
         2 * a.half <= D;
}

hipError_t launch_sparse_bf16(const AttnArgs& a, hipStream_t stream) {
  const long long total = (long long)a.B * a.hkv * a.n;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(sparse_bf16_kernel, dim3((unsigned)total), dim3(64), 0, stream, a);
  return hipGetLastError();
}

bool sparse_fp8_supported(const AttnArgs& a) {
  return sparse_bf16_supported(a) && (a.half == 0 || a.half == 32);
}

hipError_t launch_sparse_fp8(const AttnArgs& a, hipStream_t stream) {
  const long long total = (long long)a.B * a.hkv * a.n;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.half == 0)
    hipLaunchKernelGGL(sparse_fp8_kernel<0>, dim3((unsigned)total), dim3(64), 0, stream, a);
  else if (a.half == 32)
    hipLaunchKernelGGL(sparse_fp8_kernel<2>, dim3((unsigned)total), dim3(64), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hswa
