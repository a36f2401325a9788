// bf16 single-token decode on the gfx950 matrix cores.
//
// One new query token per sequence attends to its KV cache: the W-slot ring
// of an SWA layer or the contiguous prefix of a GA layer ("MiMo v2.5
// inference optimisation" (youngju.dev): dual-pool KV cache, the SWA pool
// bounded by the window, the full-attention pool growing with the
// sequence).  Decode reads the whole cache once per step, so the kernel is a
// stream over K and V at HBM rate.
//
// Split-K.  A wavefront owns (sequence b, kv head g, split s) and reads
// `split_keys` consecutive keys of that sequence.  Its G query heads form
// the N side of 16x16x32 MFMAs (S^T = K . Q^T, then O^T += V^T . P^T, as in
// the prefill kernel).  K fragments are loaded straight from HBM into the A
// operand layout; V goes through a small LDS transpose.  Each split leaves
// an unnormalised partial (m, l, O) in base 2 in the workspace.
//
// Combine.  Per (b, h): M = max(sink, m_s), denominator
// exp2(sink - M) + sum_s exp2(m_s - M) l_s, output sum_s exp2(m_s - M) O_s
// over that denominator: the sink term of "MiMo-V2-Flash: Hybrid Sliding
// Window Attention Architecture" (rslog.cc) section 4.4 enters exactly once.
#include <math.h>

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

// Rotate q (KS k-steps of 8 values, pair (ka, ka + PK) in lane) to position
// p; angles are formed and evaluated in fp64 (p reaches 2.6e5 rad here).
template <int PK>
__device__ __forceinline__ void rotate_q_at(float (&f)[KS][8], long long p, double theta, int half,
                                            int grp) {
#pragma unroll
  for (int ka = 0; ka < PK; ++ka) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 32 * ka + 8 * grp + e;
      const double ang = (double)p * pow(theta, -(double)r / (double)half);
      double sd, cd;
      sincos(ang, &sd, &cd);
      const float cs = (float)cd, sn = (float)sd;
      const float x0 = f[ka][e], x1 = f[ka + PK][e];
      f[ka][e] = x0 * cs - x1 * sn;
      f[ka + PK][e] = x1 * cs + x0 * sn;
    }
  }
}

// Key range of sequence b: `len` keys, key t is cache row `row0 + t`.
// Returns false for a position the caller's contract rules out.
__device__ __forceinline__ bool key_range(const AttnArgs& a, int layout, int b, long long* p_out,
                                          long long* row0, long long* len) {
  const long long p = a.pos[b];
  *p_out = p;
  if (p < 0 || p > a.max_pos) return false;
  if (layout == 0) {  // ring: slots 0 .. min(p, W-1) hold tokens
    *row0 = (long long)b * a.window;
    *len = (p + 1 < a.window) ? p + 1 : a.window;
    return true;
  }
  const long long off = a.seq_offsets[b];
  const long long rows = a.seq_offsets[b + 1] - off;
  if (p >= rows) return false;
  const long long lo = (a.window > 0 && p - a.window + 1 > 0) ? p - a.window + 1 : 0;
  *row0 = off + lo;
  *len = p - lo + 1;
  return true;
}

}  // namespace

__global__ __launch_bounds__(64) void decode_split_kernel(AttnArgs a, int layout) {
  __shared__ __attribute__((aligned(16))) bf16_t svt[DV * VSTR];
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, c = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;

  long long p, row0, len;
  if (!key_range(a, layout, b, &p, &row0, &len)) return;
  const long long ks0 = (long long)s * a.split_keys;
  if (ks0 >= len) return;
  const long long ks1 = (ks0 + a.split_keys < len) ? ks0 + a.split_keys : len;

  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ Vp = static_cast<const bf16_t*>(a.v);

  // q of head g*G + c at position p (columns c >= G are padding).
  bf16x8 qf[KS];
  {
    float f[KS][8];
    if (c < G) {
      const bf16_t* qrow =
          static_cast<const bf16_t*>(a.q) + ((long long)b * a.hq + g * G + c) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) unpack8(ld16(qrow + 32 * ks), f[ks]);
      switch (a.half >> 5) {
        case 0: break;
        case 1: rotate_q_at<1>(f, p, a.rope_theta, a.half, grp); break;
        case 2: rotate_q_at<2>(f, p, a.rope_theta, a.half, grp); break;
        default: rotate_q_at<3>(f, p, a.rope_theta, a.half, grp); break;
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) f[ks][e] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(pack8(f[ks]));
  }

  const float c2 = a.scale * kLog2e;   // raw score -> base-2 units
  float m = kNegInf, l = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (long long t0 = ks0; t0 < ks1; t0 += BK) {
    // K fragments for keys t0 + sub*16 + c, straight from HBM.
    uint4 kr[2][KS];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const long long key = t0 + sub * 16 + c;
      if (key < ks1) {
        const bf16_t* kp = Kp + ((row0 + key) * a.hkv + g) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kr[sub][ks] = ld16(kp + 32 * ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kr[sub][ks] = make_uint4(0, 0, 0, 0);
      }
    }
    // V rows for the transpose: lane owns two (key quad, 8-dim chunk) units.
    uint4 vr[2][4];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int u = lane + 64 * w;
      const int kq = u & 7, dc = u >> 3;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const long long key = t0 + 4 * kq + q4;
        vr[w][q4] = (key < ks1) ? ld16(Vp + ((row0 + key) * a.hkv + g) * DV + 8 * dc)
                                : make_uint4(0, 0, 0, 0);
      }
    }

    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc[0] = mfma16(as_bf16x8(kr[0][ks]), qf[ks], sc[0]);
      sc[1] = mfma16(as_bf16x8(kr[1][ks]), qf[ks], sc[1]);
    }
    if (t0 + BK > ks1) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + sub * 16 + 4 * grp + r >= ks1) sc[sub][r] = kNegInf;
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

    __syncthreads();  // previous tile's V^T reads are done
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

  l = sum_across_groups(l);
  if (c < G) {
    const long long idx = ((long long)b * a.hq + g * G + c) * a.nsplit + s;
    float* wo = a.ws + idx * DV + 4 * grp;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<float4*>(wo + 16 * t) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    if (grp == 0) {
      float* wml = a.ws + (long long)a.B * a.hq * a.nsplit * DV + idx * 2;
      wml[0] = m;
      wml[1] = l;
    }
  }
}

__global__ __launch_bounds__(64) void decode_combine_kernel(AttnArgs a, int layout) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  bf16_t* orow = static_cast<bf16_t*>(a.o) + ((long long)b * a.hq + h) * DV;
  long long p, row0, len;
  if (!key_range(a, layout, b, &p, &row0, &len)) {
    const uint16_t nan_bits = 0x7fc0;
    orow[lane] = nan_bits;
    orow[lane + 64] = nan_bits;
    return;
  }
  const int nspl = (int)((len + a.split_keys - 1) / a.split_keys);
  const long long base = ((long long)b * a.hq + h) * a.nsplit;
  const float* wml = a.ws + (long long)a.B * a.hq * a.nsplit * DV + base * 2;
  const float s2 = a.sink ? a.sink[h] * kLog2e : kNegInf;
  float M = s2;
  for (int s = 0; s < nspl; ++s) M = fmaxf(M, wml[2 * s]);
  float den = (s2 > kNegInf) ? fast_exp2(s2 - M) : 0.f;
  float o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < nspl; ++s) {
    const float w = fast_exp2(wml[2 * s] - M);
    den += w * wml[2 * s + 1];
    const float* wo = a.ws + (base + s) * DV;
    o0 += w * wo[lane];
    o1 += w * wo[lane + 64];
  }
  const float inv = (den > 0.f) ? 1.f / den : 0.f;
  orow[lane] = f32_to_bf16_bits(o0 * inv);
  orow[lane + 64] = f32_to_bf16_bits(o1 * inv);
}

bool decode_bf16_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && G >= 1 && G <= 16 && (a.half % 32) == 0 &&
         2 * a.half <= D;
}

// Keys per split and splits per (sequence, kv head).  Short key sets (the
// ring) use 32-key splits so that many wavefronts share the few keys; long
// prefixes use up to 1024 keys per split, which keeps the partials small
// next to the cache.
void decode_split_plan(int layout, int window, long long max_pos, int* split_keys, int* nsplit) {
  long long lmax;
  if (layout == 0) {
    lmax = (max_pos + 1 < window) ? max_pos + 1 : window;
  } else {
    lmax = max_pos + 1;
    if (window > 0 && window < lmax) lmax = window;
  }
  if (lmax < 1) lmax = 1;
  long long sk;
  if (lmax <= 512) {
    sk = 32;
  } else {
    sk = (lmax + 63) / 64;
    sk = ((sk + 31) / 32) * 32;
    if (sk > 1024) sk = 1024;
  }
  *split_keys = (int)sk;
  *nsplit = (int)((lmax + sk - 1) / sk);
}

hipError_t launch_decode_bf16(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  dim3 g1((unsigned)a.nsplit, (unsigned)a.hkv, (unsigned)a.B);
  hipLaunchKernelGGL(decode_split_kernel, g1, dim3(64), 0, stream, a, layout);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)a.hq, (unsigned)a.B);
  hipLaunchKernelGGL(decode_combine_kernel, g2, dim3(64), 0, stream, a, layout);
  return hipGetLastError();
}

}  // namespace hswa
