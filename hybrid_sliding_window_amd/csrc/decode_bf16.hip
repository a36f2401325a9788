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
// `split_keys` consecutive keys of that sequence, 32 per tile.  The four
// wavefronts of a workgroup take four neighbouring kv heads of the same
// keys, so together they read whole cache rows ([row][kv head][dim]) rather
// than one head's stripe of each.  Its G query
// heads form the N side of 16x16x32 MFMAs (S^T = K . Q^T, then
// O^T += V^T . P^T).  K fragments go from HBM straight into registers in
// the A operand layout and V into LDS (global_load_lds), from where the PV
// product reads V^T with ds_read_b64_tr_b16.  A wavefront waits for its
// tile before computing it; the latency is hidden by occupancy instead:
// at 128 VGPRs and 9 KB of LDS each, four wavefronts per SIMD keep a tile
// each in flight while others compute.  The query arrives rotated to its
// position by a small preparation kernel, so no fp64 work (or its
// registers) sits in this one.  Each split leaves an
// unnormalised partial (m, l, O) in base 2 in the workspace.
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
constexpr int VPITCH = DV * 2 + 32;       // V row pitch in LDS (bytes): conflict-free transposed reads
constexpr int VSLOTS = VPITCH / 16;       // 18 16-byte slots per row (16 data + 2 pad)
constexpr int VINSTR = BK * VSLOTS / 64;  // 9 load instructions of 1 KB per tile
constexpr int VSTAGE = VINSTR * 1024;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

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

// q rotated to its position, once per (sequence, head): pair (d, d + R/2),
// d < R/2, turns by p * theta^(-d / (R/2)), the angle formed and evaluated
// in fp64 (p reaches 2.6e5 rad here), the rotation itself in fp32 and the
// result rounded to bf16; the other dims are copied.
__global__ __launch_bounds__(64) void decode_rope_q_kernel(AttnArgs a, int layout) {
  const int h = blockIdx.x, b = blockIdx.y;
  long long p, row0, len;
  if (!key_range(a, layout, b, &p, &row0, &len)) return;
  const bf16_t* q = static_cast<const bf16_t*>(a.q) + ((long long)b * a.hq + h) * D;
  bf16_t* qo = static_cast<bf16_t*>(a.qrot) + ((long long)b * a.hq + h) * D;
  const int half = a.half;
  for (int d = threadIdx.x; d < D; d += 64) {
    if (d < half) {
      const float x0 = bf16_to_f32(q[d]), x1 = bf16_to_f32(q[d + half]);
      const double ang = (double)p * pow(a.rope_theta, -(double)d / (double)half);
      double sd, cd;
      sincos(ang, &sd, &cd);
      const float cs = (float)cd, sn = (float)sd;
      qo[d] = f32_to_bf16_bits(x0 * cs - x1 * sn);
      qo[d + half] = f32_to_bf16_bits(x1 * cs + x0 * sn);
    } else if (d >= 2 * half) {
      qo[d] = q[d];
    }
  }
}

__global__ __launch_bounds__(256, 3) void decode_split_kernel(AttnArgs a, int layout) {
  __shared__ __attribute__((aligned(16))) unsigned char vstages[4 * VSTAGE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int g = 4 * blockIdx.x + wave, s = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, c = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;
  if (g >= a.hkv) return;   // no workgroup barrier below: wavefronts are independent
  unsigned char* vstage = vstages + wave * VSTAGE;

  long long p, row0, len;
  if (!key_range(a, layout, b, &p, &row0, &len)) return;
  const long long ks0 = (long long)s * a.split_keys;
  if (ks0 >= len) return;
  const long long ks1 = (ks0 + a.split_keys < len) ? ks0 + a.split_keys : len;
  const int ntile = (int)((ks1 - ks0 + BK - 1) / BK);

  // Split-relative addressing: the split's first row is a wave-uniform base
  // and a key's offset, below split_keys * hkv * D elements, fits 32 bits.
  const int nkeys = (int)(ks1 - ks0);
  const bf16_t* __restrict__ Kb =
      static_cast<const bf16_t*>(a.k) + ((row0 + ks0) * a.hkv + g) * (long long)D;
  const bf16_t* __restrict__ Vb =
      static_cast<const bf16_t*>(a.v) + ((row0 + ks0) * a.hkv + g) * (long long)DV;
  const int kstride = a.hkv * D, vstride = a.hkv * DV;   // elements from one key to the next

  // K fragments of the tile at key k0: keys k0 + 16 sub + c (clamped into the
  // split; the extra keys are masked), 8 dims at 32 ks + 8 grp.
  auto load_k = [&](int k0, uint4 (&kr)[2][KS]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int key = min(k0 + sub * 16 + c, nkeys - 1);
      const bf16_t* kp = Kb + (key * kstride + 8 * grp);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[sub][ks] = ld16(kp + 32 * ks);
    }
  };
  // V tile at key k0 into an LDS stage: instruction ii, lane -> slot
  // 64 ii + lane = (row / 18, chunk % 18); pad chunks reload chunk 0.
  auto load_v = [&](int k0, unsigned char* st) {
#pragma unroll
    for (int ii = 0; ii < VINSTR; ++ii) {
      const int sl = 64 * ii + lane;
      const int row = sl / VSLOTS;
      int ch = sl - row * VSLOTS;
      if (ch >= DV / 8) ch = 0;
      const int key = min(k0 + row, nkeys - 1);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(Vb + (key * vstride + 8 * ch)),
                                       (lds_void_t*)(st + 1024 * ii), 16, 0, 0);
    }
  };

  // q of head g*G + c (rotated to position p by the preparation kernel when
  // RoPE is on); columns c >= G are padding.
  bf16x8 qf[KS];
  {
    const bf16_t* qsrc = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
    const bf16_t* qrow = qsrc + ((long long)b * a.hq + g * G + min(c, G - 1)) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(c < G ? ld16(qrow + 32 * ks) : make_uint4(0, 0, 0, 0));
  }

  const float c2 = a.scale * kLog2e;   // raw score -> base-2 units
  float m = kNegInf, l = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // transpose origin of the V^T operand: key 4 grp + c / 4, column 4 (c % 4)
  const int voff = (4 * grp + (c >> 2)) * VPITCH + 8 * (c & 3);

  for (int t = 0; t < ntile; ++t) {
    const int k0 = t * BK;
    uint4 kc[2][KS];
    load_v(k0, vstage);   // the previous tile's V reads have completed
    load_k(k0, kc);
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc[0] = mfma16(as_bf16x8(kc[0][ks]), qf[ks], sc[0]);
      sc[1] = mfma16(as_bf16x8(kc[1][ks]), qf[ks], sc[1]);
    }
    if (k0 + BK > nkeys) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (k0 + sub * 16 + 4 * grp + r >= nkeys) sc[sub][r] = kNegInf;
    }

    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = max_across_groups(mx) * c2;   // base-2 units
    const float mn = fmaxf(m, mx);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    float pv[8];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[sub * 4 + r] = fast_exp2(fmaf(sc[sub][r], c2, -ms));
    const uint4 pk = pack8(pv);
    // l sums the bf16 P that weight V
    float ps = add_bf16_pair(pk.x, 0.f);
    ps = add_bf16_pair(pk.y, ps);
    ps = add_bf16_pair(pk.z, ps);
    ps = add_bf16_pair(pk.w, ps);
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] *= alpha;
    const bf16x8 pb = as_bf16x8(pk);

    // -- O^T += V^T . P^T (keys 4 grp + r and 16 + 4 grp + r, as P^T holds them)
    const unsigned char* vb = vstage + voff;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint2 lo = lds_tr4(vb + 32 * tt);
      const uint2 hi = lds_tr4(vb + 16 * VPITCH + 32 * tt);
      acc[tt] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, acc[tt]);
    }
  }

  l = sum_across_groups(l);
  if (c < G) {
    const long long idx = ((long long)b * a.hq + g * G + c) * a.nsplit + s;
    float* wo = a.ws + idx * DV + 4 * grp;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<float4*>(wo + 16 * tt) =
          make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
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
  return a.d_qk == D && a.d_v == DV && G >= 1 && G <= 16 && 2 * a.half <= D;
}

// Keys per split and splits per (sequence, kv head).  Short key sets (the
// ring) use 32-key splits so that many wavefronts share the few keys; long
// prefixes use about lmax / 64 keys per split, at most 4096, which gives a
// few wavefronts per SIMD over the batch and keeps the partials (written and
// read once) below half a percent of the cache bytes.
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
    if (sk > 4096) sk = 4096;
  }
  *split_keys = (int)sk;
  *nsplit = (int)((lmax + sk - 1) / sk);
}

hipError_t launch_decode_bf16(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  if (a.half > 0) {
    hipLaunchKernelGGL(decode_rope_q_kernel, dim3((unsigned)a.hq, (unsigned)a.B), dim3(64), 0, stream,
                       a, layout);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 g1((unsigned)((a.hkv + 3) / 4), (unsigned)a.nsplit, (unsigned)a.B);
  hipLaunchKernelGGL(decode_split_kernel, g1, dim3(256), 0, stream, a, layout);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)a.hq, (unsigned)a.B);
  hipLaunchKernelGGL(decode_combine_kernel, g2, dim3(64), 0, stream, a, layout);
  return hipGetLastError();
}

}  // namespace hswa
