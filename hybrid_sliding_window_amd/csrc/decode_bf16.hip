// bf16 single-token decode on the gfx950 matrix cores.
//
// One new query token per sequence attends to its KV cache: the W-slot ring
// of an SWA layer or the contiguous prefix of a GA layer ("MiMo v2.5
// inference optimisation" (youngju.dev): dual-pool KV cache, the SWA pool
// bounded by the window, the full-attention pool growing with the
// sequence).  Decode reads the whole cache once per step, so the kernel is a
// stream over K and V at HBM rate.
//
// Split-K.  A workgroup owns (sequence b, four neighbouring kv heads, split
// s) and reads `split_keys` consecutive keys of that sequence, 16 per tile.
// The cache rows are [row][kv head][dim], so the four heads' K (4 x 384 B)
// and V (4 x 256 B) of a row are contiguous: the workgroup streams whole
// row runs into LDS with global_load_lds, each 1 KB load instruction
// covering 1 KB of contiguous cache, and a wavefront then takes its own
// head's stripe from LDS.  Two LDS stages: tile t+1 is requested before tile
// t is computed.  Rows are stored unpadded with an XOR swizzle (applied on
// the global side of the copy) so that the MFMA operand reads hit distinct
// banks.  Per wavefront, the G query heads of its kv head form the N side of
// the MFMAs: S^T = K . Q^T on the 16x16x32 form, then O^T += V^T . P^T on
// the 16x16x16 form, whose k-index matches the key order S^T leaves in a
// lane, with V^T read by ds_read_b64_tr_b16.  Each split leaves an
// unnormalised partial (m, l, O) in base 2 in the workspace.
//
// Combine.  Per (b, h): M = max(sink, m_s), denominator
// exp2(sink - M) + sum_s exp2(m_s - M) l_s, output sum_s exp2(m_s - M) O_s
// over that denominator: the sink term of "MiMo-V2-Flash: Hybrid Sliding
// Window Attention Architecture" (rslog.cc) section 4.4 enters exactly once.
#include <math.h>

#include "common.h"
#include "decode_keys.h"
#include "launch.h"

namespace hswa {
namespace {

constexpr int D = 192;
constexpr int DV = 128;
constexpr int KS = D / 32;
constexpr int NT = DV / 16;
constexpr int BK = 16;                    // keys per tile
constexpr int HG = 4;                     // kv heads per workgroup (one per wavefront)
constexpr int KROW = HG * D * 2;          // 1536 B: the group's K of one cache row
constexpr int VROW = HG * DV * 2;         // 1024 B: its V
constexpr int KTILE = BK * KROW;          // 24 KB
constexpr int VTILE = BK * VROW;          // 16 KB
constexpr int KINSTR = KTILE / 1024;      // 24 load instructions of 1 KB
constexpr int VINSTR = VTILE / 1024;      // 16
constexpr int DMA_PER_WAVE = (KINSTR + VINSTR) / HG;   // 10
static_assert((KINSTR + VINSTR) % HG == 0 && KINSTR % HG == 0, "even split of the loads");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

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

typedef short v4i16 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256, 2) void decode_split_kernel(AttnArgs a, int layout) {
  __shared__ __attribute__((aligned(16))) unsigned char kst0[KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char vst0[VTILE];
  __shared__ __attribute__((aligned(16))) unsigned char kst1[KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char vst1[VTILE];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int gx = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int g = HG * gx + wave;
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;

  long long p, row0, len;
  if (!key_range(a, layout, b, &p, &row0, &len)) return;   // uniform over the workgroup
  const long long ks0 = (long long)s * a.split_keys;
  if (ks0 >= len) return;
  const long long ks1 = (ks0 + a.split_keys < len) ? ks0 + a.split_keys : len;
  const int nkeys = (int)(ks1 - ks0);
  const int ntile = (nkeys + BK - 1) / BK;

  // ---- this lane's 16-byte slots of a tile ------------------------------------
  // Load instruction ii = wave + 4u fills LDS bytes [1024 ii', +1024) of the
  // K stage (ii < 24, ii' = ii) or the V stage (ii' = ii - 24).  K slot s is
  // row s / 96, physical chunk pc = s % 96 holding logical chunk pc ^ row%16
  // (XOR on the low four bits, within its aligned 256 B); V slot s is row
  // s / 64, physical 32-byte unit (s % 64) / 2 holding logical unit
  // unit ^ row%8.  Rows past the split reload its last key (masked later).
  const unsigned char* kbase = static_cast<const unsigned char*>(a.k) +
                               (((row0 + ks0) * a.hkv + HG * gx) * (long long)D) * 2;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) +
                               (((row0 + ks0) * a.hkv + HG * gx) * (long long)DV) * 2;
  const int kstride = a.hkv * D * 2, vstride = a.hkv * DV * 2;   // bytes per cache row
  int drow[DMA_PER_WAVE], doff[DMA_PER_WAVE];
#pragma unroll
  for (int u = 0; u < DMA_PER_WAVE; ++u) {
    const int ii = wave + HG * u;
    if (ii < KINSTR) {
      const int sl = 64 * ii + lane;
      const int row = sl / 96, pc = sl - row * 96;
      drow[u] = row;
      doff[u] = 16 * (pc ^ (row & 15));
    } else {
      const int sl = 64 * (ii - KINSTR) + lane;
      const int row = sl >> 6, pc = sl & 63;
      drow[u] = row;
      doff[u] = 32 * ((pc >> 1) ^ (row & 7)) + 16 * (pc & 1);
    }
  }
  // Addresses are a wave-uniform base plus a 32-bit per-lane offset (a
  // split spans at most split_keys * hkv * 384 bytes, and key and row
  // stride both fit 24 bits), the saddr form of the load: one 24-bit
  // multiply-add per instruction.
  auto issue = [&](int k0, unsigned char* kd, unsigned char* vd) {
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int ii = wave + HG * u;
      const int key = min(k0 + drow[u], nkeys - 1);
      if (u < KINSTR / HG)   // wave-uniform: the first six instructions are K, the rest V
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kbase + (__umul24(key, kstride) + doff[u])),
                                         (lds_void_t*)(kd + 1024 * ii), 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vbase + (__umul24(key, vstride) + doff[u])),
                                         (lds_void_t*)(vd + 1024 * (ii - KINSTR)), 16, 0, 0);
    }
  };
  static_assert(KINSTR / HG == 6, "the K/V split of a wavefront's loads");

  issue(0, kst0, vst0);

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
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): q and tile 0 have landed

  const float c2 = a.scale * kLog2e;   // raw score -> base-2 units
  float m = kNegInf, l = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets: K row c, logical chunk 24 wave + 4 ks + grp; the
  // transposed V read of lane (c, grp): row 4 grp + c/4, bytes 8 (c%4) of the
  // logical 32-byte unit 8 wave + tt
  const int krow = c * KROW;
  const int vr = 4 * grp + (c >> 2);
  const int vrow = vr * VROW + 8 * (c & 3);

  auto tile = [&](int t, const unsigned char* kc, const unsigned char* vc, unsigned char* kn,
                  unsigned char* vn) __attribute__((always_inline)) {
    // Tile t's loads are this wavefront's only ones in flight.  The wait is
    // explicit: the compiler does not reliably carry a pending LDS-DMA
    // write across the loop back-edge into the barrier's fence.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();   // every wavefront's share of tile t has landed; tile t-1 is consumed
    if (t + 1 < ntile) issue((t + 1) * BK, kn, vn);
    const int k0 = t * BK;
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int q = 24 * wave + 4 * ks + grp;
      sc = mfma16(as_bf16x8(ld16(kc + krow + 16 * (q ^ c))), qf[ks], sc);
    }
    // Branch-free on purpose: the first VALU read of an MFMA result needs
    // wait states after it, and with a branch between them the compiler
    // did not insert them on the path that skips the branch body.
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (k0 + 4 * grp + r < nkeys) ? sc[r] : kNegInf;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_across_groups(mx) * c2;   // base-2 units
    const float mn = fmaxf(m, mx);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(fmaf(sc[r], c2, -ms));
    const uint2 pk = make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
    // l sums the bf16 P that weight V
    l = l * alpha + add_bf16_pair(pk.y, add_bf16_pair(pk.x, 0.f));
    m = mn;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] *= alpha;
    const v4i16 pb = __builtin_bit_cast(v4i16, pk);
    // -- O^T += V^T . P^T: lane (c, grp) holds keys 4 grp + r, the k-index of
    //    the 16x16x16 form; the transposed read gives V[4 grp + r][16 tt + c]
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint2 vt = lds_tr4(vc + vrow + 32 * ((8 * wave + tt) ^ (vr & 7)));
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, vt), pb,
                                                         acc[tt], 0, 0, 0);
    }
  };

  int t = 0;
  for (; t + 2 <= ntile; t += 2) {
    tile(t, kst0, vst0, kst1, vst1);
    tile(t + 1, kst1, vst1, kst0, vst0);
  }
  if (t < ntile) tile(t, kst0, vst0, kst1, vst1);

  l = sum_across_groups(l);
  if (g < a.hkv && c < G) {
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
  return a.d_qk == D && a.d_v == DV && G >= 1 && G <= 16 && a.hkv % HG == 0 && 2 * a.half <= D;
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

hipError_t launch_decode_rope_q(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0 || a.half == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_rope_q_kernel, dim3((unsigned)a.hq, (unsigned)a.B), dim3(64), 0, stream,
                     a, layout);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  dim3 g2((unsigned)a.hq, (unsigned)a.B);
  hipLaunchKernelGGL(decode_combine_kernel, g2, dim3(64), 0, stream, a, layout);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  hipError_t e = launch_decode_rope_q(a, layout, stream);
  if (e != hipSuccess) return e;
  dim3 g1((unsigned)(a.hkv / HG), (unsigned)a.nsplit, (unsigned)a.B);
  hipLaunchKernelGGL(decode_split_kernel, g1, dim3(256), 0, stream, a, layout);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, layout, stream);
}

}  // namespace hswa
