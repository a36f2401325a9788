// Single-token decode over an FP8 (OCP E4M3) KV cache on the gfx950 matrix
// cores.
//
// Quantised KV storage: "MiMo v2.5 inference optimisation" (youngju.dev),
// closing section: a cache already narrowed by the window can also be kept
// in FP8, the two savings stack; "MiMo-V3 HySparse2" (aideepthink.cn),
// section 5, states its KV-cache sizes in FP8.  Entry j of kv head g holds an
// E4M3 code x; its value is e4m3(x) * k_scale[g] for K and e4m3(x) *
// v_scale[g] for V.
//
// The split-K structure is the bf16 decode's: a workgroup owns (sequence b,
// four neighbouring kv heads, split s), streams its keys in tiles of 16 with
// global_load_lds and leaves an unnormalised partial (m, l, O) per split
// for the shared combine kernel, which adds the sink once.  Each tile is half
// the bytes.  E4M3 values are exact in bf16 (3 mantissa bits, exponents
// 2^-9 .. 2^8), so the matrix-core products stay bf16 x bf16 with fp32
// accumulation and the cache values enter them unrounded:
//  * K: a lane reads the 8 codes of its operand slot from LDS and widens them
//    in registers (hardware E4M3 -> fp32 conversion, upper halves packed);
//  * V: the PV product needs V transposed (a lane holds 4 keys of one dim),
//    so each wavefront first widens its own head's 16 x 128 codes into a
//    bf16 copy in LDS laid out like the bf16 kernel's V tile, then reads it
//    with the same transposed reads.
// The scales enter in fp32: k_scale multiplies the raw score (folded into
// the base-2 factor), v_scale the split's partial output.
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
constexpr int BK = 16;                      // keys per tile
constexpr int HG = 4;                       // kv heads per workgroup (one per wavefront)
constexpr int KROW8 = HG * D;               // 768 B: the group's K codes of one cache row
constexpr int VROW8 = HG * DV;              // 512 B: its V codes
constexpr int VROWB = HG * DV * 2;          // 1024 B: the widened (bf16) V row
constexpr int KTILE8 = BK * KROW8;          // 12 KB
constexpr int VTILE8 = BK * VROW8;          // 8 KB
constexpr int VTILEB = BK * VROWB;          // 16 KB
constexpr int KINSTR = KTILE8 / 1024;       // 12 load instructions of 1 KB
constexpr int VINSTR = VTILE8 / 1024;       // 8
constexpr int DMA_PER_WAVE = (KINSTR + VINSTR) / HG;   // 5
static_assert(KINSTR % HG == 0 && VINSTR % HG == 0, "even split of the loads");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

}  // namespace

__global__ __launch_bounds__(256, 2) void decode_fp8_split_kernel(AttnArgs a, int layout) {
  __shared__ __attribute__((aligned(16))) unsigned char kst0[KTILE8];
  __shared__ __attribute__((aligned(16))) unsigned char vst0[VTILE8];
  __shared__ __attribute__((aligned(16))) unsigned char kst1[KTILE8];
  __shared__ __attribute__((aligned(16))) unsigned char vst1[VTILE8];
  __shared__ __attribute__((aligned(16))) unsigned char vwide[VTILEB];
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
  // K stage (ii < 12, ii' = ii) or the V stage (ii' = ii - 12).  K slot s is
  // row s / 48, physical chunk pc = s % 48 holding logical chunk pc ^ row%16
  // (XOR on the low four bits: within its aligned 256 B); V slot s is row
  // s / 32, physical chunk pc = s % 32 holding logical chunk pc ^ row%8
  // (within its head's aligned 128 B).  Rows past the split reload its last
  // key (masked later).
  const unsigned char* kbase = static_cast<const unsigned char*>(a.k) +
                               ((row0 + ks0) * a.hkv + HG * gx) * (long long)D;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) +
                               ((row0 + ks0) * a.hkv + HG * gx) * (long long)DV;
  const int kstride = a.hkv * D, vstride = a.hkv * DV;   // bytes per cache row
  int drow[DMA_PER_WAVE], doff[DMA_PER_WAVE];
#pragma unroll
  for (int u = 0; u < DMA_PER_WAVE; ++u) {
    const int ii = wave + HG * u;
    if (ii < KINSTR) {
      const int sl = 64 * ii + lane;
      const int row = sl / 48, pc = sl - row * 48;
      drow[u] = row;
      doff[u] = 16 * (pc ^ (row & 15));
    } else {
      const int sl = 64 * (ii - KINSTR) + lane;
      const int row = sl >> 5, pc = sl & 31;
      drow[u] = row;
      doff[u] = 16 * (pc ^ (row & 7));
    }
  }
  auto issue = [&](int k0, unsigned char* kd, unsigned char* vd) {
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int ii = wave + HG * u;
      const int key = min(k0 + drow[u], nkeys - 1);
      if (u < KINSTR / HG)   // wave-uniform: the first three instructions are K, the rest V
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kbase + (__umul24(key, kstride) + doff[u])),
                                         (lds_void_t*)(kd + 1024 * ii), 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vbase + (__umul24(key, vstride) + doff[u])),
                                         (lds_void_t*)(vd + 1024 * (ii - KINSTR)), 16, 0, 0);
    }
  };
  static_assert(KINSTR / HG == 3, "the K/V split of a wavefront's loads");

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
  const float kscale = a.kscale[g], vscale = a.vscale[g];
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): q and tile 0 have landed

  const float c2 = a.scale * kLog2e * kscale;   // raw code score -> base-2 units
  float m = kNegInf, l = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets: K row c; the transposed V read of lane (c, grp):
  // row 4 grp + c/4, bytes 8 (c%4) of the logical 32-byte unit 8 wave + tt.
  // Widening: lane (c, grp) converts key c's 16-code chunks 2 grp and
  // 2 grp + 1 of head `wave` (dims 32 grp .. 32 grp + 31).
  const int krow = c * KROW8;
  const int vr = 4 * grp + (c >> 2);
  const int vrow = vr * VROWB + 8 * (c & 3);

  auto tile = [&](int t, const unsigned char* kc, const unsigned char* vc, unsigned char* kn,
                  unsigned char* vn) __attribute__((always_inline)) {
    // Tile t's loads are this wavefront's only ones in flight.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();   // every wavefront's share of tile t has landed; tile t-1 is consumed
    if (t + 1 < ntile) issue((t + 1) * BK, kn, vn);
    // widen this wavefront's V stripe; LDS operations of a wavefront complete
    // in order, so its transposed reads below see these writes
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int unit = 8 * wave + 2 * grp + j;
      const uint4 codes = ld16(vc + c * VROW8 + 16 * (unit ^ (c & 7)));
      unsigned char* dst = vwide + c * VROWB + 32 * (unit ^ (c & 7));
      st16(dst, widen8(make_uint2(codes.x, codes.y)));
      st16(dst + 16, widen8(make_uint2(codes.z, codes.w)));
    }
    const int k0 = t * BK;
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // dims 32 ks + 8 grp .. + 7: logical 16-byte chunk 12 wave + 2 ks + grp/2, half grp%2
      const int lc = 12 * wave + 2 * ks + (grp >> 1);
      const uint2 w = *reinterpret_cast<const uint2*>(kc + krow + 16 * (lc ^ c) + 8 * (grp & 1));
      sc = mfma16(as_bf16x8(widen8(w)), qf[ks], sc);
    }
    // Branch-free on purpose (MFMA result read by the VALU right after).
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
    const v4i16_t pb = __builtin_bit_cast(v4i16_t, pk);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint2 vt = lds_tr4(vwide + vrow + 32 * ((8 * wave + tt) ^ (vr & 7)));
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16_t, vt), pb,
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
          make_float4(acc[tt][0] * vscale, acc[tt][1] * vscale, acc[tt][2] * vscale,
                      acc[tt][3] * vscale);
    if (grp == 0) {
      float* wml = a.ws + (long long)a.B * a.hq * a.nsplit * DV + idx * 2;
      wml[0] = m;
      wml[1] = l;
    }
  }
}

bool decode_fp8_supported(const AttnArgs& a) { return decode_bf16_supported(a); }

hipError_t launch_decode_fp8(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  hipError_t e = launch_decode_rope_q(a, layout, stream);
  if (e != hipSuccess) return e;
  dim3 g1((unsigned)(a.hkv / HG), (unsigned)a.nsplit, (unsigned)a.B);
  hipLaunchKernelGGL(decode_fp8_split_kernel, g1, dim3(256), 0, stream, a, layout);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, layout, stream);
}

}  // namespace hswa
