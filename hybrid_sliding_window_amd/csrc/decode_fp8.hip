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
static_assert(KS == 6, "six k-steps of 32 dims");
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

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// The widened V codes of two 16-code chunks (32 bytes each at a[0], a[1])
// written to LDS in asm: a plain LDS store makes the compiler wait for every
// copy in flight first (it orders the store after all pending LDS writes).
__device__ __forceinline__ void lds_st_wide(const uint32_t (&a)[2], const u32x4_t (&w)[4]) {
  asm volatile(
      "ds_write_b128 %0, %2\n\t"
      "ds_write_b128 %0, %3 offset:16\n\t"
      "ds_write_b128 %1, %4\n\t"
      "ds_write_b128 %1, %5 offset:16"
      :
      : "v"(a[0]), "v"(a[1]), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3])
      : "memory");
}

// A workgroup of 8 wavefronts takes two consecutive splits s = 2 sp and
// 2 sp + 1 of one (sequence, group of four kv heads): wavefront w computes
// head w % 4 of split 2 sp + w / 4.  Only wavefronts 0..3 (one per SIMD)
// issue copies, those of both splits (ten per tile): a wavefront stalls
// while the vector-memory path accepts its copies, and the other wavefront
// of its SIMD, which issues none, computes meanwhile.  Three LDS stages per
// split: tile t + 2 is requested while tile t is computed, so two tiles
// (40 KB per split) of loads stay in flight.
constexpr int NST = 3;
constexpr int SPW = 2;   // splits per workgroup
__global__ __launch_bounds__(64 * HG * SPW, 1) void decode_fp8_split_kernel(AttnArgs a, int layout) {
  __shared__ __attribute__((aligned(16))) unsigned char kst[SPW][NST][KTILE8];
  __shared__ __attribute__((aligned(16))) unsigned char vst[SPW][NST][VTILE8];
  __shared__ __attribute__((aligned(16))) unsigned char vwide_all[SPW][VTILEB];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int wave = wv & (HG - 1);                            // head within the group
  const int half = wv / HG;                                  // which of the two splits
  const bool producer = half == 0;
  const int gx = blockIdx.x, b = blockIdx.z;
  const int g = HG * gx + wave;
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;
  unsigned char* vwide = vwide_all[half];

  long long p, row0, len;
  if (!key_range(a, layout, b, &p, &row0, &len)) return;   // uniform over the workgroup
  // keys of split 2 sp + h: [ks0[h], ks0[h] + nk[h]); the second may be empty
  long long ks0[SPW];
  int nk[SPW];
#pragma unroll
  for (int h = 0; h < SPW; ++h) {
    ks0[h] = (long long)(SPW * blockIdx.y + h) * a.split_keys;
    const long long e = (ks0[h] + a.split_keys < len) ? ks0[h] + a.split_keys : len;
    nk[h] = (e > ks0[h]) ? (int)(e - ks0[h]) : 0;
  }
  if (nk[0] == 0) return;   // uniform: the second split starts later still
  const int ntile = (nk[0] + BK - 1) / BK;                 // steps of the loop (the longer split)
  const int my_nk = nk[half];
  const int my_ntile = (my_nk + BK - 1) / BK;

  // ---- the 16-byte slots of a tile a producer copies ------------------------
  // Load instruction ii = wave + 4u fills LDS bytes [1024 ii', +1024) of the
  // K stage (ii < 12, ii' = ii) or the V stage (ii' = ii - 12).  K slot s is
  // row s / 48, physical chunk pc = s % 48 holding logical chunk pc ^ row%16
  // (XOR on the low four bits: within its aligned 256 B); V slot s is row
  // s / 32, physical chunk pc = s % 32 holding logical chunk pc ^ row%8
  // (within its head's aligned 128 B).  Rows past a split reload its last
  // key (masked later); an empty second split reloads the first one's rows
  // (never read).
  const unsigned char* kbase[SPW];
  const unsigned char* vbase[SPW];
  int lastkey[SPW];
#pragma unroll
  for (int h = 0; h < SPW; ++h) {
    const int hh = (nk[h] > 0) ? h : 0;
    kbase[h] = static_cast<const unsigned char*>(a.k) + ((row0 + ks0[hh]) * a.hkv + HG * gx) * (long long)D;
    vbase[h] = static_cast<const unsigned char*>(a.v) + ((row0 + ks0[hh]) * a.hkv + HG * gx) * (long long)DV;
    lastkey[h] = nk[hh] - 1;
  }
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
  // the copies of tile t of both splits into stage st (producers only)
  auto issue = [&](int t, int st) {
#pragma unroll
    for (int h = 0; h < SPW; ++h) {
#pragma unroll
      for (int u = 0; u < DMA_PER_WAVE; ++u) {
        const int ii = wave + HG * u;
        const int key = min(t * BK + drow[u], lastkey[h]);
        if (u < KINSTR / HG)   // wave-uniform: the first three instructions are K, the rest V
          __builtin_amdgcn_global_load_lds(
              (glb_void_t*)(kbase[h] + (__umul24(key, kstride) + doff[u])),
              (lds_void_t*)(kst[h][st] + 1024 * ii), 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(
              (glb_void_t*)(vbase[h] + (__umul24(key, vstride) + doff[u])),
              (lds_void_t*)(vst[h][st] + 1024 * (ii - KINSTR)), 16, 0, 0);
      }
    }
  };
  static_assert(KINSTR / HG == 3, "the K/V split of a wavefront's loads");

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
  // q has landed before the first copies go out (a wait the compiler sees,
  // so that it adds none of its own inside the tile loop)
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (producer) {
    issue(0, 0);
    if (ntile > 1) issue(1, 1);
  }

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

  auto tile = [&](int t, const unsigned char* kc, const unsigned char* vc) __attribute__((always_inline)) {
    // widen this wavefront's V stripe; LDS operations of a wavefront complete
    // in order, so its transposed reads below see these writes
    const int u0 = 8 * wave + 2 * grp;
    uint4 codes[2];
    lds_b128x2(codes[0], codes[1], lds_off(vc + c * VROW8 + 16 * (u0 ^ (c & 7))),
               lds_off(vc + c * VROW8 + 16 * ((u0 + 1) ^ (c & 7))));
    uint32_t dad[2];
    u32x4_t wide[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dad[j] = lds_off(vwide + c * VROWB + 32 * ((u0 + j) ^ (c & 7)));
      wide[2 * j] = __builtin_bit_cast(u32x4_t, widen8(make_uint2(codes[j].x, codes[j].y)));
      wide[2 * j + 1] = __builtin_bit_cast(u32x4_t, widen8(make_uint2(codes[j].z, codes[j].w)));
    }
    lds_st_wide(dad, wide);
    const int k0 = t * BK;
    // dims 32 ks + 8 grp .. + 7: logical 16-byte chunk 12 wave + 2 ks + grp/2, half grp%2
    uint32_t kad[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kad[ks] = lds_off(kc + krow + 16 * ((12 * wave + 2 * ks + (grp >> 1)) ^ c) + 8 * (grp & 1));
    uint2 kw[KS];
    lds_b64x6(kw, kad);
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma16(as_bf16x8(widen8(kw[ks])), qf[ks], sc);
    // Branch-free on purpose (MFMA result read by the VALU right after).
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (k0 + 4 * grp + r < my_nk) ? sc[r] : kNegInf;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_across_groups(mx) * c2;   // base-2 units
    // lazy rescaling, as the bf16 decode
    if (__any(mx > m + kDecLazy)) {
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - ((mn == kNegInf) ? 0.f : mn));
      l *= alpha;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[tt] *= alpha;
      m = mn;
      asm volatile("s_nop 4" ::: "memory");   // the PV products read acc below
    }
    const float ms = (m == kNegInf) ? 0.f : m;
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(fmaf(sc[r], c2, -ms));
    const uint2 pk = make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
    // l sums the bf16 P that weight V
    l += add_bf16_pair(pk.y, add_bf16_pair(pk.x, 0.f));
    const v4i16_t pb = __builtin_bit_cast(v4i16_t, pk);
    uint32_t vad[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) vad[tt] = lds_off(vwide + vrow + 32 * ((8 * wave + tt) ^ (vr & 7)));
    uint2 vt[NT];
    lds_tr4x8(vt, vad);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16_t, vt[tt]), pb,
                                                         acc[tt], 0, 0, 0);
  };

  // tile t sits in stage t % 3; tile t + 2 goes to stage (t + 2) % 3, the
  // one tile t - 1 used.  A producer's loads in flight at step t: tile t's
  // ten, then (if it exists) tile t + 1's ten.
  static_assert(DMA_PER_WAVE == 5 && SPW == 2, "the waits count ten loads per tile");
  int st = 0;
  for (int t = 0; t < ntile; ++t) {
    const int sn = (st == 0) ? 2 : st - 1;
    if (producer) {
      if (t + 1 < ntile) __builtin_amdgcn_s_waitcnt(0x0F7A);   // vmcnt(10)
      else __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0)
    }
    ring_barrier();   // every share of tile t has landed; tile t-1 is consumed
    if (producer && t + 2 < ntile) issue(t + 2, sn);
    if (t < my_ntile) tile(t, kst[half][st], vst[half][st]);   // uniform per wavefront
    st = (st == NST - 1) ? 0 : st + 1;
  }

  const int s = SPW * blockIdx.y + half;
  l = sum_across_groups(l);
  if (my_nk > 0 && g < a.hkv && c < G) {
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

// Rings of at most 128 slots in one launch (as the bf16 decode's
// decode_ring_kernel): a workgroup per (sequence, kv head), wavefront w on
// slots 32 w .. 32 w + 31.  Every copy of a wavefront's slots goes out at
// once into its own LDS region (6 KB of K codes, rows of 192 B; 4 KB of V
// codes, rows of 128 B); the wavefront widens its V codes into a bf16 copy
// laid out like the bf16 ring kernel's V (rows of 256 B, 32-byte unit u at
// u ^ (row & 7)) for the transposed reads, computes its two 16-key tiles,
// and the four partials (m, l, O) are merged in LDS with the sink added
// once.  k_scale folds into the base-2 score factor, v_scale multiplies the
// merged output.
constexpr int RG_ROWS = 32;                  // ring slots per wavefront
constexpr int RG_K8 = RG_ROWS * D;           // 6 KB of K codes
constexpr int RG_V8 = RG_ROWS * DV;          // 4 KB of V codes
constexpr int RG_VB = RG_ROWS * DV * 2;      // 8 KB of widened V
constexpr int RG_REG = RG_K8 + RG_V8 + RG_VB;
static_assert(RG_REG >= 16 * DV * 4 + 32 * 4, "a region holds a wavefront's partial for the merge");

__global__ __launch_bounds__(256, 2) void decode_ring_fp8_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char reg_all[4 * RG_REG];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x, b = blockIdx.y;
  const int G = a.hq / a.hkv;
  unsigned char* kreg = reg_all + wave * RG_REG;
  unsigned char* vreg = kreg + RG_K8;
  unsigned char* vwb = vreg + RG_V8;

  long long p, row0, len;
  if (!key_range(a, 0, b, &p, &row0, &len)) {   // uniform over the workgroup
    if (c < G) {   // a broken contract: NaN outputs
      bf16_t* orow = static_cast<bf16_t*>(a.o) + ((long long)b * a.hq + g * G + c) * DV + 32 * wave + 8 * grp;
      st16(orow, make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u));
    }
    return;
  }
  const int key0 = RG_ROWS * wave;             // this wavefront's first slot
  const int nk = (int)min((long long)RG_ROWS, max(0LL, len - key0));   // its valid slots
  const int klast = (int)len - 1;              // len >= 1 here

  const float kscale = a.kscale[g], vscale = a.vscale[g];
  // q of head g*G + c (rotated to position p by the preparation kernel when
  // RoPE is on); columns c >= G repeat head G - 1 (their results are never
  // stored).  Issued before the copies, so that it lands with tile 0.
  bf16x8 qf[KS];
  {
    const bf16_t* qsrc = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
    const bf16_t* qrow = qsrc + ((long long)b * a.hq + g * G + min(c, G - 1)) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 32 * ks));
  }

  // ---- copies, tile by tile (keys 0..15, then 16..31 of the wavefront's
  // slots): K slot s = 64 ii + lane (ii < 6) is row s / 12, 16-byte chunk
  // s % 12; V slot s = 64 jj + lane (jj < 4) is row s / 8, chunk s % 8.
  // Rows past the last valid slot reload the last one (finite data,
  // masked); a wavefront with no valid slot reloads the ring's last written
  // slot, so every wavefront issues the same 10 copies and the waits below
  // count exactly.
  {
    const unsigned char* kb = static_cast<const unsigned char*>(a.k) + (row0 * a.hkv + g) * (long long)D;
    const unsigned char* vb = static_cast<const unsigned char*>(a.v) + (row0 * a.hkv + g) * (long long)DV;
    const int kstr = a.hkv * D, vstr = a.hkv * DV;
    auto slot = [&](int row) { return min(key0 + min(row, nk - 1), klast); };
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int ii = 3 * t; ii < 3 * t + 3; ++ii) {
        const int sl = 64 * ii + lane;
        const int row = sl / 12, pc = sl - row * 12;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kb + (__umul24(slot(row), kstr) + 16 * pc)),
                                         (lds_void_t*)(kreg + 1024 * ii), 16, 0, 0);
      }
#pragma unroll
      for (int jj = 2 * t; jj < 2 * t + 2; ++jj) {
        const int sl = 64 * jj + lane;
        const int row = sl >> 3, pc = sl & 7;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vb + (__umul24(slot(row), vstr) + 16 * pc)),
                                         (lds_void_t*)(vreg + 1024 * jj), 16, 0, 0);
      }
    }
  }
  static_assert(RG_K8 == 6 * 1024 && RG_V8 == 4 * 1024, "three K and two V copies per tile");

  const float c2 = a.scale * kLog2e * kscale;   // raw code score -> base-2 units
  float m = kNegInf, l = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one 16-key tile: widen its V codes (lane handles the (row, 16-code
  // chunk) items 128 t + lane and 128 t + 64 + lane) into the bf16 copy,
  // then the products.  Reads of the copy targets are inline asm that wait
  // for their own data, so the compiler's wait analysis does not add a
  // wait for the copies still in flight; the wavefront's LDS operations
  // complete in order, so its transposed reads see its widening writes.
  auto tile = [&](int t) __attribute__((always_inline)) {
    uint32_t wad[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int it = 128 * t + 64 * j + lane;
      wad[j] = lds_off(vreg + (it >> 3) * DV + 16 * (it & 7));
    }
    uint4 codes[2];
    lds_b128x2(codes[0], codes[1], wad[0], wad[1]);
    uint32_t dad[2];
    u32x4_t wide[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int it = 128 * t + 64 * j + lane;
      const int row = it >> 3, cc = it & 7;
      dad[j] = lds_off(vwb + row * (DV * 2) + 32 * (cc ^ (row & 7)));
      wide[2 * j] = __builtin_bit_cast(u32x4_t, widen8(make_uint2(codes[j].x, codes[j].y)));
      wide[2 * j + 1] = __builtin_bit_cast(u32x4_t, widen8(make_uint2(codes[j].z, codes[j].w)));
    }
    lds_st_wide(dad, wide);
    const int kr = BK * t + c;
    uint32_t kad[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kad[ks] = lds_off(kreg + kr * D + 32 * ks + 8 * grp);
    uint2 kw[KS];
    lds_b64x6(kw, kad);   // dims 32 ks + 8 grp .. + 7 of key row kr: 8 codes each
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma16(as_bf16x8(widen8(kw[ks])), qf[ks], sc);
    // branch-free masking (see the split kernels)
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (BK * t + 4 * grp + r < nk) ? sc[r] : kNegInf;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_across_groups(mx) * c2;
    const float mn = fmaxf(m, mx);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(m - ms);
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(fmaf(sc[r], c2, -ms));
    const uint2 pk = make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
    l = l * alpha + add_bf16_pair(pk.y, add_bf16_pair(pk.x, 0.f));
    m = mn;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] *= alpha;
    const v4i16_t pb = __builtin_bit_cast(v4i16_t, pk);
    const int vr = BK * t + 4 * grp + (c >> 2);
    uint32_t vad[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      vad[tt] = lds_off(vwb + vr * (DV * 2) + 32 * (tt ^ (vr & 7)) + 8 * (c & 3));
    uint2 vt[NT];
    lds_tr4x8(vt, vad);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16_t, vt[tt]), pb,
                                                         acc[tt], 0, 0, 0);
  };
  static_assert(NT == 8 && KS == 6 && RG_ROWS == 2 * BK, "two tiles; six K and eight V pieces");

  // q and tile 0's five copies have landed once at most tile 1's five are
  // in flight; tile 1 is computed after everything has landed
  __builtin_amdgcn_s_waitcnt(0x0F75);   // vmcnt(5)
  if (nk > 0) tile(0);                  // uniform
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (nk > BK) tile(1);                 // uniform
  l = sum_across_groups(l);

  // ---- merge the four wavefronts' partials (O [16 columns][128 dims], m and
  // l [16], fp32, base 2, in each wavefront's own region); then wavefront w
  // writes dims 32 w .. 32 w + 31
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float* po = reinterpret_cast<float*>(kreg);
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
    *reinterpret_cast<float4*>(po + c * DV + 16 * tt + 4 * grp) =
        make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
  if (grp == 0) {
    po[16 * DV + c] = m;
    po[16 * DV + 16 + c] = l;
  }
  __syncthreads();
  const float s2 = (c < G && a.sink) ? a.sink[g * G + c] * kLog2e : kNegInf;
  float mw[4], lw[4];
  float M = s2;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float* pw = reinterpret_cast<const float*>(reg_all + w * RG_REG);
    mw[w] = pw[16 * DV + c];
    lw[w] = pw[16 * DV + 16 + c];
    M = fmaxf(M, mw[w]);
  }
  float den = (s2 > kNegInf) ? fast_exp2(s2 - M) : 0.f;
  float o8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o8[e] = 0.f;
  const int d0 = 32 * wave + 8 * grp;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float sw = (mw[w] > kNegInf) ? fast_exp2(mw[w] - M) : 0.f;
    den += sw * lw[w];
    const float* pw = reinterpret_cast<const float*>(reg_all + w * RG_REG) + c * DV + d0;
    const float4 x0 = *reinterpret_cast<const float4*>(pw);
    const float4 x1 = *reinterpret_cast<const float4*>(pw + 4);
    o8[0] += sw * x0.x; o8[1] += sw * x0.y; o8[2] += sw * x0.z; o8[3] += sw * x0.w;
    o8[4] += sw * x1.x; o8[5] += sw * x1.y; o8[6] += sw * x1.z; o8[7] += sw * x1.w;
  }
  if (c < G) {
    const float inv = (den > 0.f) ? vscale / den : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] *= inv;
    bf16_t* orow = static_cast<bf16_t*>(a.o) + ((long long)b * a.hq + g * G + c) * DV + d0;
    st16(orow, pack8(o8));
  }
}

bool decode_fp8_supported(const AttnArgs& a) { return decode_bf16_supported(a); }

hipError_t launch_decode_fp8(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  hipError_t e = launch_decode_rope_q(a, layout, stream);
  if (e != hipSuccess) return e;
  if (decode_ring_supported(a, layout)) {
    hipLaunchKernelGGL(decode_ring_fp8_kernel, dim3((unsigned)a.hkv, (unsigned)a.B), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
  }
  dim3 g1((unsigned)(a.hkv / HG), (unsigned)((a.nsplit + SPW - 1) / SPW), (unsigned)a.B);
  hipLaunchKernelGGL(decode_fp8_split_kernel, g1, dim3(64 * HG * SPW), 0, stream, a, layout);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, layout, stream);
}

}  // namespace hswa
