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

// A workgroup of 8 wavefronts takes two consecutive splits s = 2 sp and
// 2 sp + 1 of one (sequence, group of four kv heads): wavefront w computes
// head w % 4 of split 2 sp + w / 4.  Only wavefronts 0..3 (one per SIMD)
// issue copies, those of both splits (20 per tile): a wavefront stalls while
// the vector-memory path accepts its copies, and the other wavefront of its
// SIMD, which issues none, computes meanwhile.  Two LDS stages per split
// (the CU's 160 KB): tile t + 1 is requested while tile t is computed.
constexpr int SPW = 2;   // splits per workgroup
__global__ __launch_bounds__(64 * HG * SPW, 1) void decode_split_kernel(AttnArgs a, int layout) {
  __shared__ __attribute__((aligned(16))) unsigned char kst[SPW][2][KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char vst[SPW][2][VTILE];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int wave = wv & (HG - 1);                            // head within the group
  const int half = wv / HG;                                  // which of the two splits
  const bool producer = half == 0;
  const int gx = blockIdx.x, b = blockIdx.z;
  const int g = HG * gx + wave;
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv;

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
  // K stage (ii < 24, ii' = ii) or the V stage (ii' = ii - 24).  K slot s is
  // row s / 96, physical chunk pc = s % 96 holding logical chunk pc ^ row%16
  // (XOR on the low four bits, within its aligned 256 B); V slot s is row
  // s / 64, physical 32-byte unit (s % 64) / 2 holding logical unit
  // unit ^ row%8.  Rows past a split reload its last key (masked later); an
  // empty second split reloads the first one's rows (never read).
  const unsigned char* kbase[SPW];
  const unsigned char* vbase[SPW];
  int lastkey[SPW];
#pragma unroll
  for (int h = 0; h < SPW; ++h) {
    const int hh = (nk[h] > 0) ? h : 0;
    kbase[h] = static_cast<const unsigned char*>(a.k) +
               (((row0 + ks0[hh]) * a.hkv + HG * gx) * (long long)D) * 2;
    vbase[h] = static_cast<const unsigned char*>(a.v) +
               (((row0 + ks0[hh]) * a.hkv + HG * gx) * (long long)DV) * 2;
    lastkey[h] = nk[hh] - 1;
  }
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
  // multiply-add per instruction.  The copies of tile t of both splits go
  // into stage st (producers only).
  auto issue = [&](int t, int st) {
#pragma unroll
    for (int h = 0; h < SPW; ++h) {
#pragma unroll
      for (int u = 0; u < DMA_PER_WAVE; ++u) {
        const int ii = wave + HG * u;
        const int key = min(t * BK + drow[u], lastkey[h]);
        if (u < KINSTR / HG)   // wave-uniform: the first six instructions are K, the rest V
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
  static_assert(KINSTR / HG == 6, "the K/V split of a wavefront's loads");

  if (producer) issue(0, 0);

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

  // per-lane LDS offsets: K row c, logical chunk 24 wave + 4 ks + grp; the
  // transposed V read of lane (c, grp): row 4 grp + c/4, bytes 8 (c%4) of the
  // logical 32-byte unit 8 wave + tt
  const int krow = c * KROW;
  const int vr = 4 * grp + (c >> 2);
  const int vrow = vr * VROW + 8 * (c & 3);

  // one tile from its stage; the LDS reads are inline asm that wait for
  // their own data, so the compiler's wait analysis adds no wait for the
  // copies of the next tile still in flight
  auto tile = [&](int t, const unsigned char* kc, const unsigned char* vc) __attribute__((always_inline)) {
    const int k0 = t * BK;
    uint32_t kad[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kad[ks] = lds_off(kc + krow + 16 * ((24 * wave + 4 * ks + grp) ^ c));
    uint4 kw[KS];
    lds_b128x6(kw, kad);
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma16(as_bf16x8(kw[ks]), qf[ks], sc);
    // Branch-free on purpose: the first VALU read of an MFMA result needs
    // wait states after it, and with a branch between them the compiler
    // did not insert them on the path that skips the branch body.
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (k0 + 4 * grp + r < my_nk) ? sc[r] : kNegInf;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_across_groups(mx) * c2;   // base-2 units
    // Lazy rescaling: the reference m moves only when a column's tile max
    // passes it by more than kDecLazy, so P = exp2(s - m) <= 2^kDecLazy
    // (exact in fp32 and bf16's range); (m, l, O) stay consistent for the
    // combine, which only needs them to share one reference.
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
    const v4i16 pb = __builtin_bit_cast(v4i16, pk);
    // -- O^T += V^T . P^T: lane (c, grp) holds keys 4 grp + r, the k-index of
    //    the 16x16x16 form; the transposed read gives V[4 grp + r][16 tt + c]
    uint32_t vad[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) vad[tt] = lds_off(vc + vrow + 32 * ((8 * wave + tt) ^ (vr & 7)));
    uint2 vt[NT];
    lds_tr4x8(vt, vad);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, vt[tt]), pb,
                                                         acc[tt], 0, 0, 0);
  };
  static_assert(NT == 8 && KS == 6, "the read helpers take six K and eight V pieces");

  // A producer's loads in flight at step t are tile t's 20 (and, at t = 0,
  // its q loads); tile t + 1 goes to the stage tile t - 1 used.
  for (int t = 0; t < ntile; ++t) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    ring_barrier();   // every share of tile t has landed; tile t-1 is consumed
    if (producer && t + 1 < ntile) issue(t + 1, (t + 1) & 1);
    if (t < my_ntile) tile(t, kst[half][t & 1], vst[half][t & 1]);   // uniform per wavefront
  }

  const int s = SPW * blockIdx.y + half;
  l = sum_across_groups(l);
  if (my_nk > 0 && g < a.hkv && c < G) {
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
  // Splits in batches of eight whose loads are all issued before any is
  // used (one memory round trip per batch, not per split); the sums run in
  // split order.  Indices past the last split re-read it and are ignored.
  float M = s2;
  for (int s0 = 0; s0 < nspl; s0 += 8) {
    float mv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) mv[j] = wml[2 * min(s0 + j, nspl - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) M = fmaxf(M, mv[j]);
  }
  float den = (s2 > kNegInf) ? fast_exp2(s2 - M) : 0.f;
  float o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < nspl; s0 += 8) {
    float mv[8], lv[8], x0[8], x1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sj = min(s0 + j, nspl - 1);
      mv[j] = wml[2 * sj];
      lv[j] = wml[2 * sj + 1];
      const float* wo = a.ws + (base + sj) * DV;
      x0[j] = wo[lane];
      x1[j] = wo[lane + 64];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < nspl) {   // uniform
        const float w = fast_exp2(mv[j] - M);
        den += w * lv[j];
        o0 += w * x0[j];
        o1 += w * x1[j];
      }
    }
  }
  const float inv = (den > 0.f) ? 1.f / den : 0.f;
  orow[lane] = f32_to_bf16_bits(o0 * inv);
  orow[lane + 64] = f32_to_bf16_bits(o1 * inv);
}

// ---- ring caches of at most 128 slots: one launch -------------------------
// The SWA layer's ring is small (W = 128 keys per sequence and kv head), so
// the split-K form above spends its time in launches and in waits, not in
// bytes.  Here a workgroup owns (sequence b, kv head g) and its 4
// wavefronts take 32 ring slots each: every wavefront issues all copies of
// its slots into its own LDS region at once (one memory latency, no
// barrier before the products), computes S^T = K . Q^T and O^T += V^T P^T
// over its two 16-key tiles as the split kernel does, and the four partial
// (m, l, O) are merged through LDS with the sink added once (the output
// rule of rslog.cc section 4.4), written as o directly: no workspace
// partials and no second launch.
constexpr int RG_ROWS = 32;                 // ring slots per wavefront
constexpr int RG_KREG = RG_ROWS * D * 2;    // 12 KB: 32 rows of 384 B
constexpr int RG_VREG = RG_ROWS * DV * 2;   // 8 KB: 32 rows of 256 B

__global__ __launch_bounds__(256, 2) void decode_ring_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char kreg_all[4 * RG_KREG];
  __shared__ __attribute__((aligned(16))) unsigned char vreg_all[4 * RG_VREG];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x, b = blockIdx.y;
  const int G = a.hq / a.hkv;
  unsigned char* kreg = kreg_all + wave * RG_KREG;
  unsigned char* vreg = vreg_all + wave * RG_VREG;

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

  // q of head g*G + c (rotated to position p by the preparation kernel when
  // RoPE is on); columns c >= G repeat head G - 1 (their results are never
  // stored).  Issued first, so that it lands with tile 0.
  bf16x8 qf[KS];
  {
    const bf16_t* qsrc = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
    const bf16_t* qrow = qsrc + ((long long)b * a.hq + g * G + min(c, G - 1)) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 32 * ks));
  }

  // ---- copies, tile by tile (keys 0..15, then 16..31 of the wavefront's
  // slots): K slot s = 64 ii + lane (ii < 12) is row s / 24, physical chunk
  // s % 24 holding logical chunk pc ^ ((row >> 1) & 7); V slot s = 64 jj +
  // lane (jj < 8) is row s / 16, 16-byte chunk s % 16 of physical 32-byte
  // unit u holding logical unit u ^ (row & 7).  Rows past the last valid
  // slot reload the last one (finite data, masked); a wavefront with no
  // valid slot reloads the ring's last written slot, so every wavefront
  // issues the same 20 copies and the waits below count exactly.
  {
    const unsigned char* kb = static_cast<const unsigned char*>(a.k) + (row0 * a.hkv + g) * (long long)(D * 2);
    const unsigned char* vb = static_cast<const unsigned char*>(a.v) + (row0 * a.hkv + g) * (long long)(DV * 2);
    const int kstr = a.hkv * D * 2, vstr = a.hkv * DV * 2;
    auto slot = [&](int row) { return min(key0 + min(row, nk - 1), klast); };
#pragma unroll
    for (int half16 = 0; half16 < 2; ++half16) {
#pragma unroll
      for (int ii = 6 * half16; ii < 6 * half16 + 6; ++ii) {
        const int sl = 64 * ii + lane;
        const int row = sl / 24, pc = sl - row * 24;
        const int lc = pc ^ ((row >> 1) & 7);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kb + (__umul24(slot(row), kstr) + 16 * lc)),
                                         (lds_void_t*)(kreg + 1024 * ii), 16, 0, 0);
      }
#pragma unroll
      for (int jj = 4 * half16; jj < 4 * half16 + 4; ++jj) {
        const int sl = 64 * jj + lane;
        const int row = sl >> 4, pc = sl & 15;
        const int lc = 2 * ((pc >> 1) ^ (row & 7)) + (pc & 1);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vb + (__umul24(slot(row), vstr) + 16 * lc)),
                                         (lds_void_t*)(vreg + 1024 * jj), 16, 0, 0);
      }
    }
  }

  const float c2 = a.scale * kLog2e;
  float m = kNegInf, l = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one 16-key tile from the wavefront's region; its LDS reads are inline
  // asm that wait for their own data, so the compiler's wait analysis does
  // not add a wait for the copies still in flight
  auto tile = [&](int t) __attribute__((always_inline)) {
    const int kr = BK * t + c;
    uint32_t kad[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kad[ks] = lds_off(kreg + kr * (D * 2) + 16 * ((4 * ks + grp) ^ ((kr >> 1) & 7)));
    uint4 kw[KS];
    lds_b128x6(kw, kad);
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma16(as_bf16x8(kw[ks]), qf[ks], sc);
    // branch-free masking (see the split kernel)
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
    const v4i16 pb = __builtin_bit_cast(v4i16, pk);
    const int vr = BK * t + 4 * grp + (c >> 2);
    uint32_t vad[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      vad[tt] = lds_off(vreg + vr * (DV * 2) + 32 * (tt ^ (vr & 7)) + 8 * (c & 3));
    uint2 vt[NT];
    lds_tr4x8(vt, vad);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, vt[tt]), pb,
                                                         acc[tt], 0, 0, 0);
  };
  static_assert(NT == 8 && KS == 6, "the read helpers take six K and eight V pieces");

  // q and tile 0's ten copies have landed once at most tile 1's ten are in
  // flight; tile 1 is computed after everything has landed
  __builtin_amdgcn_s_waitcnt(0x0F7A);   // vmcnt(10)
  if (nk > 0) tile(0);                  // uniform
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (nk > BK) tile(1);                 // uniform
  l = sum_across_groups(l);

  // ---- merge the four wavefronts' partials -----------------------------------
  // each wavefront leaves O [16 columns][128 dims], m and l [16] (fp32, base
  // 2) in its own K region; then wavefront w writes dims 32w .. 32w + 31
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
    const float* pw = reinterpret_cast<const float*>(kreg_all + w * RG_KREG);
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
    const float* pw = reinterpret_cast<const float*>(kreg_all + w * RG_KREG) + c * DV + d0;
    const float4 x0 = *reinterpret_cast<const float4*>(pw);
    const float4 x1 = *reinterpret_cast<const float4*>(pw + 4);
    o8[0] += sw * x0.x; o8[1] += sw * x0.y; o8[2] += sw * x0.z; o8[3] += sw * x0.w;
    o8[4] += sw * x1.x; o8[5] += sw * x1.y; o8[6] += sw * x1.z; o8[7] += sw * x1.w;
  }
  if (c < G) {
    const float inv = (den > 0.f) ? 1.f / den : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] *= inv;
    bf16_t* orow = static_cast<bf16_t*>(a.o) + ((long long)b * a.hq + g * G + c) * DV + d0;
    st16(orow, pack8(o8));
  }
}

bool decode_ring_supported(const AttnArgs& a, int layout) {
  const int G = a.hq / a.hkv;
  return layout == 0 && a.window > 0 && a.window <= 4 * RG_ROWS && a.d_qk == D && a.d_v == DV &&
         G >= 1 && G <= 16 && 2 * a.half <= D;
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
  if (decode_ring_supported(a, layout)) {
    hipLaunchKernelGGL(decode_ring_kernel, dim3((unsigned)a.hkv, (unsigned)a.B), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
  }
  dim3 g1((unsigned)(a.hkv / HG), (unsigned)((a.nsplit + SPW - 1) / SPW), (unsigned)a.B);
  hipLaunchKernelGGL(decode_split_kernel, g1, dim3(64 * HG * SPW), 0, stream, a, layout);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(a, layout, stream);
}

}  // namespace hswa
