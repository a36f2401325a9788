// Multi-token decode: one verification step of multi-token prediction.
//
// The MTP drafts are checked by the main model in one forward pass ("visual
// reading: MiMo MTP/SWA, not MLA" (syt-nju.github.io), MTP section: with the
// attention FLOPs saved by SWA the model is memory-bound, and verifying the
// three drafts costs almost nothing extra).  Sequence b brings T queries at
// positions pos[b] .. pos[b] + T - 1 (the last accepted token, then T - 1
// drafts); each attends causally, also among the drafts, to positions
// max(0, p - W + 1) .. p (W = 0: 0 .. p) of its cache, whose rows up to
// pos[b] + T - 1 are written.  A ring cache holds token j in slot j mod S
// with S >= W + T - 1 slots, so that the drafts have not overwritten a key
// the first query still sees.
//
// The split-K stream is the single-token decode's: a workgroup owns
// (sequence b, four kv heads, split s) and streams its keys in 16-key tiles
// through LDS with global_load_lds.  Each tile now serves all T * G query
// columns of a kv head: the N side of the MFMAs is one or two blocks of 16
// columns (column n = token n / G, head n % G), and past 32 columns two
// wavefronts share a kv head, each with its half of the columns.  The cache
// is read once for all T tokens, so the step costs about what a single-token
// step does while the matrix cores do T times the work.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

// The split kernel checks the sum of a lane's four P of a tile against the
// current reference (rather than the tile max against kDecLazy), so every P
// stays below 2^10.
constexpr float kDecLazySum = 1024.f;

constexpr int D = 192;
constexpr int DV = 128;
constexpr int KS = D / 32;
static_assert(KS == 6, "six k-steps of 32 dims");
constexpr int NT = DV / 16;
static_assert(NT == 8, "eight 16-dim output tiles");
constexpr int BK = 16;                    // keys per tile
constexpr int HG = 4;                     // kv heads per workgroup
constexpr int KROW = HG * D * 2;          // 1536 B: the group's K of one cache row
constexpr int VROW = HG * DV * 2;         // 1024 B: its V
constexpr int KTILE = BK * KROW;          // 24 KB
constexpr int VTILE = BK * VROW;          // 16 KB
constexpr int KINSTR = KTILE / 1024;      // 24 load instructions of 1 KB
constexpr int VINSTR = VTILE / 1024;      // 16

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Keys of sequence b: cache rows row0 .. row0 + len - 1.  p0 = pos[b].
// Returns false for a sequence the caller's contract rules out.
__device__ __forceinline__ bool multi_range(const AttnArgs& a, int layout, int b, long long* p0,
                                            long long* row0, long long* len) {
  const long long p = a.pos[b];
  const long long last = p + a.nq - 1;
  *p0 = p;
  if (p < 0 || last > a.max_pos) return false;
  if (layout == 0) {  // ring: slots 0 .. min(last, S-1) hold tokens
    *row0 = (long long)b * a.slots;
    *len = (last + 1 < a.slots) ? last + 1 : a.slots;
    return true;
  }
  const long long off = a.seq_offsets[b];
  const long long rows = a.seq_offsets[b + 1] - off;
  if (last >= rows) return false;
  const long long lo = (a.window > 0 && p - a.window + 1 > 0) ? p - a.window + 1 : 0;
  *row0 = off + lo;
  *len = last - lo + 1;
  return true;
}

// Sequence position of key kk (0-based in the key range).
struct KeyPos {
  long long base;    // contiguous: position of key 0; ring: newest position
  int nm, S;         // ring: newest mod S, slot count; S = 0 for a contiguous cache
  __device__ __forceinline__ long long operator()(long long kk) const {
    if (S == 0) return base + kk;
    int dd = nm - (int)kk;                   // (newest - slot) mod S
    dd += (dd < 0) ? S : 0;
    return base - dd;
  }
};

__device__ __forceinline__ KeyPos key_pos(const AttnArgs& a, int layout, long long p0,
                                          long long row0, long long off) {
  KeyPos kp;
  if (layout == 0) {
    kp.base = p0 + a.nq - 1;
    kp.S = a.slots;
    kp.nm = (int)(kp.base % a.slots);
  } else {
    kp.base = row0 - off;
    kp.S = 0;
    kp.nm = 0;
  }
  return kp;
}

}  // namespace

// q of every (sequence, token, head) rotated to its position p0 + t; the
// angle in fp64 (positions reach 2.6e5), the rotation in fp32, rounded to bf16.
__global__ __launch_bounds__(64) void decode_multi_rope_q_kernel(AttnArgs a, int layout) {
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  long long p0, row0, len;
  if (!multi_range(a, layout, b, &p0, &row0, &len)) return;
  const long long p = p0 + t;
  const long long rowi = ((long long)b * a.nq + t) * a.hq + h;
  const bf16_t* q = static_cast<const bf16_t*>(a.q) + rowi * D;
  bf16_t* qo = static_cast<bf16_t*>(a.qrot) + rowi * D;
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

// s_waitcnt operand with vmcnt n (0..63) and the other counters open.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// NB: 16-column blocks per wavefront; CW: wavefronts per kv head (each with
// NB * 16 of the T * G columns); NST: LDS stages of 40 KB.  Long splits take
// four stages, which fill the compute unit's 160 KB: tiles t + 1 .. t + 3
// are in flight while tile t is computed (120 KB of loads per compute unit,
// one workgroup each).  Short splits (a ring of a few tiles) take two, so
// that two workgroups of four wavefronts share a compute unit.
template <int NB, int CW, int NST>
__global__ __launch_bounds__(256 * CW, (NST == 2 && CW == 1) ? 2 : 1) void decode_multi_split_kernel(
    AttnArgs a, int layout) {
  constexpr int NWAVE = HG * CW;
  constexpr int DMA_PER_WAVE = (KINSTR + VINSTR) / HG;   // producers: the wavefronts of column half 0
  static_assert((KINSTR + VINSTR) % HG == 0 && KINSTR % HG == 0, "even split of the loads");
  static_assert(DMA_PER_WAVE * (NST - 2) <= 63, "the vmcnt field holds the loads in flight");
  static_assert(NST == 2 || NST == 4, "stage arithmetic below");
  __shared__ __attribute__((aligned(16))) unsigned char kst[NST][KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char vst[NST][VTILE];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int hw = wave % HG, ch = wave / HG;                     // kv head in group, column half
  const int gx = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int g = HG * gx + hw;
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int G = a.hq / a.hkv, T = a.nq;

  long long p0, row0, len;
  if (!multi_range(a, layout, b, &p0, &row0, &len)) return;   // uniform over the workgroup
  const long long ks0 = (long long)s * a.split_keys;
  if (ks0 >= len) return;
  const long long ks1 = (ks0 + a.split_keys < len) ? ks0 + a.split_keys : len;
  const int nkeys = (int)(ks1 - ks0);
  const int ntile = (nkeys + BK - 1) / BK;
  const KeyPos kpos = key_pos(a, layout, p0, row0, layout == 0 ? 0 : a.seq_offsets[b]);

  // ---- tile copies: the single-token decode's slot map (K slot s: row s / 96,
  // physical chunk s % 96 holding logical chunk pc ^ row%16; V slot s: row
  // s / 64, 32-byte unit (s % 64) / 2 holding unit ^ row%8) -----------------
  const unsigned char* kbase = static_cast<const unsigned char*>(a.k) +
                               (((row0 + ks0) * a.hkv + HG * gx) * (long long)D) * 2;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) +
                               (((row0 + ks0) * a.hkv + HG * gx) * (long long)DV) * 2;
  const int kstride = a.hkv * D * 2, vstride = a.hkv * DV * 2;
  int drow[DMA_PER_WAVE], doff[DMA_PER_WAVE];
#pragma unroll
  for (int u = 0; u < DMA_PER_WAVE; ++u) {
    const int ii = hw + HG * u;
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
  // Only the wavefronts of column half 0 (one per SIMD when CW = 2) issue
  // the copies: issuing stalls a wavefront until the vector-memory path
  // accepts each copy, and the SIMD's other wavefront computes meanwhile.
  const bool producer = ch == 0;
  auto issue = [&](int k0, unsigned char* kd, unsigned char* vd) {
    if (!producer) return;
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int ii = hw + HG * u;
      const int key = min(k0 + drow[u], nkeys - 1);
      if (u < KINSTR / HG)   // wave-uniform: K instructions first, then V
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kbase + (__umul24(key, kstride) + doff[u])),
                                         (lds_void_t*)(kd + 1024 * ii), 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vbase + (__umul24(key, vstride) + doff[u])),
                                         (lds_void_t*)(vd + 1024 * (ii - KINSTR)), 16, 0, 0);
    }
  };

  // ---- this lane's query columns: n = 16 (NB ch + nb) + c -------------------
  bf16x8 qf[NB][KS];
  int ctok[NB];
  bool cval[NB];
  {
    const bf16_t* qsrc = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = 16 * (NB * ch + nb) + c;
      cval[nb] = n < T * G;
      const int tn = cval[nb] ? n / G : 0, hn = cval[nb] ? n - tn * G : 0;
      ctok[nb] = tn;
      const bf16_t* qrow =
          qsrc + (((long long)b * T + tn) * a.hq + g * G + hn) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[nb][ks] = as_bf16x8(cval[nb] ? ld16(qrow + 32 * ks) : make_uint4(0, 0, 0, 0));
    }
  }
  // q has landed before the first copies go out (a wait the compiler sees,
  // so that it adds none of its own inside the tile loop)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  for (int t = 0; t < NST - 1 && t < ntile; ++t) issue(t * BK, kst[t], vst[t]);

  const float c2 = a.scale * kLog2e;
  const int W = a.window;
  float m[NB], l[NB];
  f32x4 acc[NT][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf;
    l[nb] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int krow = c * KROW;
  const int vr = 4 * grp + (c >> 2);
  const int vrow = vr * VROW + 8 * (c & 3);

  auto tile = [&](int t, const unsigned char* kc, const unsigned char* vc, unsigned char* kn,
                  unsigned char* vn) __attribute__((always_inline)) {
    // this wavefront's loads issued after tile t's: those of the (up to
    // NST - 2) tiles after it
    const int ahead = min(ntile - 1 - t, NST - 2);
    if (NST == 4 && ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA_PER_WAVE));
    else if (NST == 4 && ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA_PER_WAVE));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    ring_barrier();   // every wavefront's share of tile t has landed; tile t-1 is consumed
    if (t + NST - 1 < ntile) issue((t + NST - 1) * BK, kn, vn);
    const int k0 = t * BK;
    // key 4 grp + r of the tile is visible to column token tn iff it exists
    // and its position lies in [p0 + tn - W + 1, p0 + tn].  Decided before the
    // score products, with bitwise logic on 32-bit offsets from p0 (a key
    // range spans less than 2^31 positions), so that only selects follow the
    // MFMAs: no branch may sit between them and the first VALU read.
    bool vis[NB][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rel = (int)(kpos(ks0 + k0 + 4 * grp + r) - p0);
      const bool here = k0 + 4 * grp + r < nkeys;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vis[nb][r] = here & (rel <= ctok[nb]) & ((W == 0) | (rel > ctok[nb] - W));
    }
    f32x4 sc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint32_t kad[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kad[ks] = lds_off(kc + krow + 16 * ((24 * hw + 4 * ks + grp) ^ c));
    uint4 kf[KS];
    lds_b128x6(kf, kad);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc[nb] = mfma16(as_bf16x8(kf[ks]), qf[nb][ks], sc[nb]);
    uint2 pk[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[nb][r] = vis[nb][r] ? sc[nb][r] : kNegInf;
      // lazy rescaling checked on the P sum: P against the current
      // reference first; only a lane whose four P sum past kDecLazySum (a key
      // more than ~10 above the reference in log2 units) or a column with no
      // reference yet sends the wavefront to take the column max across the
      // lane groups and move the reference, so the common path has no max
      float ms = (m[nb] == kNegInf) ? 0.f : m[nb];
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(fmaf(sc[nb][r], c2, -ms));
      pk[nb] = make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
      float ts = add_bf16_pair(pk[nb].y, add_bf16_pair(pk[nb].x, 0.f));
      if (__any(m[nb] == kNegInf || !(ts <= kDecLazySum))) {
        float mx = fmaxf(fmaxf(sc[nb][0], sc[nb][1]), fmaxf(sc[nb][2], sc[nb][3]));
        mx = max_across_groups(mx) * c2;
        const float mn = fmaxf(m[nb], mx);
        const float alpha = fast_exp2(m[nb] - ((mn == kNegInf) ? 0.f : mn));
        l[nb] *= alpha;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[tt][nb] *= alpha;
        m[nb] = mn;
        ms = (mn == kNegInf) ? 0.f : mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(fmaf(sc[nb][r], c2, -ms));
        pk[nb] = make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
        ts = add_bf16_pair(pk[nb].y, add_bf16_pair(pk[nb].x, 0.f));
        asm volatile("s_nop 4" ::: "memory");   // the PV products read acc below
      }
      l[nb] += ts;
    }
    uint32_t vad[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) vad[tt] = lds_off(vc + vrow + 32 * ((8 * hw + tt) ^ (vr & 7)));
    uint2 vt[NT];
    lds_tr4x8(vt, vad);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[tt][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(v4i16_t, vt[tt]), __builtin_bit_cast(v4i16_t, pk[nb]), acc[tt][nb],
            0, 0, 0);
  };

  // tile t sits in stage t % NST; tile t + NST - 1 goes to the stage tile
  // t - 1 used
  for (int t = 0; t < ntile; ++t) {
    const int st = t & (NST - 1), sn = (t + NST - 1) & (NST - 1);
    tile(t, kst[st], vst[st], kst[sn], vst[sn]);
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = sum_across_groups(l[nb]);
    if (cval[nb]) {
      const int n = 16 * (NB * ch + nb) + c;
      const int hn = n - ctok[nb] * G;
      const long long idx =
          (((long long)b * T + ctok[nb]) * a.hq + g * G + hn) * a.nsplit + s;
      float* wo = a.ws + idx * DV + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
        *reinterpret_cast<float4*>(wo + 16 * tt) =
            make_float4(acc[tt][nb][0], acc[tt][nb][1], acc[tt][nb][2], acc[tt][nb][3]);
      if (grp == 0) {
        float* wml = a.ws + (long long)a.B * T * a.hq * a.nsplit * DV + idx * 2;
        wml[0] = m[nb];
        wml[1] = lt;
      }
    }
  }
}

// Per (b, t, h): M = max(sink, m_s), denominator exp2(sink - M) +
// sum_s exp2(m_s - M) l_s, output sum_s exp2(m_s - M) O_s over it (the sink
// enters once).  Splits with no visible key carry m = -inf and drop out.
__global__ __launch_bounds__(64) void decode_multi_combine_kernel(AttnArgs a, int layout) {
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const long long rowi = ((long long)b * a.nq + t) * a.hq + h;
  bf16_t* orow = static_cast<bf16_t*>(a.o) + rowi * DV;
  long long p0, row0, len;
  if (!multi_range(a, layout, b, &p0, &row0, &len)) {
    orow[lane] = 0x7fc0;
    orow[lane + 64] = 0x7fc0;
    return;
  }
  const int nspl = (int)((len + a.split_keys - 1) / a.split_keys);
  const long long base = rowi * a.nsplit;
  const float* wml = a.ws + (long long)a.B * a.nq * a.hq * a.nsplit * DV + base * 2;
  const float s2 = a.sink ? a.sink[h] * kLog2e : kNegInf;
  // Splits in batches of eight whose loads are all issued before any is
  // used; the sums run in split order, splits with no visible key (m = -inf)
  // drop out.  Indices past the last split re-read it and are ignored.
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
      if (s0 + j < nspl && mv[j] != kNegInf) {   // uniform
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

// Any shape, bf16 or fp32 storage: one wavefront per (sequence, token, head)
// row, a running (max, sum, output) over the key range seeded with the sink.
template <typename T>
__global__ __launch_bounds__(64) void decode_multi_generic_kernel(AttnArgs a, int layout) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int G = a.hq / a.hkv, g = h / G;
  const long long rowi = ((long long)b * a.nq + t) * a.hq + h;
  const T* q = static_cast<const T*>(a.q) + rowi * a.d_qk;
  const T* kc = static_cast<const T*>(a.k);
  const T* vc = static_cast<const T*>(a.v);
  T* orow = static_cast<T*>(a.o) + rowi * a.d_v;
  auto ld = [](const T* p, long long i) -> float {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const bf16_t*>(p)[i]);
    else return (float)p[i];
  };
  auto st = [](T* p, long long i, float x) {
    if constexpr (sizeof(T) == 2) reinterpret_cast<bf16_t*>(p)[i] = f32_to_bf16_bits(x);
    else p[i] = x;
  };
  long long p0, row0, len;
  if (!multi_range(a, layout, b, &p0, &row0, &len)) {
    for (int d = lane; d < a.d_v; d += 64) {
      if constexpr (sizeof(T) == 2) reinterpret_cast<bf16_t*>(orow)[d] = 0x7fc0;
      else reinterpret_cast<uint32_t*>(orow)[d] = 0x7fc00000u;
    }
    return;
  }
  const long long pq = p0 + t;
  const KeyPos kpos = key_pos(a, layout, p0, row0, layout == 0 ? 0 : a.seq_offsets[b]);
  const int R = 2 * a.half;
  float qd[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    qd[u] = 0.f;
    if (d >= a.d_qk) continue;
    if (d < R) {
      const int r = (d < a.half) ? d : d - a.half;
      const double ang = (double)pq * pow(a.rope_theta, -(double)r / (double)a.half);
      double sd, cd;
      sincos(ang, &sd, &cd);
      const float cs = (float)cd, sn = (float)sd;
      qd[u] = (d < a.half) ? ld(q, d) * cs - ld(q, d + a.half) * sn
                           : ld(q, d) * cs + ld(q, d - a.half) * sn;
    } else {
      qd[u] = ld(q, d);
    }
  }
  float m = a.sink ? a.sink[h] : kNegInf;
  float l = (m > kNegInf) ? 1.f : 0.f;
  float od[4] = {0.f, 0.f, 0.f, 0.f};
  for (long long kk = 0; kk < len; ++kk) {
    const long long P = kpos(kk);
    if (P > pq || (a.window > 0 && P <= pq - a.window)) continue;
    const T* krow = kc + ((row0 + kk) * a.hkv + g) * (long long)a.d_qk;
    const T* vrow = vc + ((row0 + kk) * a.hkv + g) * (long long)a.d_v;
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = lane + 64 * u;
      if (d < a.d_qk) part += qd[u] * ld(krow, d);
    }
    const float sc = wave_sum(part) * a.scale;
    const float mn = fmaxf(m, sc);
    const float alpha = expf(m - mn);
    const float pj = expf(sc - mn);
    l = l * alpha + pj;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = lane + 64 * u;
      if (d < a.d_v) od[u] = od[u] * alpha + pj * ld(vrow, d);
    }
    m = mn;
  }
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    if (d < a.d_v) st(orow, d, od[u] * inv);
  }
}

// Ring caches of at most 160 slots in one launch: a workgroup per
// (sequence, kv head), wavefront w on slots 32 w .. 32 w + 31 (five
// wavefronts).  Every copy of a wavefront's slots goes out at once into its
// own LDS region (the single-token ring kernel's layout: K rows of 384 B
// with 16-byte chunk c at c ^ ((row >> 1) & 7), V rows of 256 B with 32-byte
// unit u at u ^ (row & 7)); the wavefront runs its (at most two) 16-key
// tiles over all T * G query columns of the kv head (NB blocks of 16) with
// the split kernel's visibility rule; the five partials (m, l, O) per
// column are merged in LDS with the sink added once, as the combine does.
constexpr int MR_ROWS = 32;                  // ring slots per wavefront
constexpr int MR_NW = 5;                     // wavefronts per workgroup
constexpr int MR_K = MR_ROWS * D * 2;        // 12 KB
constexpr int MR_V = MR_ROWS * DV * 2;       // 8 KB
constexpr int MR_REG = MR_K + MR_V;
static_assert(MR_REG >= 32 * DV * 4 + 64 * 4, "a region holds a wavefront's partial for the merge");

template <int NB>
__global__ __launch_bounds__(64 * MR_NW, 1) void decode_multi_ring_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char reg_all[MR_NW * MR_REG];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x, b = blockIdx.y;
  const int G = a.hq / a.hkv, T = a.nq, W = a.window;
  unsigned char* kreg = reg_all + wave * MR_REG;
  unsigned char* vreg = kreg + MR_K;

  long long p0, row0, len;
  if (!multi_range(a, 0, b, &p0, &row0, &len)) {   // uniform over the workgroup
    // a broken contract: NaN outputs (wavefronts 0..3 own 32 dims each)
    if (wave < 4) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = 16 * nb + c;
        if (n < T * G) {
          const int tn = n / G, hn = n - tn * G;
          bf16_t* orow = static_cast<bf16_t*>(a.o) +
                         (((long long)b * T + tn) * a.hq + g * G + hn) * DV + 32 * wave + 8 * grp;
          st16(orow, make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u));
        }
      }
    }
    return;
  }
  const int key0 = MR_ROWS * wave;             // this wavefront's first slot
  const int nk = (int)min((long long)MR_ROWS, max(0LL, len - key0));   // its valid slots
  const int klast = (int)len - 1;              // len >= 1 here

  // this lane's query columns: n = 16 nb + c (token n / G, head n % G);
  // columns n >= T * G repeat column 0 (their results are never stored).
  // Issued before the copies, so that q lands with tile 0.
  bf16x8 qf[NB][KS];
  int ctok[NB];
  bool cval[NB];
  {
    const bf16_t* qsrc = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = 16 * nb + c;
      cval[nb] = n < T * G;
      const int tn = cval[nb] ? n / G : 0, hn = cval[nb] ? n - tn * G : 0;
      ctok[nb] = tn;
      const bf16_t* qrow = qsrc + (((long long)b * T + tn) * a.hq + g * G + hn) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[nb][ks] = as_bf16x8(ld16(qrow + 32 * ks));
    }
  }

  // copies, tile by tile (slots 0..15, then 16..31 of the wavefront's
  // range); rows past the last valid slot reload the last one (finite data,
  // masked), and a wavefront with no valid slot reloads the ring's last
  // written slot, so every wavefront issues the same 20 copies and the waits
  // below count exactly
  {
    const unsigned char* kb = static_cast<const unsigned char*>(a.k) + (row0 * a.hkv + g) * (long long)(D * 2);
    const unsigned char* vb = static_cast<const unsigned char*>(a.v) + (row0 * a.hkv + g) * (long long)(DV * 2);
    const int kstr = a.hkv * D * 2, vstr = a.hkv * DV * 2;
    auto slot = [&](int row) { return min(key0 + min(row, nk - 1), klast); };
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int ii = 6 * t; ii < 6 * t + 6; ++ii) {
        const int sl = 64 * ii + lane;
        const int row = sl / 24, pc = sl - row * 24;
        const int lc = pc ^ ((row >> 1) & 7);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kb + (__umul24(slot(row), kstr) + 16 * lc)),
                                         (lds_void_t*)(kreg + 1024 * ii), 16, 0, 0);
      }
#pragma unroll
      for (int jj = 4 * t; jj < 4 * t + 4; ++jj) {
        const int sl = 64 * jj + lane;
        const int row = sl >> 4, pc = sl & 15;
        const int lc = 2 * ((pc >> 1) ^ (row & 7)) + (pc & 1);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(vb + (__umul24(slot(row), vstr) + 16 * lc)),
                                         (lds_void_t*)(vreg + 1024 * jj), 16, 0, 0);
      }
    }
  }
  static_assert(MR_K == 12 * 1024 && MR_V == 8 * 1024 && MR_ROWS == 2 * BK, "two tiles of 10 copies");

  const KeyPos kpos = key_pos(a, 0, p0, row0, 0);
  const float c2 = a.scale * kLog2e;
  float m[NB], l[NB];
  f32x4 acc[NT][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf;
    l[nb] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // one 16-key tile from the wavefront's region; its LDS reads are inline
  // asm that wait for their own data, so the compiler's wait analysis does
  // not add a wait for the copies still in flight
  auto tile = [&](int t) __attribute__((always_inline)) {
    // visibility of slot key0 + 16 t + 4 grp + r to column token tn, decided
    // before the score products (see the split kernel)
    bool vis[NB][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = BK * t + 4 * grp + r;
      const int rel = (int)(kpos(key0 + kk) - p0);
      const bool here = kk < nk;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vis[nb][r] = here & (rel <= ctok[nb]) & ((W == 0) | (rel > ctok[nb] - W));
    }
    f32x4 sc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kr = BK * t + c;
    uint32_t kad[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kad[ks] = lds_off(kreg + kr * (D * 2) + 16 * ((4 * ks + grp) ^ ((kr >> 1) & 7)));
    uint4 kw[KS];
    lds_b128x6(kw, kad);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc[nb] = mfma16(as_bf16x8(kw[ks]), qf[nb][ks], sc[nb]);
    }
    uint2 pk[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[nb][r] = vis[nb][r] ? sc[nb][r] : kNegInf;
      float mx = fmaxf(fmaxf(sc[nb][0], sc[nb][1]), fmaxf(sc[nb][2], sc[nb][3]));
      mx = max_across_groups(mx) * c2;
      const float mn = fmaxf(m[nb], mx);
      const float ms = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[nb] - ms);
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(fmaf(sc[nb][r], c2, -ms));
      pk[nb] = make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
      l[nb] = l[nb] * alpha + add_bf16_pair(pk[nb].y, add_bf16_pair(pk[nb].x, 0.f));
      m[nb] = mn;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[tt][nb] *= alpha;
    }
    const int vr = BK * t + 4 * grp + (c >> 2);
    uint32_t vad[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      vad[tt] = lds_off(vreg + vr * (DV * 2) + 32 * (tt ^ (vr & 7)) + 8 * (c & 3));
    uint2 vt[NT];
    lds_tr4x8(vt, vad);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[tt][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(v4i16_t, vt[tt]), __builtin_bit_cast(v4i16_t, pk[nb]), acc[tt][nb],
            0, 0, 0);
    }
  };
  static_assert(NT == 8 && KS == 6, "the read helpers take six K and eight V pieces");

  // q and tile 0's ten copies have landed once at most tile 1's ten are in
  // flight; tile 1 is computed after everything has landed
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(10));
  if (nk > 0) tile(0);                  // uniform
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (nk > BK) tile(1);                 // uniform

  // ---- merge: each wavefront leaves O [16 NB columns][128 dims], m and l
  // [16 NB] (fp32, base 2) in its own region; wavefronts 0..3 then write
  // dims 32 w .. 32 w + 31 of every column
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float* po = reinterpret_cast<float*>(kreg);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = sum_across_groups(l[nb]);
    const int n = 16 * nb + c;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<float4*>(po + n * DV + 16 * tt + 4 * grp) =
          make_float4(acc[tt][nb][0], acc[tt][nb][1], acc[tt][nb][2], acc[tt][nb][3]);
    if (grp == 0) {
      po[32 * DV + n] = m[nb];
      po[32 * DV + 32 + n] = lt;
    }
  }
  __syncthreads();
  if (wave < 4) {
    const int d0 = 32 * wave + 8 * grp;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = 16 * nb + c;
      const int hn = n - ctok[nb] * G;
      const float s2 = (cval[nb] && a.sink) ? a.sink[g * G + hn] * kLog2e : kNegInf;
      float mw[MR_NW], lw[MR_NW];
      float M = s2;
#pragma unroll
      for (int w = 0; w < MR_NW; ++w) {
        const float* pw = reinterpret_cast<const float*>(reg_all + w * MR_REG);
        mw[w] = pw[32 * DV + n];
        lw[w] = pw[32 * DV + 32 + n];
        M = fmaxf(M, mw[w]);
      }
      float den = (s2 > kNegInf) ? fast_exp2(s2 - M) : 0.f;
      float o8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = 0.f;
#pragma unroll
      for (int w = 0; w < MR_NW; ++w) {
        const float sw = (mw[w] > kNegInf) ? fast_exp2(mw[w] - M) : 0.f;
        den += sw * lw[w];
        const float* pw = reinterpret_cast<const float*>(reg_all + w * MR_REG) + n * DV + d0;
        const float4 x0 = *reinterpret_cast<const float4*>(pw);
        const float4 x1 = *reinterpret_cast<const float4*>(pw + 4);
        o8[0] += sw * x0.x; o8[1] += sw * x0.y; o8[2] += sw * x0.z; o8[3] += sw * x0.w;
        o8[4] += sw * x1.x; o8[5] += sw * x1.y; o8[6] += sw * x1.z; o8[7] += sw * x1.w;
      }
      if (cval[nb]) {
        const float inv = (den > 0.f) ? 1.f / den : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] *= inv;
        bf16_t* orow = static_cast<bf16_t*>(a.o) +
                       (((long long)b * T + ctok[nb]) * a.hq + g * G + hn) * DV + d0;
        st16(orow, pack8(o8));
      }
    }
  }
}

bool decode_multi_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && G >= 1 && a.nq * G <= 64 && a.hkv % HG == 0 &&
         2 * a.half <= D;
}

hipError_t launch_decode_multi(const AttnArgs& a, int layout, hipStream_t stream) {
  if (a.B == 0 || a.nq == 0) return hipSuccess;
  const dim3 rows((unsigned)a.hq, (unsigned)a.nq, (unsigned)a.B);
  if (a.half > 0) {
    hipLaunchKernelGGL(decode_multi_rope_q_kernel, rows, dim3(64), 0, stream, a, layout);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int cols = a.nq * (a.hq / a.hkv);
  // a ring of at most 160 slots and at most 32 columns per kv head: one launch
  if (layout == 0 && a.slots <= MR_NW * MR_ROWS && cols <= 32) {
    const dim3 gr((unsigned)a.hkv, (unsigned)a.B);
    if (cols <= 16)
      hipLaunchKernelGGL((decode_multi_ring_kernel<1>), gr, dim3(64 * MR_NW), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_multi_ring_kernel<2>), gr, dim3(64 * MR_NW), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 g1((unsigned)(a.hkv / HG), (unsigned)a.nsplit, (unsigned)a.B);
  // four stages once a split spans at least 32 tiles
  const bool deep = a.split_keys >= 32 * BK;
  if (cols <= 16) {
    if (deep) hipLaunchKernelGGL((decode_multi_split_kernel<1, 1, 4>), g1, dim3(256), 0, stream, a, layout);
    else hipLaunchKernelGGL((decode_multi_split_kernel<1, 1, 2>), g1, dim3(256), 0, stream, a, layout);
  } else if (cols <= 32) {
    if (deep) hipLaunchKernelGGL((decode_multi_split_kernel<2, 1, 4>), g1, dim3(256), 0, stream, a, layout);
    else hipLaunchKernelGGL((decode_multi_split_kernel<2, 1, 2>), g1, dim3(256), 0, stream, a, layout);
  } else {
    if (deep) hipLaunchKernelGGL((decode_multi_split_kernel<2, 2, 4>), g1, dim3(512), 0, stream, a, layout);
    else hipLaunchKernelGGL((decode_multi_split_kernel<2, 2, 2>), g1, dim3(512), 0, stream, a, layout);
  }
  {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_multi_combine_kernel, rows, dim3(64), 0, stream, a, layout);
  return hipGetLastError();
}

hipError_t launch_decode_multi_generic(const AttnArgs& a, int layout, bool bf16,
                                       hipStream_t stream) {
  if (a.B == 0 || a.nq == 0) return hipSuccess;
  const dim3 rows((unsigned)a.hq, (unsigned)a.nq, (unsigned)a.B);
  if (bf16)
    hipLaunchKernelGGL((decode_multi_generic_kernel<bf16_t>), rows, dim3(64), 0, stream, a, layout);
  else
    hipLaunchKernelGGL((decode_multi_generic_kernel<float>), rows, dim3(64), 0, stream, a, layout);
  return hipGetLastError();
}

}  // namespace hswa
