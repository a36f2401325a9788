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
// LDS serves all of them.  Each wavefront holds 32 rows: the 32 columns of
// one 32x32x16 MFMA operand (that shape issues twice the flops per cycle of
// the 16x16x32 one on gfx950).
//
// Orientation.  Scores are computed transposed, S^T = K . Q^T: one MFMA
// chain of 12 k-steps gives the wavefront's 32 rows against the tile's 32
// keys, a lane (i, h) holding row i against keys 8j + 4h + r (j, r < 4).
// Those 16 values are, lane for lane, the B operand of the next product
// O^T += V^T . P^T once its 32 keys are taken in that order, so P never
// leaves registers; V^T's A operand is read in the same key order.  The
// row max needs one cross-lane step (lanes i and i + 32).
//
// Softmax in base 2.  The fp32 scores are scaled by scale * log2(e) inside
// the exp2 argument (one FMA), so q is rounded to bf16 only where RoPE
// changed it; the sink is multiplied by log2(e) only.  The state starts at
// m = sink, l = 1 (one lane per row): the sink's exp(sink - m) term.  The
// reference max m moves only when a row's max exceeds it by more than
// kLazy (in log2 units); until then P = exp2(s - m) <= 2^kLazy, which fp32
// sums and bf16 P hold as well as values below 1, and neither the row max
// nor the rescale of O is needed.  O and l always share the same m, so
// o = O / l is unchanged.  Each lane adds the bf16 P it feeds the MFMA into
// l (v_dot2 against ones), so l sums exactly the weights applied to V.
//
// RoPE.  q is rotated in registers (pair d, d + R/2 sits in one lane when
// R/2 is a multiple of 16) from a cos/sin table; K's rotated dims were
// rotated once per call by the preparation kernel and are staged as is.
//
// Pipelining.  A wavefront computes S for tile t+1 in the same stretch of
// code as the softmax of tile t, then O += P(t) V(t): the MFMA chain of the
// scores runs while the exponentials are evaluated, instead of each waiting
// for the other.
//
// Staging.  K and V tiles go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane) through two rings of three stages,
// each stage its own LDS array.  In step t the wavefronts read K(t+1) and
// V(t) and request K(t+3) and V(t+2), so each load has two steps of work to
// land behind, and because the stages are distinct objects the compiler can
// tell that reads of one stage do not depend on loads still landing in
// another.  Rows are padded (K 400 B, V 320 B) so the MFMA operand reads
// hit distinct banks; the pad slots are filled from a valid address and
// never read.  V stays row-major: the A operand of the PV product is read
// with ds_read_b64_tr_b16, whose 16-lane transpose hands lane i the values
// V[k0 + k][d0 + i], k = 0..3, when lane j points at V[k0 + j/4][d0 +
// 4 * (j % 4)].  q goes straight to registers in the MFMA operand layout,
// its loads in flight together with the first three tiles.
#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

constexpr int D = 192;                 // q/k head dim
constexpr int DV = 128;                // v head dim
constexpr int KS = D / 16;             // k-steps of the 32x32x16 MFMA: 12
constexpr int MT = DV / 32;            // 32-row output tiles of O^T: 4
constexpr int BK = 32;                 // keys per staged tile
constexpr int ROWS = 128;              // query rows per workgroup
constexpr int KPITCH = D * 2 + 16;     // K row pitch in LDS (bytes)
constexpr int VPITCH = DV * 2 + 64;    // V row pitch in LDS (bytes)
constexpr int KSLOTS = KPITCH / 16;    // 25 16-byte slots per K row (24 data + pad)
constexpr int VSLOTS = VPITCH / 16;    // 20 per V row (16 data + 4 pad)
constexpr int KINSTR = (BK * KSLOTS + 63) / 64;   // 13 load instructions of 1 KB
constexpr int VINSTR = BK * VSLOTS / 64;          // 10
constexpr int KBYTES = KINSTR * 1024;             // 13312 per K stage
constexpr int VBYTES = VINSTR * 1024;             // 10240 per V stage
constexpr int NWAVE = 4;
// Every wavefront issues the same number of load instructions per tile, so
// one vmcnt value means "this tile has landed" on all of them; the one
// instruction past the 23 a tile needs reloads V slots into a spare 1 KB.
constexpr int DMA_PER_WAVE = (KINSTR + VINSTR + NWAVE - 1) / NWAVE;   // 6
constexpr int OPITCH = DV * 2 + 16;    // output row pitch in LDS (bytes) for the store transpose
static_assert(32 * OPITCH <= VBYTES, "a wavefront's outputs fit one V stage");
static_assert(DMA_PER_WAVE == 6, "vmcnt immediates below assume 6 loads per tile");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (lds_base uniform).
__device__ __forceinline__ void g2lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_base, 16, 0, 0);
}

// Workgroup barrier for the staging ring.  Unlike __syncthreads() it carries
// no release fence, which would wait for every tile load of this wavefront
// still in flight (they write LDS); the caller waits for the tile it needs
// with vmcnt first.  The empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr float kLazy = 8.f;
constexpr float kLazyPow = 256.f;      // 2^kLazy

// Rotate the rotary k-steps of q (pair (ka, ka + PK) sits in one lane, dims
// 16 ka + 8 h + e and + R/2) and round them to bf16; the other k-steps keep
// their exact input values.
template <int PK>
__device__ __forceinline__ void rotate_q(bf16x8 (&qf)[KS], const uint4 (&raw)[KS],
                                         const float2* __restrict__ trow, int h) {
#pragma unroll
  for (int ka = 0; ka < PK; ++ka) {
    const float2* t = trow + 16 * ka + 8 * h;
    float x0[8], x1[8];
    unpack8(raw[ka], x0);
    unpack8(raw[ka + PK], x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = t[e];
      const float y0 = x0[e] * cs.x - x1[e] * cs.y;
      const float y1 = x1[e] * cs.x + x0[e] * cs.y;
      x0[e] = y0;
      x1[e] = y1;
    }
    qf[ka] = as_bf16x8(pack8(x0));
    qf[ka + PK] = as_bf16x8(pack8(x1));
  }
}

}  // namespace

// 4 wavefronts of 32 rows per workgroup, 2 workgroups (2 wavefronts per
// SIMD) per CU.
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(AttnArgs a, int log2g, int nblk,
                                                              int balance) {
  __shared__ __attribute__((aligned(16))) unsigned char kst0[KBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kst1[KBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kst2[KBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char vst0[VBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char vst1[VBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char vst2[VBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char spare[1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 31, h = lane >> 5;

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
  const int hkv = a.hkv;

  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ Kr = static_cast<const bf16_t*>(a.krot);
  const bf16_t* __restrict__ Vp = static_cast<const bf16_t*>(a.v);
  bf16_t* __restrict__ Op = static_cast<bf16_t*>(a.o);

  // ---- key range of the workgroup ----------------------------------------
  const int W = a.window;
  const int kstart = (W > 0) ? max(0, i0 - W + 1) : 0;
  const int kend = min(n, i0 + T);
  const int ntiles = (kend - kstart + BK - 1) / BK;

  // ---- this lane's six 16-byte slots of every tile ------------------------
  // Load instruction ii = wave + 4u (u = 0..5) of a step fills 1 KB of a
  // stage.  ii < 13: K slot s = 64 ii + lane (row s / 25, chunk s % 25) at
  // byte 1024 ii of a K stage; 13 <= ii < 23: V slot s = 64 (ii - 13) + lane
  // (row s / 20, chunk s % 20) at byte 1024 (ii - 13) of a V stage; ii = 23
  // repeats V instruction 13 into the spare buffer.  Pad slots load chunk 0
  // of their row.  K chunk ch < R/8 comes from the rotated copy (row pitch
  // R), the rest from K (pitch D).  Rows past kend load row kend - 1:
  // finite, and masked out.  Tiles past the last are requested as well (all
  // rows kend - 1, so they cost little) to keep exactly one step's loads in
  // flight behind the ones waited for: the vmcnt of every step is then the
  // same constant, on every path through the loop.
  const int rchunks = a.half >> 2;
  const unsigned char* dsrc[DMA_PER_WAVE];   // address of this slot's chunk at key 0
  int drow[DMA_PER_WAVE];                    // row within the tile
  int dstride[DMA_PER_WAVE];                 // bytes from one key to the next
#pragma unroll
  for (int u = 0; u < DMA_PER_WAVE; ++u) {
    const int ii = wave + NWAVE * u;
    int row, ch, pitch;
    const bf16_t* base;
    if (ii < KINSTR) {
      const int sl = 64 * ii + lane;
      row = sl / KSLOTS;
      ch = sl - row * KSLOTS;
      if (row >= BK) { row = BK - 1; ch = 0; }
      if (ch >= D / 8) ch = 0;
      const bool rot = ch < rchunks;
      pitch = rot ? 2 * a.half : D;
      base = rot ? Kr : Kp;
    } else {
      const int sl = (ii < KINSTR + VINSTR) ? 64 * (ii - KINSTR) + lane : lane;
      row = sl / VSLOTS;
      ch = sl - row * VSLOTS;
      if (ch >= DV / 8) ch = 0;
      pitch = DV;
      base = Vp;
    }
    dsrc[u] = reinterpret_cast<const unsigned char*>(base + (tokbase * hkv + g) * pitch + 8 * ch);
    drow[u] = row;
    dstride[u] = hkv * pitch * 2;
  }
  // K slots of the tile at key jk into kdst, V slots of the tile at jv into vdst
  auto issue = [&](int jk, unsigned char* kdst, int jv, unsigned char* vdst) {
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int ii = wave + NWAVE * u;
      const bool isk = ii < KINSTR;
      const int key = min((isk ? jk : jv) + drow[u], kend - 1);
      unsigned char* dst = isk ? kdst + 1024 * ii
                               : (ii < KINSTR + VINSTR) ? vdst + 1024 * (ii - KINSTR) : spare;
      g2lds16(dsrc[u] + (long long)key * dstride[u], dst);
    }
  };
  auto issue_k = [&](int jk, unsigned char* kdst) {   // K slots only (prologue)
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u) {
      const int ii = wave + NWAVE * u;
      if (ii < KINSTR)
        g2lds16(dsrc[u] + (long long)min(jk + drow[u], kend - 1) * dstride[u], kdst + 1024 * ii);
    }
  };

  // ---- the query row of this lane ----------------------------------------
  const int r = wave * 32 + i;
  const int tok = i0 + (r >> log2g);
  const int head = g * G + (r & (G - 1));
  const bool rv = tok < n;
  const int tw0 = i0 + ((wave * 32) >> log2g);
  const int tw1 = min(n - 1, i0 + ((wave * 32 + 31) >> log2g));

  // ---- prologue: K0..K2, V0, V1 requested, then q and its rotation ---------
  issue(kstart, kst0, kstart, vst0);
  issue(kstart + BK, kst1, kstart + BK, vst1);
  issue_k(kstart + 2 * BK, kst2);

  bf16x8 qf[KS];
  {
    const bf16_t* qrow = Qp + ((tokbase + (rv ? tok : n - 1)) * a.hq + head) * D + 8 * h;
    uint4 qraw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qraw[ks] = ld16(qrow + 16 * ks);
      qf[ks] = as_bf16x8(qraw[ks]);
    }
    if (a.half > 0 && rv) {
      const float2* trow = a.rope + (long long)tok * a.half;
      switch (a.half >> 4) {
        case 1: rotate_q<1>(qf, qraw, trow, h); break;
        case 2: rotate_q<2>(qf, qraw, trow, h); break;
        case 3: rotate_q<3>(qf, qraw, trow, h); break;
        case 4: rotate_q<4>(qf, qraw, trow, h); break;
        case 5: rotate_q<5>(qf, qraw, trow, h); break;
        default: rotate_q<6>(qf, qraw, trow, h); break;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): q and the prologue's tiles have landed

  // ---- softmax state seeded with the sink -------------------------------
  const float c2 = a.scale * kLog2e;   // raw score -> base-2 units
  const float s2 = a.sink ? a.sink[head] * kLog2e : kNegInf;
  float m = s2;
  float l = (h == 0 && s2 > kNegInf) ? 1.f : 0.f;   // this lane's share of the row sum
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;

  // per-lane LDS offsets of the MFMA operands
  const int koffA = i * KPITCH + h * 16;                       // K row i, chunk 2 ks + h
  const int jv = lane & 15;                                    // lane within its 16-lane group
  const int voffA = (4 * h + (jv >> 2)) * VPITCH +             // transpose origin: key 4h + jv/4,
                    (16 * ((lane >> 4) & 1) + 4 * (jv & 3)) * 2;   // column 16 (i/16) + 4 (jv%4)

  auto scores = [&](const unsigned char* kst) __attribute__((always_inline)) {
    f32x16 sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma32(as_bf16x8(ld16(kst + koffA + 32 * ks)), qf[ks], sc);
    return sc;
  };

  // ---- step t: wait, request K(t+3) and V(t+2), softmax of tile t with the
  // scores of tile t+1 alongside, then O += P(t) V(t) ----------------------
  // At the top of step t the loads pending are at most those requested in
  // steps t-1 and t-2 (six per wavefront each); the ones step t reads, K(t+1)
  // and V(t), came from step t-2 (or the prologue), so vmcnt <= 6 means they
  // have landed for this wavefront.  The barrier then covers the others and
  // ends every read of K(t) and V(t-1), whose stages the new requests reuse.
  stage_barrier();           // every wavefront's share of the prologue tiles has landed
  f32x16 s = scores(kst0);   // tile 0
  auto step = [&](int t, const unsigned char* knext, const unsigned char* vcur,
                  unsigned char* kput, unsigned char* vput) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6)
    stage_barrier();
    issue(kstart + (t + 3) * BK, kput, kstart + (t + 2) * BK, vput);
    const int j0 = kstart + t * BK;
    const bool need_mask = (j0 + BK - 1 > tw0) || (W > 0 && j0 < tw1 - W + 1);
    if (need_mask) {
      // key j0 + 4h + kk (kk = 8j + r) is visible iff dlo <= kk <= dhi
      const int dhi = tok - (j0 + 4 * h);
      const int dlo = (W > 0) ? dhi - (W - 1) : -0x7fffffff;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = 8 * (v >> 2) + (v & 3);
        if (kk > dhi || kk < dlo) s[v] = kNegInf;
      }
    }

    // -- online softmax (base 2, lazy reference max) and P in bf16 --------
    // Fast path: P against the current reference m, checked lane-locally.
    // A row with no reference yet, or with a P above 2^kLazy, sends the
    // whole wave through the slow path: exact row max across the two lanes
    // of each row, rescale of O and l, and P again.
    float p[16];
    float ms = (m == kNegInf) ? 0.f : m;
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(s[v], c2, -ms));
    float pm = p[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) pm = fmaxf(pm, p[v]);
    const bool slow = __any(m == kNegInf || pm > kLazyPow);
    // scores of the next tile (none after the last)
    f32x16 sn;
    if (t + 1 < ntiles) sn = scores(knext);
    if (slow) {
      float mx = s[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
      const float mn = fmaxf(m, mx);
      if (mn > m) {
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
        m = mn;
      }
      ms = (m == kNegInf) ? 0.f : m;
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(s[v], c2, -ms));
    }
    // B operand of k-step kk: keys 16 kk + 8 (e / 4) + 4h + e % 4 = p[8 kk + e]
    const uint4 pb0 = pack8(p), pb1 = pack8(p + 8);
    l = add_bf16_pair(pb0.x, l); l = add_bf16_pair(pb0.y, l);
    l = add_bf16_pair(pb0.z, l); l = add_bf16_pair(pb0.w, l);
    l = add_bf16_pair(pb1.x, l); l = add_bf16_pair(pb1.y, l);
    l = add_bf16_pair(pb1.z, l); l = add_bf16_pair(pb1.w, l);

    // -- O^T += V^T . P^T, V^T read with the transpose loads in that key order
    const unsigned char* vb = vcur + voffA;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint2 lo = lds_tr4(vb + 16 * kk * VPITCH + 64 * mt);
        const uint2 hi = lds_tr4(vb + (16 * kk + 8) * VPITCH + 64 * mt);
        const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[mt] = mfma32(vf, as_bf16x8(kk ? pb1 : pb0), acc[mt]);
      }
    }
    s = sn;
  };

  // K(t) sits in K stage t % 3, V(t) in V stage t % 3 (ntiles >= 1 always)
  int t = 0;
  for (; t + 3 <= ntiles; t += 3) {
    step(t, kst1, vst0, kst0, vst2);
    step(t + 1, kst2, vst1, kst1, vst0);
    step(t + 2, kst0, vst2, kst2, vst1);
  }
  if (t < ntiles) {
    step(t, kst1, vst0, kst0, vst2);
    if (t + 1 < ntiles) step(t + 1, kst2, vst1, kst1, vst0);
  }

  // ---- epilogue: o = O / l, rounded to bf16 -----------------------------
  // The O^T fragments go through LDS (one wavefront per V stage or the
  // spare-padded K stage; the fence of the barrier waits for the last tile
  // requests, and the barrier ends every read of the stages) so that the
  // global stores are 16 bytes per lane and each instruction covers four
  // whole 256-byte rows.
  const float lt = l + __shfl_xor(l, 32);
  const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
  __syncthreads();
  unsigned char* obuf = wave == 0 ? vst0 : wave == 1 ? vst1 : wave == 2 ? vst2 : kst0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 w = make_uint2(pack_bf16x2(acc[mt][4 * j] * inv, acc[mt][4 * j + 1] * inv),
                                 pack_bf16x2(acc[mt][4 * j + 2] * inv, acc[mt][4 * j + 3] * inv));
      st8(obuf + i * OPITCH + (32 * mt + 8 * j + 4 * h) * 2, w);
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int it = 0; it < 32 * (DV / 8) / 64; ++it) {
    const int idx = lane + 64 * it;
    const int rr = idx >> 4, ch = idx & 15;       // row of this wavefront, 16-byte chunk
    const int rw = wave * 32 + rr;
    const int tk = i0 + (rw >> log2g);
    if (tk < n) {
      const int hd = g * G + (rw & (G - 1));
      st16(Op + ((tokbase + tk) * a.hq + hd) * DV + 8 * ch, ld16(obuf + rr * OPITCH + 16 * ch));
    }
  }
}

bool prefill_bf16_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && G >= 1 && G <= ROWS && (G & (G - 1)) == 0 &&
         (a.half % 16) == 0 && 2 * a.half <= D;
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
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)total), dim3(256), 0, stream, a,
                     log2g, nblk, balance);
  return hipGetLastError();
}

}  // namespace hswa
