// Persistent bf16 prefill for the common shapes (GQA group >= 8, rotary
// half-width <= 32): the same operation as prefill_bf16.hip ("MiMo-V2-Flash:
// Hybrid Sliding Window Attention Architecture" (rslog.cc) sections 2.1,
// 2.3, 4.4 and 5), organised so that the HBM stream of one work item
// overlaps the arithmetic of the previous one.
//
// Work.  One workgroup of 8 wavefronts per CU (two per SIMD) walks a
// sequence of items.  An item is one kv head g and T = 256 / G consecutive
// query tokens: 256 rows (tokens x the G query heads of group g), 32 per
// wavefront.  Items go out in rounds of one per workgroup, numbered so that
// the 32 workgroups of an XCD take neighbouring token blocks of one head
// (their K/V tiles overlap and are fetched once into that XCD's L2), with
// the order reversed every other round so that long and short causal rows
// even out per workgroup.
//
// Overlap.  Wavefronts 4..7 copy the K/V tiles of 32 keys into two
// three-stage LDS rings with global_load_lds, two tiles ahead, as one
// stream across item boundaries; wavefronts 0..3 copy the next item's q
// block (256 rows x 384 B) into LDS in four parts during the first tiles of
// the current item.  The split keeps each wavefront's in-order memory
// counter free of the other kind of copy: a wait for a tile that hits L2
// never also waits for a q block coming from HBM.  Every wavefront waits
// for its own copies and then meets the others at a barrier per tile.  q is
// rotated in registers with cos/sin evaluated in the kernel (fp64 angle in
// revolutions, reduced, then the hardware sine/cosine).  Outputs leave
// straight from registers: the V^T operand is read with its rows permuted
// so that each lane ends up holding 16 consecutive output dims, stored as
// two 16-byte writes.
//
// Arithmetic per tile is that of prefill_bf16.hip: S^T = K . Q^T on the
// 32x32x16 MFMA (a lane holds row i against keys 8j + 4h + r), base-2 online
// softmax seeded with the sink and a lazily moved reference max, l summed
// from the bf16 P with v_dot2, O^T += V^T . P^T.
//
// LDS layout (unpadded rows, XOR swizzles applied on the global side of the
// copies so that the MFMA operand reads hit distinct banks):
//   q buffer   256 rows x 384 B   16-byte chunk c of row r at c ^ ((r >> 1) & 7)
//   K stage     32 rows x 384 B   same swizzle as q
//   V stage     32 rows x 256 B   64-byte unit u of row r at u ^ (r & 3)
#include "common.h"
#include "launch.h"
#include "tile_ops.h"

namespace hswa {
namespace {

constexpr int NW = 8;                  // wavefronts per workgroup
constexpr int ROWS = 32 * NW;          // 256 query rows per item
constexpr int QBUF = ROWS * KROW;      // 96 KB = 96
constexpr int KSTAGES = 3;
constexpr int VSTAGES = 3;

// One item: kv head g of sequence b, the query tokens at sequence positions
// [i0, i0 + T).  The queries are the last nq of the n positions (qoff =
// n - nq), so the q / o row of position p is qbase + p and the K / V row of
// key position j is kbase + j.
struct Item {
  long long kbase;   // b * n
  long long qbase;   // b * nq - qoff
  int g, i0, kstart, kend, ntiles;
};

__device__ __forceinline__ Item make_item(const AttnArgs& a, int k, int nblk, int T) {
  Item it;
  const int bg = k / nblk;
  const int blk = k - bg * nblk;
  const int b = bg / a.hkv;
  it.g = bg - b * a.hkv;
  it.kbase = (long long)b * a.n;
  it.qbase = (long long)b * a.nq - a.qoff;
  it.i0 = a.qoff + blk * T;
  it.kstart = (a.window > 0) ? max(0, it.i0 - a.window + 1) : 0;
  it.kend = min(a.n, it.i0 + T);
  it.ntiles = (it.kend - it.kstart + BK - 1) / BK;
  return it;
}

// Item of round j for the workgroup at position pos of P: the items go out
// in rounds of P consecutive indices, the position reversed every other
// round, so that (causal layer) the long and short blocks of successive
// rounds even out per workgroup.  Positions are numbered XCD by XCD, so the
// workgroups of one XCD work on neighbouring blocks of one head at the same
// time and share their K/V tiles in that XCD's L2.
__device__ __forceinline__ int item_of(int j, int pos, int P) {
  return j * P + ((j & 1) ? P - 1 - pos : pos);
}

}  // namespace

__global__ __launch_bounds__(512, 1) void prefill_persist_kernel(AttnArgs a, int log2g, int nblk,
                                                                 int items) {
  __shared__ __attribute__((aligned(16))) unsigned char qbuf[QBUF];
  __shared__ __attribute__((aligned(16))) unsigned char kring[KSTAGES * KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char vring[VSTAGES * VTILE];
  __shared__ float sinkbuf[MAX_HQ];
  __shared__ double revbuf[MAX_HALF];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i = lane & 31, h = lane >> 5;
  const int G = 1 << log2g;
  const int T = ROWS >> log2g;
  const int n = a.n, hkv = a.hkv, hq = a.hq;
  const int W = a.window;
  const int half = a.half;
  const int R = 2 * half;

  // this workgroup's items
  const int P = gridDim.x;
  // hardware dispatch sends workgroup b to XCD b % 8
  const int pos = (P % 8 == 0) ? (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  if (item_of(0, pos, P) >= items) return;   // uniform over the workgroup

  // sink of every head in log2 units, read once before any copy is in flight
  for (int j = tid; j < hq; j += NW * 64) sinkbuf[j] = a.sink ? a.sink[j] * kLog2e : kNegInf;
  // rotary frequency of pair p in revolutions per position
  if (tid < half) revbuf[tid] = pow(a.rope_theta, -(double)tid / (double)half) * 0.15915494309189535;
  __syncthreads();

  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ Kr = static_cast<const bf16_t*>(a.krot);
  const bf16_t* __restrict__ Vp = static_cast<const bf16_t*>(a.v);
  bf16_t* __restrict__ Op = static_cast<bf16_t*>(a.o);

  // ---- copy duties -----------------------------------------------------------
  // Wavefronts 4..7 copy the K/V tiles, wavefronts 0..3 the q blocks.  The
  // vector-memory counter of a wavefront retires in issue order, so a wait
  // for a tile never also waits for a q block still coming from HBM.
  const bool tile_wave = wave >= NW / 2;
  const int cw = tile_wave ? wave - NW / 2 : wave;   // index within the duty group

  // A tile is 12 K copies and 8 V copies; tile wavefront cw issues copies
  // c = cw + 4u, u = 0..4 (u < 3: K copy c, else V copy c - 12).
  // K copy c: slot s = 64 c + lane, row s / 24, physical chunk s % 24 holding
  // logical chunk pc ^ ((row >> 1) & 7); chunks below R/8 come from the
  // rotated copy (row pitch R), the rest from K (pitch D).  V copy c: slot
  // s = 64 c + lane, row s / 16, physical chunk pc = s % 16 of 64-byte unit
  // pc / 4 holding logical unit (pc / 4) ^ (row & 3).  Offsets are in
  // elements from the tile's first row.
  constexpr int TCOPY = (KTILE + VTILE) / 1024 / (NW / 2);   // 5 per tile wavefront
  static_assert(TCOPY == 5 && KTILE / 1024 == 3 * (NW / 2), "copy split");

  // ---- the K/V stream: tiles of consecutive items, two ahead ----------------
  // (pj, pt) is the next tile to request.  Past the last item the last tile
  // is requested again (finite data, never read).  Tile u goes to stage
  // u % 3 of the K and of the V ring.
  int nis = 0;   // vector-memory operations issued by this wavefront so far
  int pj = 0, pt = 0;   // round and tile of the next request
  int kput = 0, vput = 0;   // stages of the next request
  Item pc = make_item(a, item_of(0, pos, P), nblk, T);
  // per-lane constants of the five tile copies (elements from the tile's
  // first row; the row is clamped to the item's last key at issue)
  int krow[3], kcol[3], kstr[3], vrow[2], vcol[2];
  bool krot[3];
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int c = cw + 4 * u;
    const int sl = 64 * c + lane;
    const int row = sl / 24, pc = sl - row * 24;
    const int lc = pc ^ ((row >> 1) & 7);
    krot[u] = !a.k_rotated && lc < (half >> 2);   // keys stored rotated: every dim from K
    krow[u] = row;
    kcol[u] = 8 * lc;
    kstr[u] = hkv * (krot[u] ? R : D);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = cw + 4 * u;
    const int sl = 64 * c + lane;
    const int row = sl >> 4, pc = sl & 15;
    vrow[u] = row;
    vcol[u] = 8 * (4 * ((pc >> 2) ^ (row & 3)) + (pc & 3));
  }
  auto request_next = [&]() {
    if (tile_wave) {
      const int j0 = pc.kstart + pt * BK;
      const int lim = pc.kend - 1 - j0;
      const long long rb = (pc.kbase + j0) * hkv + pc.g;
      const bf16_t* kb = Kp + rb * D;
      const bf16_t* rbp = Kr + rb * R;
      const bf16_t* vb = Vp + rb * DV;
      unsigned char* kd = kring + kput * KTILE;
      unsigned char* vd = vring + vput * VTILE;
#pragma unroll
      for (int u = 0; u < 3; ++u)
        g2lds16((krot[u] ? rbp : kb) + (min(krow[u], lim) * kstr[u] + kcol[u]), kd + 1024 * (cw + 4 * u));
#pragma unroll
      for (int u = 0; u < 2; ++u)
        g2lds16(vb + (min(vrow[u], lim) * (hkv * DV) + vcol[u]), vd + 1024 * (cw + 4 * u));
      asm volatile("" ::: "memory");
      nis += TCOPY;
    }
    kput = (kput == KSTAGES - 1) ? 0 : kput + 1;
    vput = (vput == VSTAGES - 1) ? 0 : vput + 1;
    if (pt + 1 < pc.ntiles) {
      ++pt;
    } else if (item_of(pj + 1, pos, P) < items) {
      ++pj;
      pt = 0;
      pc = make_item(a, item_of(pj, pos, P), nblk, T);
    }
  };
  // Part `part` (0..3) of the q copies of item `c`, issued by the q
  // wavefronts: copies ii = cw + 4j, j = 6 part .. 6 part + 5 (slot
  // s = 64 ii + lane, row s / 24, physical chunk s % 24, swizzled as K).
  // The parts are spread over the first tiles of the previous item.
  constexpr int QPARTS = 4;
  constexpr int QCOPY = QBUF / 1024 / (NW / 2) / QPARTS;   // 6 per part
  static_assert(QCOPY * QPARTS * (NW / 2) * 1024 == QBUF && QCOPY % 3 == 0, "q copies split evenly");
  // q copy j of a q wavefront covers slots 64 (cw + 4j) + lane: row and
  // chunk step by (10, +16) or (11, -8) per copy (256 slots of 24 chunks)
  const int qsl0 = 64 * cw + lane;
  const int qrow0 = qsl0 / 24, qpc0 = qsl0 - qrow0 * 24;
  auto issue_q = [&](const Item& c, int part) {
    if (!tile_wave) {
      const bf16_t* qb = Qp + ((c.qbase + c.i0) * hq + c.g * G) * (long long)D;
      const int tlim = n - 1 - c.i0;
      int row = qrow0 + (QCOPY * 32 / 3) * part, pc = qpc0;   // QCOPY copies = QCOPY * 32 / 3 rows
#pragma unroll
      for (int jj = 0; jj < QCOPY; ++jj) {
        const int ii = cw + (NW / 2) * (QCOPY * part + jj);
        const int lc = pc ^ ((row >> 1) & 7);
        const int tk = min(row >> log2g, tlim);
        g2lds16_nt(qb + ((tk * hq + (row & (G - 1))) * D + 8 * lc), qbuf + 1024 * ii);
        const bool wrap = pc >= 8;
        row += wrap ? 11 : 10;
        pc += wrap ? -8 : 16;
      }
      asm volatile("" ::: "memory");
      nis += QCOPY;
    }
  };

  // qmark: nis after the latest q copy; ma, mb: nis after the copies of the
  // next two tiles to be consumed (each only advances in the wavefronts
  // that issue those copies)
  for (int part = 0; part < QPARTS; ++part) issue_q(pc, part);
  int qmark = nis;
  request_next();
  int ma = nis;
  request_next();
  int mb = nis;

  // per-lane LDS offsets of the operand reads.  Row r of K and q holds
  // logical chunk c at physical chunk c ^ ((r >> 1) & 7); for k-step
  // ks = 4q + j this lane (row i, half h) reads chunk 8q + 2 (j ^ s1) + h1.
  const int sw = (i >> 1) & 7;
  const int s1 = sw >> 1, h1 = h ^ (sw & 1);
  uint32_t krd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) krd[j] = i * KROW + 16 * (2 * (j ^ s1) + h1);
  const uint32_t qrow = lds_addr(qbuf) + (wave * 32) * KROW;
  // transposed V read: key row 4h + jv/4 (+ 16 kk, + 8), 8-byte piece jv % 4
  // at dim 16 (p & 1) + 4 (p >> 1) + 8 ihi of the 32-dim tile, so that lane
  // (i, h) receives dims 16 h + 0..15 of each tile in its 16 outputs; the
  // 64-byte unit of output tile mt in that row is mt ^ (row & 3) = mt ^ (jv / 4)
  const int jv = lane & 15, ihi = (lane >> 4) & 1;
  uint32_t vrd[4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    vrd[mt] = (4 * h + (jv >> 2)) * VROW + 32 * (jv & 1) + 8 * ((jv >> 1) & 1) + 16 * ihi +
              64 * (mt ^ (jv >> 2));
  const uint32_t kring0 = lds_addr(kring), vring0 = lds_addr(vring);

  const float c2 = a.scale * kLog2e;
  int kget = 0, vget = 0;   // stages of the next tile to consume

  for (int j = 0; item_of(j, pos, P) < items; ++j) {
    const Item c = make_item(a, item_of(j, pos, P), nblk, T);
    const bool has_next = item_of(j + 1, pos, P) < items;
    const Item cn = make_item(a, has_next ? item_of(j + 1, pos, P) : item_of(j, pos, P), nblk, T);
    const int r = wave * 32 + i;
    const int tok = c.i0 + (r >> log2g);
    const int head = c.g * G + (r & (G - 1));
    const bool rv = tok < n;
    const int tw0 = c.i0 + ((wave * 32) >> log2g);
    const int tw1 = min(n - 1, c.i0 + ((wave * 32 + 31) >> log2g));

    float m = sinkbuf[head];
    float l = (h == 0 && m > kNegInf) ? 1.f : 0.f;
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;
    u32x4 qf[KS];

    // S^T = K . Q^T of the tile at LDS address kaddr (one accumulation chain;
    // the other wavefront of the SIMD fills its dependency gaps)
    f32x16 sa;
    auto scores = [&](uint32_t kaddr) __attribute__((always_inline)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sa[v] = 0.f;
      u32x4 kf[KS];
      lds_ksteps_lo(kf, kaddr + krd[0], kaddr + krd[1], kaddr + krd[2], kaddr + krd[3]);
#pragma unroll
      for (int ks = 0; ks < 6; ++ks)
        sa = mfma32(__builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, qf[ks]), sa);
      lds_ksteps_hi(kf, kaddr + krd[0], kaddr + krd[1], kaddr + krd[2], kaddr + krd[3]);
#pragma unroll
      for (int ks = 6; ks < KS; ++ks)
        sa = mfma32(__builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, qf[ks]), sa);
    };

    // Softmax of tile t (scores in sa) and O^T += V^T . P^T with its V
    // rows at LDS address vaddr.  The first half of the V^T operand is read
    // before the softmax, while the score products may still be running.
    auto finish = [&](int t, uint32_t vaddr) __attribute__((always_inline)) {
      u32x2 vf[8];
      lds_vhalf<0>(vf, vaddr + vrd[0], vaddr + vrd[1], vaddr + vrd[2], vaddr + vrd[3]);
      f32x16 x = sa;
      const int j0 = c.kstart + t * BK;
      if ((j0 + BK - 1 > tw0) || (W > 0 && j0 < tw1 - W + 1)) {
        // key j0 + 4h + kk (kk = 8j + r) is visible iff dlo <= kk <= dhi
        const int dhi = tok - (j0 + 4 * h);
        const int dlo = (W > 0) ? dhi - (W - 1) : -0x7fffffff;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 8 * (v >> 2) + (v & 3);
          x[v] = (kk > dhi || kk < dlo) ? kNegInf : x[v];
        }
      }
      // x = s * c2 - ms; the slow path (reference max unset or more than
      // kLazy below the row max) moves m, rescales O and l, and shifts x
      const float ms = (m == kNegInf) ? 0.f : m;
      float xm = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[v] = fmaf(x[v], c2, -ms);
        xm = fmaxf(xm, x[v]);
      }
      if (__any(m == kNegInf || xm > kLazy)) {
        // keep the PV products issued before at a safe distance from the
        // VALU reads of their results below
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        const float mx = fmaxf(xm, __shfl_xor(xm, 32)) + ms;
        const float mn = fmaxf(m, mx);
        if (mn > m) {
          const float alpha = fast_exp2(m - mn);
          l *= alpha;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
          m = mn;
        }
        const float shift = ms - ((m == kNegInf) ? 0.f : m);
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] += shift;
        asm volatile("s_nop 4" ::: "memory");
      }
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = fast_exp2(x[v]);
      const uint4 pb0 = pack8(p), pb1 = pack8(p + 8);
      l = add_bf16_pair(pb0.x, l); l = add_bf16_pair(pb0.y, l);
      l = add_bf16_pair(pb0.z, l); l = add_bf16_pair(pb0.w, l);
      l = add_bf16_pair(pb1.x, l); l = add_bf16_pair(pb1.y, l);
      l = add_bf16_pair(pb1.z, l); l = add_bf16_pair(pb1.w, l);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = mfma32(as_bf16x8(make_uint4(vf[2 * mt][0], vf[2 * mt][1], vf[2 * mt + 1][0],
                                              vf[2 * mt + 1][1])),
                         as_bf16x8(pb0), acc[mt]);
      lds_vhalf<1>(vf, vaddr + vrd[0], vaddr + vrd[1], vaddr + vrd[2], vaddr + vrd[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = mfma32(as_bf16x8(make_uint4(vf[2 * mt][0], vf[2 * mt][1], vf[2 * mt + 1][0],
                                              vf[2 * mt + 1][1])),
                         as_bf16x8(pb1), acc[mt]);
    };

    // Tile t: wait until it (and, for t = 0, this item's q) has landed; the
    // barrier then also retires stage (t - 1) of both rings for every
    // wavefront, so tile t + 2 can be requested into it.
    for (int t = 0; t < c.ntiles; ++t) {
      if (tile_wave) wait_copy(nis - ma);
      else if (t == 0) wait_copy(nis - qmark);
      ring_barrier();
      request_next();
      ma = mb;
      mb = nis;
      if (t == 0) {
        lds_ksteps_lo(qf, qrow + krd[0], qrow + krd[1], qrow + krd[2], qrow + krd[3]);
        lds_ksteps_hi(qf, qrow + krd[0], qrow + krd[1], qrow + krd[2], qrow + krd[3]);
        if (half > 0) {
          const double pos = (double)(a.pos_offset + tok);
          if (half == 16) rotate_q<1>(qf, revbuf, pos, h);
          else rotate_q<2>(qf, revbuf, pos, h);
        }
      } else if (has_next && t <= QPARTS) {
        // every wavefront has passed the barrier after its q reads
        issue_q(cn, t - 1);
        qmark = nis;
      }
      const uint32_t kaddr = kring0 + kget * KTILE;
      const uint32_t vaddr = vring0 + vget * VTILE;
      kget = (kget == KSTAGES - 1) ? 0 : kget + 1;
      vget = (vget == VSTAGES - 1) ? 0 : vget + 1;
      scores(kaddr);
      finish(t, vaddr);
    }
    if (has_next && c.ntiles <= QPARTS) {
      // the q parts not yet requested (short items); with a single tile no
      // barrier has followed the q reads yet
      if (c.ntiles == 1) ring_barrier();
      for (int part = c.ntiles - 1; part < QPARTS; ++part) issue_q(cn, part);
      qmark = nis;
    }

    // ---- output: o = O / l in bf16, 16 consecutive dims per lane per tile --
    // pad the distance from the last PV product to the first VALU read of
    // its result explicitly (the loop above ends in branches)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const float lt = l + __shfl_xor(l, 32);
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
    if (tw0 < n) {   // the wavefront's first row is a real token: 8 stores issued
      if (rv) {
        bf16_t* orow = Op + ((c.qbase + tok) * hq + head) * DV + 16 * h;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          float f[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) f[v] = acc[mt][v] * inv;
          st16(orow + 32 * mt, pack8(f));
          st16(orow + 32 * mt + 8, pack8(f + 8));
        }
      }
      asm volatile("" ::: "memory");
      nis += 2 * MT;
    }
  }
  __builtin_amdgcn_s_waitcnt(VMCNT(0));   // no copy into LDS outlives the workgroup
}

bool prefill_persist_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && a.hq == G * a.hkv && G >= 8 && G <= ROWS &&
         (G & (G - 1)) == 0 && a.hq <= MAX_HQ && (a.half == 0 || a.half == 16 || a.half == 32);
}

hipError_t launch_prefill_persist(const AttnArgs& a, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  int log2g = 0;
  while ((1 << log2g) < G) ++log2g;
  const int T = ROWS >> log2g;
  const int nblk = (a.nq + T - 1) / T;
  const long long items = (long long)a.B * a.hkv * nblk;
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = (int)((items < cus) ? items : cus);
  hipLaunchKernelGGL(prefill_persist_kernel, dim3((unsigned)grid), dim3(NW * 64), 0, stream, a,
                     log2g, nblk, (int)items);
  return hipGetLastError();
}

}  // namespace hswa
