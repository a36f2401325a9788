// Sliding-window bf16 prefill that walks each kv head's query blocks in
// order and keeps the window's K/V tiles resident in LDS ("MiMo-V2-Flash:
// Hybrid Sliding Window Attention Architecture" (rslog.cc) sections 2.1,
// 2.3, 4.4 and 5), for windowed layers whose query blocks need only a few
// key tiles; prefill_causal.hip serves full causal layers and wider windows.
//
// Why.  With a 128-token window a block of 32 query tokens reads 5 key tiles
// of 32 keys, 4 of which the previous block of the same head also read.
// Fetching every block's tiles afresh sends five times the K/V bytes
// through each CU's vector-memory path; here consecutive blocks of one head
// run on the same workgroup and only the one new tile per block is copied.
//
// Work.  One workgroup of 8 wavefronts per CU (two per SIMD) takes a
// contiguous run of items; an item is one kv head g and T = 256 / G
// consecutive query tokens (256 rows: tokens x the G query heads), 32 rows
// per wavefront.  Key tiles are aligned to multiples of 32 positions and
// tile x lives in ring slot x % NS.  At the start of an item, after a
// barrier, the tiles that the next item adds are requested (the next item
// never needs more than NS tiles together with this one; wavefronts 0..3
// copy K, 4..7 V); the item's own tiles were requested one item earlier.  A
// run that crosses to another sequence or head requests the new item's
// tiles when it gets there.  K is copied unrotated; each K-copying
// wavefront turns the rotary dims of the rows it copied in LDS once they
// have landed, before the barrier that publishes the tile.  q goes straight
// into registers (no q staging in LDS, no barrier per tile): the two
// wavefronts of a SIMD work out of phase, one storing its output and
// loading the next item's q at the end of an item, the other at the start
// of the next, after touching the rows into L2 during its last tile.
//
// Arithmetic per tile (as in prefill_causal.hip): S^T = K . Q^T on the
// 32x32x16 MFMA (a lane holds query row i against keys 8j + 4h + r), base-2
// online softmax seeded with the sink and a lazily moved reference max, l
// summed from the bf16 P with v_dot2, O^T += V^T . P^T with the V^T operand
// read transposed from LDS so each lane ends up with 16 consecutive output
// dims, stored as two 16-byte range-checked buffer writes per output tile.
#include "common.h"
#include "launch.h"
#include "tile_ops.h"

namespace hswa {
namespace {

constexpr int SW_NW = 8;                   // wavefronts per workgroup
constexpr int SW_ROWS = 256;               // query rows per item
constexpr int SLOT = KTILE + VTILE;        // 20 KB: K tile then V tile
constexpr int NS = 7;                      // ring slots

template <bool B>
struct GroupTag {
  static constexpr bool value = B;
};

// Item k of the (sequence, kv head, query block) order.
struct SeqItem {
  long long kbase;   // b * n
  long long qbase;   // b * nq - qoff
  int bg;            // b * hkv + g
  int g, i0, ta, tb; // first query position; first and last key tile
};

__device__ __forceinline__ SeqItem seq_item(const AttnArgs& a, int k, int nblk, int T) {
  SeqItem it;
  it.bg = k / nblk;
  const int blk = k - it.bg * nblk;
  const int b = it.bg / a.hkv;
  it.g = it.bg - b * a.hkv;
  it.kbase = (long long)b * a.n;
  it.qbase = (long long)b * a.nq - a.qoff;
  it.i0 = a.qoff + blk * T;
  const int kf = max(0, it.i0 - a.window + 1);
  const int kl = min(a.n - 1, it.i0 + T - 1);
  it.ta = kf / BK;
  it.tb = kl / BK;
  return it;
}

}  // namespace

__global__ __launch_bounds__(512, 1) void prefill_seq_kernel(AttnArgs a, int log2g, int nblk,
                                                              int items, int run) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[NS * SLOT];
  __shared__ float sinkbuf[MAX_HQ];
  __shared__ double revbuf[MAX_HALF];
  __shared__ __attribute__((aligned(16))) unsigned char qtouch[SW_NW * 256];   // never read

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i = lane & 31, h = lane >> 5;
  const int G = 1 << log2g;
  const int T = SW_ROWS >> log2g;
  const int n = a.n, hkv = a.hkv, hq = a.hq;
  const int W = a.window;
  const int half = a.half;

  const int j_begin = blockIdx.x * run;
  const int j_end = min(items, j_begin + run);
  if (j_begin >= j_end) return;   // uniform over the workgroup

  for (int j = tid; j < hq; j += SW_NW * 64) sinkbuf[j] = a.sink ? a.sink[j] * kLog2e : kNegInf;
  if (tid < half) revbuf[tid] = pow(a.rope_theta, -(double)tid / (double)half) * 0.15915494309189535;
  __syncthreads();

  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ Vp = static_cast<const bf16_t*>(a.v);
  bf16_t* __restrict__ Op = static_cast<bf16_t*>(a.o);

  // ---- tile copies: 12 K copies of 1 KB by wavefronts 0..3, 8 V by 4..7 --
  // K copy c = 3 cw + u (u < 3): slot s = 64 c + lane, row s / 24, physical
  // chunk s % 24 holding logical chunk pc ^ ((row >> 1) & 7), so wavefront
  // cw copies whole rows 8 cw .. 8 cw + 7 (and rotates their rotary dims
  // once they have landed, see rotate_k_rows).
  // V copy c = cw + 4u (u < 2): row s / 16, 64-byte unit (pc / 4) ^ (row & 3).
  const bool kwave = wave < SW_NW / 2;
  // The two wavefronts of a SIMD work out of phase: the early one (0..3)
  // stores an item's output and loads the next item's q at the end of the
  // item, the late one (4..7) does both at the start of the next item, so
  // that each one's memory traffic overlaps the other's products.
  const int cw = kwave ? wave : wave - SW_NW / 2;
  int krow[3], kcol[3], vrow[2], vcol[2];
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int sl = 64 * (3 * cw + u) + lane;
    const int row = sl / 24, pc = sl - row * 24;
    krow[u] = row;
    kcol[u] = 8 * (pc ^ ((row >> 1) & 7));
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = 64 * (cw + 4 * u) + lane;
    const int row = sl >> 4, pc = sl & 15;
    vrow[u] = row;
    vcol[u] = 8 * (4 * ((pc >> 2) ^ (row & 3)) + (pc & 3));
  }
  int nis = 0;   // vector-memory operations issued by this wavefront so far
  // copies of key tile x of the item's sequence into slot x % NS; rows past
  // the sequence's last key repeat that key (finite data, masked)
  auto request_tile = [&](const SeqItem& c, int x) {
    const int j0 = x * BK;
    const int lim = n - 1 - j0;
    const long long rb = (c.kbase + j0) * hkv + c.g;
    const bf16_t* kb = Kp + rb * D;
    const bf16_t* vb = Vp + rb * DV;
    unsigned char* kd = ring + (x % NS) * SLOT;
    unsigned char* vd = kd + KTILE;
    if (kwave) {
#pragma unroll
      for (int u = 0; u < 3; ++u)
        g2lds16(kb + (min(krow[u], lim) * (hkv * D) + kcol[u]), kd + 1024 * (3 * cw + u));
      asm volatile("" ::: "memory");
      nis += 3;
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        g2lds16(vb + (min(vrow[u], lim) * (hkv * DV) + vcol[u]), vd + 1024 * (cw + 4 * u));
      asm volatile("" ::: "memory");
      nis += 2;
    }
  };

  // ---- q rows of an item straight into registers -------------------------
  // this wavefront's rows 32 wave + i (token row >> log2g, head row & (G - 1));
  // lane (i, h) holds dims 16 ks + 8 h .. + 7 of k-step ks
  auto load_q = [&](const SeqItem& c, u32x4 (&qf)[KS]) {
    const int row = 32 * wave + i;
    const int tk = min(c.i0 + (row >> log2g), n - 1);
    const bf16_t* qrow = Qp + ((c.qbase + tk) * hq + c.g * G + (row & (G - 1))) * (long long)D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
    nis += KS;
  };

  // The output rows of an item as a buffer resource (token i0, head 0 at
  // offset 0; the sequence's tokens from i0 on in range): stores of rows
  // past the sequence's last token fall outside it and are dropped by the
  // hardware, so every wavefront issues the same 8 stores and the explicit
  // vector-memory waits can count them.
  auto out_rsrc = [&](const SeqItem& c) __attribute__((always_inline)) {
    const int rows = max(0, min(T, n - c.i0));
    return __builtin_amdgcn_make_buffer_rsrc(Op + (c.qbase + c.i0) * hq * DV, 0, rows * hq * DV * 2,
                                             0x00020000);
  };
  // o = O / l in bf16, 16 consecutive dims per lane per output tile
  auto store_block = [&](const f32x16 (&acc)[MT], float l, int row, __amdgpu_buffer_rsrc_t rs)
      __attribute__((always_inline)) {
    const float lt = l + __shfl_xor(l, 32);
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
    const int off = row * (DV * 2) + 32 * h;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float f[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) f[v] = acc[mt][v] * inv;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pack8(f)), rs, off + 64 * mt, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pack8(f + 8)), rs,
                                             off + 64 * mt + 16, 0, 0);
    }
    asm volatile("" ::: "memory");
    nis += 2 * MT;
  };

  uint32_t krd[4], vrd[4];   // per-lane LDS offsets of the operand reads
  operand_offsets(lane, krd, vrd);
  const uint32_t ring0 = lds_addr(ring);

  // RoPE of the keys in LDS (K stored unrotated): an early wavefront turns
  // the rotary dims of the rows it copied (rows 8 cw .. 8 cw + 7 of tile x,
  // keys x * 32 + row at positions pos_offset + key) once its copies have
  // landed and before the barrier that publishes the tile.  Lane (row
  // lane / 8, chunk pair (lane / 2) % 4, elements 4 (lane % 2) .. + 3):
  // dims 8 p + e and their partners half further on, with the angle formed
  // in fp64 revolutions and evaluated by the hardware sine and cosine, as the
  // rotated-K preparation does.
  const bool rot_k = half > 0 && !a.k_rotated;
  auto rotate_k_rows = [&](int x) __attribute__((always_inline)) {
    const int r = 8 * cw + (lane >> 3);
    const int pr = (lane >> 1) & 3;
    const int e0 = 4 * (lane & 1);
    if (pr < (half >> 3)) {
      const int sw = (r >> 1) & 7;
      const uint32_t rowa = ring0 + (x % NS) * SLOT + r * KROW + 2 * e0;
      const uint32_t a0 = rowa + 16 * (pr ^ sw);
      const uint32_t a1 = rowa + 16 * ((pr + (half >> 3)) ^ sw);
      u32x2 w0, w1;
      asm volatile("ds_read_b64 %0, %2\n\tds_read_b64 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(w0), "=&v"(w1) : "v"(a0), "v"(a1) : "memory");
      float f0[4], f1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u0 = w0[e >> 1], u1 = w1[e >> 1];
        f0[e] = __uint_as_float((e & 1) ? (u0 & 0xffff0000u) : (u0 << 16));
        f1[e] = __uint_as_float((e & 1) ? (u1 & 0xffff0000u) : (u1 << 16));
      }
      const double pos = (double)(a.pos_offset + (long long)x * BK + r);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double turns = pos * revbuf[8 * pr + e0 + e];
        const float f = (float)(turns - floor(turns));
        const float co = __builtin_amdgcn_cosf(f), si = __builtin_amdgcn_sinf(f);
        const float y0 = f0[e] * co - f1[e] * si;
        const float y1 = f1[e] * co + f0[e] * si;
        f0[e] = y0;
        f1[e] = y1;
      }
      const u32x2 o0 = {pack_bf16x2(f0[0], f0[1]), pack_bf16x2(f0[2], f0[3])};
      const u32x2 o1 = {pack_bf16x2(f1[0], f1[1]), pack_bf16x2(f1[2], f1[3])};
      asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %2, %3\n\ts_waitcnt lgkmcnt(0)"
                   :: "v"(a0), "v"(o0), "v"(a1), "v"(o1) : "memory");
    }
  };
  const float c2 = a.scale * kLog2e;

  // The item loop, generated once per group so that each group's stores,
  // loads and waits form straight-line code the compiler's wait analysis
  // can follow.
  auto run_items = [&](auto group) __attribute__((always_inline)) {
  constexpr bool late = decltype(group)::value;
  // ---- prologue: the first item's tiles and q rows ------------------------
  SeqItem cur = seq_item(a, j_begin, nblk, T);
  int req_bg = cur.bg, req_hi = cur.tb;   // highest tile requested for sequence req_bg
  int rot_bg = -1, rot_hi = 0;            // highest tile rotated for sequence rot_bg
  for (int x = cur.ta; x <= cur.tb; ++x) request_tile(cur, x);
  int mark_cur = nis;                     // nis after the copies the current item reads
  u32x4 q0[KS];                           // q of the current item (then of the next)
  if (!late) load_q(cur, q0);
  bool fresh = false;                     // the current item's tiles are still to request

  // O, l of the item being finished; the late group keeps them (and the
  // item's output coordinates) across the barrier and stores them at the
  // start of the next item
  f32x16 acc0[MT];
  float l0 = 0.f;
  int prow = 0;                                                    // (token - i0) hq + head
  __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(Op, 0, 0, 0x00020000);   // no rows

  for (int j = j_begin; j < j_end; ++j) {
    const bool has_next = j + 1 < j_end;
    const SeqItem nx = seq_item(a, has_next ? j + 1 : j, nblk, T);

    // this item's tiles have landed (each wavefront waits for its own
    // copies); the barrier also retires every slot the previous item read
    if (fresh) {
      ring_barrier();
      for (int x = cur.ta; x <= cur.tb; ++x) request_tile(cur, x);
      req_bg = cur.bg;
      req_hi = cur.tb;
      mark_cur = nis;
    }
    wait_copy(nis - mark_cur);
    if (!late && rot_k) {   // the tiles this item adds, now landed
      for (int x = (cur.bg == rot_bg) ? max(rot_hi + 1, cur.ta) : cur.ta; x <= cur.tb; ++x)
        rotate_k_rows(x);
      rot_bg = cur.bg;
      rot_hi = cur.tb;
    }
    ring_barrier();
    // this item's q rows have landed (the late group first loads them and
    // then stores the previous item's output, whose 8 stores it does not
    // wait for); waiting here, before any new copy is issued, keeps the
    // compiler from waiting for those copies too at the first use of q
    if (late) {
      load_q(cur, q0);
      store_block(acc0, l0, prow, prs);   // nothing in range before the first item
      __builtin_amdgcn_s_waitcnt(VMCNT(2 * MT));
    } else {
      __builtin_amdgcn_s_waitcnt(VMCNT(0));
    }
    // tiles the next item adds (same sequence: at most NS with this item's)
    fresh = has_next && nx.bg != req_bg;
    if (has_next && !fresh) {
      for (int x = max(req_hi + 1, nx.ta); x <= nx.tb; ++x) request_tile(nx, x);
      req_hi = max(req_hi, nx.tb);
    }
    int mark_next = nis;
    // this item's q, rotated at its positions
    const int rw0 = 32 * wave + i;
    const int tok0 = cur.i0 + (rw0 >> log2g);
    const int head0 = cur.g * G + (rw0 & (G - 1));
    if (half > 0) {
      if (half == 16) rotate_q<1>(q0, revbuf, (double)(a.pos_offset + tok0), h);
      else rotate_q<2>(q0, revbuf, (double)(a.pos_offset + tok0), h);
    }
    // wave-uniform token range of the rows (for the edge-tile test)
    const int b0lo = cur.i0 + ((32 * wave) >> log2g);
    const int b0hi = min(n - 1, cur.i0 + ((32 * wave + 31) >> log2g));

    float m0 = sinkbuf[head0];
    l0 = (h == 0 && m0 > kNegInf) ? 1.f : 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc0[mt][v] = 0.f;

    // Softmax of one block's scores x for the tile at key j0 and P in bf16
    auto softmax = [&](f32x16& x, float& m, float& l, f32x16 (&acc)[MT], int tok, int lo, int hi,
                       int j0, uint4& pb0, uint4& pb1) __attribute__((always_inline)) {
      if ((j0 + BK - 1 > lo) || (j0 < hi - W + 1)) {
        const int dhi = tok - (j0 + 4 * h);
        const int dlo = dhi - (W - 1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 8 * (v >> 2) + (v & 3);
          x[v] = (kk > dhi || kk < dlo) ? kNegInf : x[v];
        }
      }
      // P against the current reference first; only a tile whose P sum
      // passes kLazySum (a key more than ~12 above the reference in log2
      // units) or a row with no reference yet takes the row max and moves
      // the reference, so the common path has no max over the scores
      const float ms = (m == kNegInf) ? 0.f : m;
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(x[v], c2, -ms));
      pb0 = pack8(p);
      pb1 = pack8(p + 8);
      float t = 0.f;
      t = add_bf16_pair(pb0.x, t); t = add_bf16_pair(pb0.y, t);
      t = add_bf16_pair(pb0.z, t); t = add_bf16_pair(pb0.w, t);
      t = add_bf16_pair(pb1.x, t); t = add_bf16_pair(pb1.y, t);
      t = add_bf16_pair(pb1.z, t); t = add_bf16_pair(pb1.w, t);
      if (__any(m == kNegInf || !(t <= kLazySum))) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        float xm = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) xm = fmaxf(xm, x[v]);
        const float mx = fmaxf(xm, __shfl_xor(xm, 32)) * c2;
        const float mn = fmaxf(m, mx);
        if (mn > m) {
          const float alpha = fast_exp2(m - mn);
          l *= alpha;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
          m = mn;
        }
        const float mr = (m == kNegInf) ? 0.f : m;
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(x[v], c2, -mr));
        pb0 = pack8(p);
        pb1 = pack8(p + 8);
        t = 0.f;
        t = add_bf16_pair(pb0.x, t); t = add_bf16_pair(pb0.y, t);
        t = add_bf16_pair(pb0.z, t); t = add_bf16_pair(pb0.w, t);
        t = add_bf16_pair(pb1.x, t); t = add_bf16_pair(pb1.y, t);
        t = add_bf16_pair(pb1.z, t); t = add_bf16_pair(pb1.w, t);
        asm volatile("s_nop 4" ::: "memory");
      }
      l += t;
    };

    for (int x = cur.ta; x <= cur.tb; ++x) {
      const uint32_t kaddr = ring0 + (x % NS) * SLOT;
      const uint32_t vaddr = kaddr + KTILE;
      const int j0 = x * BK;
      // Bring the next item's q rows into L2 (one dword per 128-byte line
      // of this wavefront's 32 rows, copied into a scratch area nobody
      // reads) two tiles before the item's end (early group) or in its last
      // tile (late group), so that the q loads hit L2 (earlier touches
      // measured slower: the lines leave L2 again).
      if (has_next && x == max(cur.ta, cur.tb - (late ? 0 : 2))) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ln = 64 * u + lane;
          if (ln < 96) {
            const int row = 32 * wave + ln / 3;
            const int tk = min(nx.i0 + (row >> log2g), n - 1);
            const bf16_t* src = Qp + ((nx.qbase + tk) * hq + nx.g * G + (row & (G - 1))) * (long long)D +
                                64 * (ln % 3);
            __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(qtouch + 256 * wave), 4, 0, 0);
          }
        }
        asm volatile("" ::: "memory");
        nis += 2;
      }

      f32x16 sc0;
#pragma unroll
      for (int v = 0; v < 16; ++v) sc0[v] = 0.f;
      u32x4 kf[KS];
      lds_ksteps_lo(kf, kaddr + krd[0], kaddr + krd[1], kaddr + krd[2], kaddr + krd[3]);
#pragma unroll
      for (int ks = 0; ks < 6; ++ks)
        sc0 = mfma32(__builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, q0[ks]), sc0);
      lds_ksteps_hi(kf, kaddr + krd[0], kaddr + krd[1], kaddr + krd[2], kaddr + krd[3]);
#pragma unroll
      for (int ks = 6; ks < KS; ++ks)
        sc0 = mfma32(__builtin_bit_cast(bf16x8, kf[ks]), __builtin_bit_cast(bf16x8, q0[ks]), sc0);
      u32x2 vf[8];
      lds_vhalf<0>(vf, vaddr + vrd[0], vaddr + vrd[1], vaddr + vrd[2], vaddr + vrd[3]);
      uint4 p00, p01;
      softmax(sc0, m0, l0, acc0, tok0, b0lo, b0hi, j0, p00, p01);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc0[mt] = mfma32(as_bf16x8(make_uint4(vf[2 * mt][0], vf[2 * mt][1], vf[2 * mt + 1][0],
                                               vf[2 * mt + 1][1])),
                          as_bf16x8(p00), acc0[mt]);
      lds_vhalf<1>(vf, vaddr + vrd[0], vaddr + vrd[1], vaddr + vrd[2], vaddr + vrd[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc0[mt] = mfma32(as_bf16x8(make_uint4(vf[2 * mt][0], vf[2 * mt][1], vf[2 * mt + 1][0],
                                               vf[2 * mt + 1][1])),
                          as_bf16x8(p01), acc0[mt]);
    }

    // ---- output (early group): o = O / l, then the next item's q --------
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const int row0 = (tok0 - cur.i0) * hq + head0;
    if (!late) {
      store_block(acc0, l0, row0, out_rsrc(cur));
      if (has_next) load_q(nx, q0);
    } else {
      prow = row0;
      prs = out_rsrc(cur);
    }

    mark_cur = mark_next;
    cur = nx;
  }
  if (late) store_block(acc0, l0, prow, prs);   // the run's last item
  };
  if (kwave) run_items(GroupTag<false>{});
  else run_items(GroupTag<true>{});
  __builtin_amdgcn_s_waitcnt(VMCNT(0));   // no copy into LDS outlives the workgroup
}

// Windowed layers of the shapes above whose items need at most NS tiles
// together with the next item's.
bool prefill_seq_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  if (!(a.d_qk == D && a.d_v == DV && a.hq == G * a.hkv && G >= 8 && G <= SW_ROWS &&
        (G & (G - 1)) == 0 && a.hq <= MAX_HQ && (a.half == 0 || a.half == 16 || a.half == 32)))
    return false;
  if (a.window <= 0) return false;
  const int T = SW_ROWS / G;
  // key tiles of two consecutive items together (keys i0 - W + 1 ..
  // i0 + 2T - 1) at the worst alignment
  const int span = a.window + 2 * T - 1;
  return (span - 1) / BK + 2 <= NS;
}

hipError_t launch_prefill_seq(const AttnArgs& a, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  int log2g = 0;
  while ((1 << log2g) < G) ++log2g;
  const int T = SW_ROWS >> log2g;
  const int nblk = (a.nq + T - 1) / T;
  const long long items = (long long)a.B * a.hkv * nblk;
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int run = (int)((items + cus - 1) / cus);
  const int grid = (int)((items + run - 1) / run);
  hipLaunchKernelGGL(prefill_seq_kernel, dim3((unsigned)grid), dim3(SW_NW * 64), 0, stream, a,
                     log2g, nblk, (int)items, run);
  return hipGetLastError();
}

}  // namespace hswa
