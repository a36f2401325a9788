// bf16 prefill for layers whose query blocks read many key tiles: full
// causal (the GA layers) and windows wider than the resident ring of
// prefill_seq.hip ("MiMo-V2-Flash: Hybrid Sliding Window Attention
// Architecture" (rslog.cc) sections 2.1, 2.3, 4.4 and 5).  Shapes: GQA
// group G >= 8 (a power of two), d_qk 192, d_v 128, rotary half-width 0, 16
// or 32, at most 256 query heads.
//
// Work.  One persistent workgroup of 8 wavefronts per CU (two per SIMD)
// walks its items (kv head g, T = 256 / G query tokens, 256 rows, 32 per
// wavefront) in rounds of one item per workgroup, numbered XCD by XCD so
// that the 32 workgroups of an XCD take neighbouring blocks of one head and
// share their K/V tiles in that XCD's L2, the order reversed every other
// round so that long and short causal rows even out per workgroup.  The key tiles of its
// items form one stream; tile number x of the stream lives in stage x % 6
// of a ring of 20 KB K/V tiles.  A step consumes two tiles behind one
// barrier; between them wavefronts 0..3 issue the 40 copies of the step two
// ahead, into the stages the previous step has just released.  q
// goes straight from memory into each wavefront's registers when an item
// starts (long items: the load is paid once per item).
#include "common.h"
#include "launch.h"
#include "tile_ops.h"

namespace hswa {
namespace {

constexpr int CA_NW = 8;                   // wavefronts per workgroup
constexpr int CA_ROWS = 32 * CA_NW;        // 256 query rows per item
constexpr int CA_SLOT = KTILE + VTILE;     // 20 KB: K tile then V tile
constexpr int CA_NS = 6;                   // ring stages: 3 steps of 2 tiles

struct CItem {
  long long kbase;   // b * n
  long long qbase;   // b * nq - qoff
  int g, i0, kstart, kend, ntiles;
};

__device__ __forceinline__ CItem citem(const AttnArgs& a, int k, int nblk, int T) {
  CItem it;
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

__device__ __forceinline__ int citem_of(int j, int pos, int P) {
  return j * P + ((j & 1) ? P - 1 - pos : pos);
}

}  // namespace

__global__ __launch_bounds__(512, 1) void prefill_causal_kernel(AttnArgs a, int log2g, int nblk,
                                                                 int items) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[CA_NS * CA_SLOT];
  __shared__ float sinkbuf[MAX_HQ];
  __shared__ double revbuf[MAX_HALF];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i = lane & 31, h = lane >> 5;
  const int G = 1 << log2g;
  const int T = CA_ROWS >> log2g;
  const int n = a.n, hkv = a.hkv, hq = a.hq;
  const int W = a.window;
  const int half = a.half;
  const int R = 2 * half;

  const int P = gridDim.x;
  // hardware dispatch sends workgroup b to XCD b % 8
  const int pos = (P % 8 == 0) ? (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  if (citem_of(0, pos, P) >= items) return;   // uniform over the workgroup

  for (int j = tid; j < hq; j += CA_NW * 64) sinkbuf[j] = a.sink ? a.sink[j] * kLog2e : kNegInf;
  if (tid < half) revbuf[tid] = pow(a.rope_theta, -(double)tid / (double)half) * 0.15915494309189535;
  __syncthreads();

  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ Kr = static_cast<const bf16_t*>(a.krot);
  const bf16_t* __restrict__ Vp = static_cast<const bf16_t*>(a.v);
  bf16_t* __restrict__ Op = static_cast<bf16_t*>(a.o);

  // ---- copies: a step is 2 tiles x (12 K + 8 V copies of 1 KB) ------------
  // Only wavefronts 0..3 issue copies, ten each: copy c = wave + 4u (u < 10)
  // of a step is tile c / 20, copy cc = c % 20 of that tile (below 12: K
  // copy, slot s = 64 cc + lane, row s / 24, physical chunk s % 24 holding
  // logical chunk pc ^ ((row >> 1) & 7), chunks below R/8 from the rotated
  // copy unless K is stored rotated; else V copy cc - 12, row s / 16, 64-byte
  // unit (pc / 4) ^ (row & 3)).  Issuing a copy stalls the wavefront until
  // the vector-memory path accepts it (about 1700 cycles for a step's 40
  // copies when every wavefront issued five right after the barrier, and no
  // wavefront computed meanwhile); with the copies on one wavefront of each
  // SIMD, the other one keeps the SIMD busy while its partner waits.

  // request cursor: round rj, tile rt of item rc; past the last item the last
  // tile is requested again (finite data, never read)
  int rj = 0, rt = 0;
  CItem rc = citem(a, citem_of(0, pos, P), nblk, T);
  int put = 0;   // stream number of the next tile requested
  int nis = 0;   // vector-memory operations issued by this wavefront so far
  const bool producer = wave < 4;
  auto request_step = [&]() {
    uintptr_t bk[2], br[2], bv[2];
    int lim[2], st[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j0 = rc.kstart + rt * BK;
      lim[k] = rc.kend - 1 - j0;
      const long long rb = (rc.kbase + j0) * hkv + rc.g;
      bk[k] = reinterpret_cast<uintptr_t>(Kp + rb * D);
      br[k] = reinterpret_cast<uintptr_t>(Kr + rb * R);
      bv[k] = reinterpret_cast<uintptr_t>(Vp + rb * DV);
      st[k] = put % CA_NS;
      ++put;
      if (rt + 1 < rc.ntiles) {
        ++rt;
      } else if (citem_of(rj + 1, pos, P) < items) {
        ++rj;
        rt = 0;
        rc = citem(a, citem_of(rj, pos, P), nblk, T);
      }
    }
    if (producer) {
      // the per-lane offsets are recomputed here (an opaque copy of the lane
      // index keeps the compiler from hoisting them into registers held for
      // the whole kernel)
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int u = 0; u < 10; ++u) {
        const int c = wave + 4 * u;
        const int k = c / 20;
        const int cc = c - 20 * k;
        uint32_t off;
        uintptr_t base;
        int dst;
        if (cc < 12) {
          const int sl = 64 * cc + ln;
          const int row = sl / 24, pc = sl - row * 24;
          const int lc = pc ^ ((row >> 1) & 7);
          const bool rot = !a.k_rotated && lc < (half >> 2);
          off = (uint32_t)(min(row, lim[k]) * (hkv * (rot ? R : D)) + 8 * lc) * 2u;
          // the K rows or their rotated copy, chosen by arithmetic: a select
          // here was lowered to a lookup in scratch memory, whose load then
          // waited for every copy in flight
          base = bk[k] + ((br[k] - bk[k]) & (uintptr_t)(0 - (uintptr_t)rot));
          dst = 1024 * cc;
        } else {
          const int sl = 64 * (cc - 12) + ln;
          const int row = sl >> 4, pc = sl & 15;
          off = (uint32_t)(min(row, lim[k]) * (hkv * DV) + 8 * (4 * ((pc >> 2) ^ (row & 3)) + (pc & 3))) *
                2u;
          base = bv[k];
          dst = KTILE + 1024 * (cc - 12);
        }
        g2lds16(reinterpret_cast<const void*>(base + off), ring + st[k] * CA_SLOT + dst);
      }
      nis += 10;
    }
    asm volatile("" ::: "memory");
  };
  request_step();
  int ma = nis;   // nis after the copies of the step about to be consumed
  request_step();
  int mb = nis;   // ... and of the step after it

  uint32_t krd[4], vrd[4];   // per-lane LDS offsets of the operand reads
  operand_offsets(lane, krd, vrd);
  const uint32_t ring0 = lds_addr(ring);
  const float c2 = a.scale * kLog2e;
  const int row = 32 * wave + i;

  // consume cursor: round cj, tile ct of item cur
  int cj = 0, ct = 0;
  CItem cur = citem(a, citem_of(0, pos, P), nblk, T);
  int get = 0;   // stream number of the next tile consumed
  bool done = false;

  // state of the current item
  int tok = 0, head = 0, lo = 0, hi = 0;
  float m = kNegInf, l = 0.f;
  f32x16 acc[MT];
  u32x4 qf[KS];

  auto store_out = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const float lt = l + __shfl_xor(l, 32);
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
    if (lo < n) {   // the wavefront's first row is a real token: 8 stores issued
      if (tok < n) {
        bf16_t* orow = Op + ((cur.qbase + tok) * hq + head) * DV + 16 * h;
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
  };

  auto start_item = [&]() {
    tok = cur.i0 + (row >> log2g);
    head = cur.g * G + (row & (G - 1));
    lo = cur.i0 + ((32 * wave) >> log2g);
    hi = min(n - 1, cur.i0 + ((32 * wave + 31) >> log2g));
    const int tk = min(tok, n - 1);
    const bf16_t* qrow = Qp + ((cur.qbase + tk) * hq + head) * (long long)D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
    nis += KS;
    // wait for the q rows here, once per item (this also waits for the
    // copies in flight), so that no use of q inside the tile loop waits
    __builtin_amdgcn_s_waitcnt(VMCNT(0));
    if (half > 0) {
      if (half == 16) rotate_q<1>(qf, revbuf, (double)(a.pos_offset + tok), h);
      else rotate_q<2>(qf, revbuf, (double)(a.pos_offset + tok), h);
    }
    m = sinkbuf[head];
    l = (h == 0 && m > kNegInf) ? 1.f : 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;
  };

  // one key tile of the current item from its stage
  auto consume = [&]() {
    if (ct == 0) start_item();
    const int stage = get % CA_NS;
    ++get;
    const uint32_t kaddr = ring0 + stage * CA_SLOT;
    const uint32_t vaddr = kaddr + KTILE;
    const int j0 = cur.kstart + ct * BK;
    f32x16 sa;
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
    u32x2 vf[8];
    lds_vhalf<0>(vf, vaddr + vrd[0], vaddr + vrd[1], vaddr + vrd[2], vaddr + vrd[3]);
    // the score products may have been placed after the V reads: keep the
    // VALU reads of their result (behind the branches below) at a safe
    // distance
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
    f32x16 x = sa;
    if ((j0 + BK - 1 > lo) || (W > 0 && j0 < hi - W + 1)) {
      // key j0 + 4h + kk (kk = 8j + r) is visible iff dlo <= kk <= dhi
      const int dhi = tok - (j0 + 4 * h);
      const int dlo = (W > 0) ? dhi - (W - 1) : -0x7fffffff;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = 8 * (v >> 2) + (v & 3);
        x[v] = (kk > dhi || kk < dlo) ? kNegInf : x[v];
      }
    }
    // P against the current reference first; only a tile whose P sum passes
    // kLazySum (a key more than ~12 above the reference in log2 units) or a
    // row with no reference yet takes the row max and moves the reference,
    // so the common path has no max over the tile's scores
    const float ms = (m == kNegInf) ? 0.f : m;
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(x[v], c2, -ms));
    uint4 pb0 = pack8(p), pb1 = pack8(p + 8);
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
    if (++ct == cur.ntiles) {
      store_out();
      ct = 0;
      if (citem_of(cj + 1, pos, P) < items) {
        ++cj;
        cur = citem(a, citem_of(cj, pos, P), nblk, T);
      } else {
        done = true;
      }
    }
  };

  // Step: wait for this step's two tiles (copied by the request two steps
  // back); the barrier also releases the two stages the previous step read,
  // into which the request of the step two ahead goes, issued between the
  // step's two tiles (measured faster than right after the barrier).
  while (!done) {
    wait_copy(nis - ma);
    ring_barrier();
    const int mnext = mb;
    consume();
    request_step();
    ma = mnext;
    mb = nis;
    if (!done) consume();
  }
  __builtin_amdgcn_s_waitcnt(VMCNT(0));   // no copy into LDS outlives the workgroup
}

bool prefill_causal_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && a.hq == G * a.hkv && G >= 8 && G <= CA_ROWS &&
         (G & (G - 1)) == 0 && a.hq <= MAX_HQ && (a.half == 0 || a.half == 16 || a.half == 32);
}

hipError_t launch_prefill_causal(const AttnArgs& a, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  int log2g = 0;
  while ((1 << log2g) < G) ++log2g;
  const int T = CA_ROWS >> log2g;
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
  hipLaunchKernelGGL(prefill_causal_kernel, dim3((unsigned)grid), dim3(CA_NW * 64), 0, stream, a,
                     log2g, nblk, (int)items);
  return hipGetLastError();
}

}  // namespace hswa
