// Token selection for the sparse layers on the gfx950 matrix cores.
//
// "MiMo-V3 HySparse2" (aideepthink.cn), section 4: the sparse layers reuse
// the token-selection indices of the preceding full-attention layer.  The
// importance of token j for query i and kv head g is the attention the
// full-attention layer gives it, summed over the group's query heads,
//     I_j = sum_{h in g} exp(a_hij - lse_hi)   (softmax over 0 .. i, no sink),
// and each (i, g) keeps the max_sel candidates 0 .. i - recent of largest
// importance, equal importances going to the lower position, in ascending
// order: the lists sparse attention reads.
//
// Two kernels.  The first, select_lse_kernel (select_lse.hip), writes lse_hi
// (base 2) for every (row, head) of the rows that rank their candidates.  In
// the second, select_tokens_kernel, a workgroup of eight wavefronts owns 32
// consecutive query rows of one (sequence, kv head) with G = 16 query heads,
// four rows per wavefront, so every per-row state (histograms, thresholds,
// output offsets) belongs to one wavefront and needs no synchronisation.  A
// wavefront's scores are S = Q . K^T on 32x32x16 MFMAs, two blocks of two
// rows x 16 heads on M and the 32 keys of a tile on N: lane (key c, half h)
// holds eight heads of each row for key c, so a key's importance is eight
// exponentials summed in the lane and one exchange across the halves, and
// lanes 0..31 own the keys in order.  K tiles of 32 keys stream through LDS
// with global_load_lds, shared by all 32 rows.  Passes:
//   1. (first kernel) lse_hi per (row, head), online sum in base 2;
//   2. importance of every candidate (probabilities summed over the 16
//      heads), stored to the workgroup's scratch slot and counted in a
//      1024-bin histogram of its bits 30..21 per row in LDS (importances are
//      >= 0, so bit 31 is 0), then the bin holding the max_sel-th largest;
//   3. inside that bin, a histogram of bits 20..10: the threshold t of the
//      22-bit key (importance >> 10, i.e. exponent and 13 mantissa bits) and
//      how many keys equal to t are taken;
//   4. the keys above t, then the ties at t in position order, written in
//      ascending order with ballots over the key-owning lanes.
// Importances are compared at that 22-bit resolution (relative 2^-13):
// keys that agree to it count as ties and the lower positions win.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "select_ops.h"

namespace hswa {
namespace {

constexpr int NW = 8;                    // wavefronts per workgroup
constexpr int RW = 4;                    // rows per wavefront: two blocks of 2 rows x 16 heads
constexpr int ROWS = NW * RW;            // 32 query rows per workgroup
static_assert(ROWS == kSelectRows, "select_scratch_bytes sizes slots of kSelectRows rows");
constexpr int NBIN1 = 1024;              // level-1 bins: bits 30..21 (importances are >= 0)
constexpr int NBIN2 = 2048;              // level-2 bins: bits 20..10
constexpr int UNR = 8;                   // 16-byte scratch loads in flight per lane
constexpr int LCAP = kSelectListCap;     // compact-list entries per row

// Wave-wide inclusive sum of v over lanes >= this lane (suffix sum).
__device__ __forceinline__ unsigned suffix_sum(unsigned v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned o = __shfl_down(v, off);
    v += (lane + off < 64) ? o : 0u;
  }
  return v;
}

// Largest bin b of the histogram h[0 .. NBIN) with (count above b) < need
// <= (count above b) + h[b], scanning from the top.  Returns b and the
// count strictly above it (uniform over the wavefront).
template <int NBIN>
__device__ __forceinline__ void find_bin(const unsigned* h, unsigned need, int lane, int* bin,
                                         unsigned* above) {
  constexpr int PER = NBIN / 64;          // bins per lane
  unsigned mine = 0;
#pragma unroll 8
  for (int t = 0; t < PER; ++t) mine += h[PER * lane + t];
  const unsigned incl = suffix_sum(mine, lane);   // this chunk and all above it
  const unsigned excl = incl - mine;
  const bool here = excl < need && need <= incl;
  const unsigned long long m = __ballot(here);
  const int src = m ? (int)__builtin_ctzll(m) : 0;
  int b = 0;
  unsigned ab = 0;
  if (lane == src) {
    unsigned cum = excl;
    b = PER * lane;
    for (int t = PER - 1; t >= 0; --t) {
      const unsigned c = h[PER * lane + t];
      if (cum + c >= need) {
        b = PER * lane + t;
        break;
      }
      cum += c;
    }
    ab = cum;
  }
  *bin = __shfl(b, src);
  *above = __shfl(ab, src);
}

// The same operands in two halves of six k-steps (0..5, then 6..11), so that
// only half of them is live at a time.
__device__ __forceinline__ void lds_k6_lo(bf16x8 (&f)[KS], const uint32_t (&ad)[4]) {
  uint4 r0, r1, r2, r3, r4, r5;
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b128 %4, %6 offset:128\n\t"
      "ds_read_b128 %5, %7 offset:128\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
  f[0] = as_bf16x8(r0);
  f[1] = as_bf16x8(r1);
  f[2] = as_bf16x8(r2);
  f[3] = as_bf16x8(r3);
  f[4] = as_bf16x8(r4);
  f[5] = as_bf16x8(r5);
}
__device__ __forceinline__ void lds_k6_hi(bf16x8 (&f)[KS], const uint32_t (&ad)[4]) {
  uint4 r6, r7, r8, r9, r10, r11;
  asm volatile(
      "ds_read_b128 %0, %8 offset:128\n\t"
      "ds_read_b128 %1, %9 offset:128\n\t"
      "ds_read_b128 %2, %6 offset:256\n\t"
      "ds_read_b128 %3, %7 offset:256\n\t"
      "ds_read_b128 %4, %8 offset:256\n\t"
      "ds_read_b128 %5, %9 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r6), "=&v"(r7), "=&v"(r8), "=&v"(r9), "=&v"(r10), "=&v"(r11)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
  f[6] = as_bf16x8(r6);
  f[7] = as_bf16x8(r7);
  f[8] = as_bf16x8(r8);
  f[9] = as_bf16x8(r9);
  f[10] = as_bf16x8(r10);
  f[11] = as_bf16x8(r11);
}

// Sum of x (0 .. 4) over the lanes below this one, from three ballots of
// its bits; *total = the sum over all 64 lanes.
__device__ __forceinline__ unsigned prefix_before(unsigned x, unsigned long long below,
                                                  unsigned* total) {
  const unsigned long long b0 = __ballot(x & 1u), b1 = __ballot(x & 2u), b2 = __ballot(x & 4u);
  *total = (unsigned)(__builtin_popcountll(b0) + 2 * __builtin_popcountll(b1) +
                      4 * __builtin_popcountll(b2));
  return (unsigned)(__builtin_popcountll(b0 & below) + 2 * __builtin_popcountll(b1 & below) +
                    4 * __builtin_popcountll(b2 & below));
}

// The same for x in 0 .. 32 (six ballots).
__device__ __forceinline__ unsigned prefix_before6(unsigned x, unsigned long long below,
                                                   unsigned* total) {
  unsigned t = 0, p = 0;
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    const unsigned long long bb = __ballot((x >> bit) & 1u);
    t += (unsigned)__builtin_popcountll(bb) << bit;
    p += (unsigned)__builtin_popcountll(bb & below) << bit;
  }
  *total = t;
  return p;
}

// Histogram increment at LDS address addr, in asm for the same reason (a
// plain atomic would wait for the copies in flight).  No value is returned;
// the wavefront's later reads of the histogram see it, as its LDS
// operations complete in order.
__device__ __forceinline__ void lds_inc(uint32_t addr) {
  asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(1u) : "memory");
}

}  // namespace

__global__ __launch_bounds__(512, 1) void select_tokens_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char kst0[KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char kst1[KTILE];
  // level-1 histograms of the 32 rows; once a wavefront has found its four
  // rows' level-1 bins, it reuses their 16 KB for the level-2 histogram of
  // one row at a time
  __shared__ __attribute__((aligned(16))) unsigned hist[ROWS][NBIN1];
  static_assert(RW * NBIN1 >= NBIN2, "a wavefront's level-1 rows hold one level-2 histogram");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 31, hi = lane >> 5;
  const int n = a.n, hkv = a.hkv, K = a.max_sel, recent = a.recent;
  const int nblk = (n + ROWS - 1) / ROWS;
  const int ngrp = a.B * hkv;
  const int items = ngrp * nblk;
  const int ncap = (n + 63) & ~63;               // scratch words per row
  const int nwg = (int)gridDim.x, wg = (int)blockIdx.x;
  unsigned* const scr_wg = a.sel_ws + (size_t)wg * ROWS * ncap;
  uint2* const lst_wg = reinterpret_cast<uint2*>(a.sel_ws + (size_t)nwg * ROWS * ncap) +
                        (size_t)wg * ROWS * LCAP;
  const float c2 = a.scale * kLog2e;
  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.half > 0 ? a.krot : a.k);
  const int kstride = hkv * KROW;

  // ---- K tile copies: instruction ii (12 per tile) fills LDS bytes [1024 ii, +1024):
  // slot s = 64 ii + lane, key row s / 24, physical chunk pc = s % 24 holding
  // logical chunk pc ^ ((row >> 1) & 7) (within its aligned 128 B): rows lie
  // 384 B apart, so rows r and r + 1 start half a 256-byte bank line apart,
  // and the sixteen lanes that read one line each cycle (rows c .. c + 15,
  // same logical chunk) hit sixteen different 16-byte bank groups.
  // Wavefront w issues ii = w and, for w < 4, ii = w + 8.
  int drow[2], doff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ii = wave + NW * u;
    const int sl = 64 * ii + lane;
    const int row = sl / 24, pc = sl - row * 24;
    drow[u] = row;
    doff[u] = 16 * (pc ^ ((row >> 1) & 7));
  }
  // K operand of key c, k-step ks = 4 u + b: logical chunk 2 ks + hi =
  // 8 u + (2 b + hi), so 128 u bytes on from the chunk of k-step b
  uint32_t koff[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) koff[bb] = c * KROW + 16 * ((2 * bb + hi) ^ ((c >> 1) & 7));
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // Items run heaviest first (late row blocks, long key ranges), round r
  // giving item r * nwg + w to workgroup w, or to nwg - 1 - w in odd rounds,
  // so that each pair of rounds costs every workgroup about the same.
  for (int r = 0; r * nwg < items; ++r) {
  const int item = r * nwg + ((r & 1) ? nwg - 1 - wg : wg);
  if (item >= items) continue;
  const int blk = nblk - 1 - item / ngrp;
  const int bg = item - (item / ngrp) * ngrp;
  const int b = bg / hkv, g = bg - b * hkv;
  const int i0 = blk * ROWS;
  const long long tokbase = (long long)b * n;

  // this wavefront's rows i0 + 4 w + rr
  // mode: 0 keeps nothing, 1 keeps every candidate, 2 ranks them
  int row_i[RW], ncand[RW], kwant[RW], mode[RW];
  bool row_ok[RW];
  bool mine = false;
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    row_i[rr] = i0 + RW * wave + rr;
    row_ok[rr] = row_i[rr] < n;
    ncand[rr] = row_ok[rr] ? max(0, row_i[rr] - recent + 1) : 0;
    kwant[rr] = min(K, ncand[rr]);
    mode[rr] = (kwant[rr] == 0) ? 0 : (ncand[rr] <= kwant[rr]) ? 1 : 2;
    mine = mine || mode[rr] == 2;
  }
  const int ilast = min(n - 1, i0 + ROWS - 1);       // last row of the workgroup
  const int cand_keys = max(0, ilast - recent + 1);   // passes 2-4 cover 0 .. ilast - recent
  // the selection needs importances only where a row has more candidates than it keeps
  const bool any_rank = __syncthreads_or((lane == 0) && mine);

  // this wavefront's rows of the workgroup's scratch slot
  unsigned* scr[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) scr[rr] = scr_wg + (size_t)(RW * wave + rr) * ncap;

  int bin1[RW];
  unsigned above1[RW], cnt1[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    bin1[rr] = 0;
    above1[rr] = 0;
    cnt1[rr] = 0;
  }
  if (any_rank) {
    // q operand of block nb: M row c is head g*16 + c % 16 of the
    // wavefront's row 2 nb + c / 16; k-step ks holds dims 16 ks + 8 hi .. + 7
    bf16x8 qf[2][KS];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bf16_t* qrow =
          Qp + ((tokbase + min(row_i[2 * nb + (c >> 4)], n - 1)) * a.hq + g * GQ + (c & 15)) * D +
          8 * hi;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[nb][ks] = as_bf16x8(ld16(qrow + 16 * ks));
    }
    // lse_hi (base 2) of element e of block nb, from the first kernel: row
    // 2 nb + e / 8, head 8 ((e / 4) % 2) + 4 hi + e % 4
    float lse[2][16];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 2 * nb + (e >> 3);
        lse[nb][e] = (mode[rr] == 2)
                         ? a.sel_lse[(tokbase + row_i[rr]) * a.hq + g * GQ + 8 * ((e >> 2) & 1) +
                                     4 * hi + (e & 3)]
                         : 0.f;
      }

    const unsigned char* kbase =
        reinterpret_cast<const unsigned char*>(Kp + (tokbase * hkv + g) * D);
    auto issue = [&](int k0, int kend, unsigned char* kd) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ii = wave + NW * u;
        if (ii < KINSTR) {
          const int key = min(k0 + drow[u], kend - 1);
          __builtin_amdgcn_global_load_lds(
              (glb_void_t*)(kbase + ((long long)key * kstride + doff[u])),
              (lds_void_t*)(kd + 1024 * ii), 16, 0, 0);
        }
      }
    };

    // ---- pass 2: importances of the candidates, stored to the scratch
    // rows, and the level-1 histogram (bits 30..21) of each ranking row.
    // S = Q . K^T per block: element e of the lane is key c against M row
    // 8 (e / 4) + 4 hi + e % 4, i.e. block row e / 8, head
    // 8 ((e / 4) % 2) + 4 hi + e % 4.  A key's importance for a row is the
    // lane's eight exponentials summed plus the other half's eight, so both
    // halves end with all four rows' importances of key c; lane (c, h)
    // stores and counts rows h and 2 + h.
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      uint4* hrow = reinterpret_cast<uint4*>(hist[RW * wave + rr]);
      for (int t = lane; t < NBIN1 / 4; t += 64) hrow[t] = make_uint4(0u, 0u, 0u, 0u);
    }
    const int ntile = (cand_keys + BK - 1) / BK;
    __syncthreads();                       // the previous item's tiles are consumed
    if (ntile > 0) issue(0, cand_keys, kst0);
    // A tile's importances are stored one tile late, right after the next
    // tile's copies have gone out: the vmcnt(0) that waits for a tile's
    // copies also waits for every store issued before it, and these were
    // issued a whole tile earlier instead of just before the wait.
    unsigned* const st0 = hi ? scr[1] : scr[0];   // this lane's stored rows: 1 or 0 ...
    unsigned* const st1 = hi ? scr[3] : scr[2];   // ... and 3 or 2
    unsigned pend0 = 0u, pend1 = 0u;
    int jpend = 0;
    // the candidate count and ranking mode of the rows this lane stores
    const int ncl[2] = {hi ? ncand[1] : ncand[0], hi ? ncand[3] : ncand[2]};
    const bool rankl[2] = {(hi ? mode[1] : mode[0]) == 2, (hi ? mode[3] : mode[2]) == 2};
    for (int t = 0; t < ntile; ++t) {
      unsigned char* cur = (t & 1) ? kst1 : kst0;
      unsigned char* nxt = (t & 1) ? kst0 : kst1;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's copies of tile t
      __syncthreads();                     // everyone's copies landed; tile t - 1 consumed
      if (t + 1 < ntile) issue((t + 1) * BK, cand_keys, nxt);
      if (t > 0) {   // words past the row's candidates, within its round64(n), are never read
        st0[jpend] = pend0;
        st1[jpend] = pend1;
      }
      const uint32_t base = lds_addr(cur);
      uint32_t ad[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) ad[bb] = base + koff[bb];
      bf16x8 kf[KS];
      f32x16 sc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[nb][e] = 0.f;
      lds_k6_lo(kf, ad);
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sc[nb] = mfma32(qf[nb][ks], kf[ks], sc[nb]);
      lds_k6_hi(kf, ad);
#pragma unroll
      for (int ks = KS / 2; ks < KS; ++ks)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) sc[nb] = mfma32(qf[nb][ks], kf[ks], sc[nb]);
      const int j = t * BK + c;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float imp2[2];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          float v = 0.f;
#pragma unroll
          for (int q = 0; q < 8; ++q)
            v += fast_exp2(fmaf(sc[nb][8 * r2 + q], c2, -lse[nb][8 * r2 + q]));
          const Pair p = halves32(v);
          imp2[r2] = p.a + p.b;
        }
        const int rr = 2 * nb + hi;          // the row this lane stores and counts
        const unsigned u = __float_as_uint(hi ? imp2[1] : imp2[0]);
        const int nc = ncl[nb];
        const bool rank = rankl[nb];
        if (nb == 0) pend0 = u;
        else pend1 = u;
        if (j < nc && rank) lds_inc(lds_addr(&hist[RW * wave + rr][u >> 21]));
      }
      jpend = j;
    }
    if (ntile > 0) {
      st0[jpend] = pend0;
      st1[jpend] = pend1;
    }

    // ---- level-1 bin of each ranking row, and how many candidates are in it
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      bin1[rr] = 0;
      above1[rr] = 0;
      cnt1[rr] = 0;
      if (mode[rr] == 2) {
        find_bin<NBIN1>(hist[RW * wave + rr], (unsigned)kwant[rr], lane, &bin1[rr], &above1[rr]);
        cnt1[rr] = hist[RW * wave + rr][bin1[rr]];
      }
    }
    // The scratch rows are this wavefront's own, on this compute unit: a
    // workgroup-scope fence (the stores complete) makes them visible to its
    // loads.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }

  // ---- per row: the threshold inside bin1 (level 2, bits 20..10) and the
  // lists, ascending.  A row whose candidates at or above bin1 fit in LCAP
  // is read once: the candidates above bin1 and those in it go, in position
  // order, to a compact list (position, 22-bit key), from which the level-2
  // histogram of bin1 and then the ranking are taken.  Otherwise the
  // importances are read twice, for the histogram and then to emit.  The
  // level-2 histogram lives in the wavefront's own level-1 rows.
  unsigned* const h2 = hist[RW * wave];
  for (int rr = 0; rr < RW; ++rr) {
    if (!row_ok[rr]) continue;
    int* out = a.sel_out + ((tokbase + row_i[rr]) * hkv + g) * (long long)K;
    const int nc = ncand[rr];
    unsigned emitted = 0;
    if (mode[rr] == 1) {                       // every candidate
      for (int t = lane; t < nc; t += 64) out[t] = t;
      emitted = (unsigned)nc;
    } else if (mode[rr] == 2) {
      const int want = kwant[rr], b1 = bin1[rr];
      for (int t = lane; t < NBIN2 / 4; t += 64)
        reinterpret_cast<uint4*>(h2)[t] = make_uint4(0u, 0u, 0u, 0u);
      const uint4* row = reinterpret_cast<const uint4*>(scr[rr]);
      const int nc4 = (nc + 3) >> 2;
      if (above1[rr] + cnt1[rr] <= (unsigned)LCAP) {
        // one read: lane l scans the 32 consecutive candidates
        // 32 l .. 32 l + 31 of each 2048, so that one prefix over the lanes
        // orders the kept ones
        uint2* lst = lst_wg + (size_t)(RW * wave + rr) * LCAP;
        unsigned count = 0;
        // the next round's loads are issued before this round is counted
        uint4 u[UNR], un[UNR];
#pragma unroll
        for (int t = 0; t < UNR; ++t) {
          const int q = UNR * lane + t;
          un[t] = (q < nc4) ? row[q] : make_uint4(0u, 0u, 0u, 0u);
        }
        for (int q0 = 0; q0 < nc4; q0 += 64 * UNR) {
#pragma unroll
          for (int t = 0; t < UNR; ++t) u[t] = un[t];
          if (q0 + 64 * UNR < nc4) {
#pragma unroll
            for (int t = 0; t < UNR; ++t) {
              const int q = q0 + 64 * UNR + UNR * lane + t;
              un[t] = (q < nc4) ? row[q] : make_uint4(0u, 0u, 0u, 0u);
            }
          }
          const int j0 = 4 * (q0 + UNR * lane);
          unsigned nk = 0;
#pragma unroll
          for (int t = 0; t < UNR; ++t) {
            const unsigned w[4] = {u[t].x, u[t].y, u[t].z, u[t].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              nk += (j0 + 4 * t + e < nc && (int)(w[e] >> 21) >= b1) ? 1u : 0u;
          }
          unsigned total;
          unsigned at = count + prefix_before6(nk, below, &total);
          if (nk) {
#pragma unroll
            for (int t = 0; t < UNR; ++t) {
              const unsigned w[4] = {u[t].x, u[t].y, u[t].z, u[t].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int j = j0 + 4 * t + e;
                if (j < nc && (int)(w[e] >> 21) >= b1) lst[at++] = make_uint2((unsigned)j, w[e] >> 10);
              }
            }
          }
          count += total;
        }
        // the list is this wavefront's own stores: visible after a fence;
        // the level-2 histogram of its bin1 entries
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        for (int q = lane; q < (int)count; q += 64) {
          const unsigned key = lst[q].y;
          if ((int)(key >> 11) == b1) lds_inc(lds_addr(&h2[key & (NBIN2 - 1)]));
        }
        int bin2;
        unsigned above2;
        find_bin<NBIN2>(h2, (unsigned)want - above1[rr], lane, &bin2, &above2);
        const unsigned t22 = ((unsigned)b1 << 11) | (unsigned)bin2;
        const unsigned quota = (unsigned)want - above1[rr] - above2;   // ties at t22 to take
        unsigned ties = 0;
        for (int q0 = 0; q0 < (int)count; q0 += 64) {
          const int q = q0 + lane;
          const uint2 en = (q < (int)count) ? lst[q] : make_uint2(0u, 0u);
          const bool in = q < (int)count;
          const bool tie = in && en.y == t22;
          const unsigned long long bt = __ballot(tie);
          const bool take = in && (en.y > t22 || (tie && ties + (unsigned)__builtin_popcountll(bt & below) < quota));
          const unsigned long long bk = __ballot(take);
          const unsigned at = emitted + (unsigned)__builtin_popcountll(bk & below);
          if (take && at < (unsigned)want) out[at] = (int)en.x;
          ties += (unsigned)__builtin_popcountll(bt);
          emitted += (unsigned)__builtin_popcountll(bk);
        }
      } else {
        // level 2 over the whole row, then a second read to emit; lane l
        // owns candidates 4 l .. 4 l + 3 of each 256, ranks from ballots of
        // the per-lane counts
        for (int q0 = 0; q0 < nc4; q0 += 64 * UNR) {
          uint4 u[UNR];
#pragma unroll
          for (int t = 0; t < UNR; ++t) {
            const int q = q0 + 64 * t + lane;
            u[t] = (q < nc4) ? row[q] : make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
          for (int t = 0; t < UNR; ++t) {
            const int j = 4 * (q0 + 64 * t + lane);
            const unsigned w[4] = {u[t].x, u[t].y, u[t].z, u[t].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j + e < nc && (int)(w[e] >> 21) == b1)
                lds_inc(lds_addr(&h2[(w[e] >> 10) & (NBIN2 - 1)]));
          }
        }
        int bin2;
        unsigned above2;
        find_bin<NBIN2>(h2, (unsigned)want - above1[rr], lane, &bin2, &above2);
        const int t22 = (b1 << 11) | bin2;
        const unsigned quota = (unsigned)want - above1[rr] - above2;
        unsigned ties = 0;
        for (int q0 = 0; q0 < nc4; q0 += 64 * UNR) {
          uint4 u[UNR];
#pragma unroll
          for (int t = 0; t < UNR; ++t) {
            const int q = q0 + 64 * t + lane;
            u[t] = (q < nc4) ? row[q] : make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
          for (int t = 0; t < UNR; ++t) {
            // the lane's four consecutive candidates j .. j + 3
            const int j = 4 * (q0 + 64 * t + lane);
            const unsigned w[4] = {u[t].x, u[t].y, u[t].z, u[t].w};
            bool above[4], tie[4];
            unsigned ntie = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = (int)(w[e] >> 10);
              above[e] = j + e < nc && key > t22;
              tie[e] = j + e < nc && key == t22;
              ntie += tie[e] ? 1u : 0u;
            }
            unsigned tie_total;
            const unsigned tie_at = ties + prefix_before(ntie, below, &tie_total);
            bool take[4];
            unsigned ntake = 0, rk = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              take[e] = above[e] || (tie[e] && tie_at + rk < quota);
              rk += tie[e] ? 1u : 0u;
              ntake += take[e] ? 1u : 0u;
            }
            unsigned take_total;
            unsigned at = emitted + prefix_before(ntake, below, &take_total);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (take[e]) {
                if (at < (unsigned)want) out[at] = j + e;
                ++at;
              }
            ties += tie_total;
            emitted += take_total;
          }
        }
      }
    }
    for (int t = min((int)emitted, kwant[rr]) + lane; t < K; t += 64) out[t] = -1;
    if (lane == 0) a.cnt_out[(tokbase + row_i[rr]) * hkv + g] = (int)min(emitted, (unsigned)kwant[rr]);
  }
  }  // items
}

bool select_tokens_supported(const AttnArgs& a) {
  return a.d_qk == D && a.hq == GQ * a.hkv && 2 * a.half <= D;
}

hipError_t launch_select_tokens(const AttnArgs& a, hipStream_t stream) {
  const long long items = (long long)a.B * a.hkv * ((a.n + ROWS - 1) / ROWS);
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = launch_select_lse(a, cus, stream);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(items < kSelectSlots ? items : kSelectSlots);
  hipLaunchKernelGGL(select_tokens_kernel, dim3(grid), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hswa
