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
// A workgroup of eight wavefronts owns 16 consecutive query rows of one
// (sequence, kv head) with G = 16 query heads, two rows per wavefront, so
// every per-row state (softmax totals, histograms, thresholds, output
// offsets) belongs to one wavefront and needs no synchronisation.  A
// wavefront's scores are S = Q . K^T on 32x32x16 MFMAs with its two rows'
// 16 heads each on M and the 32 keys of a tile on N: lane (key c, half h)
// holds eight heads of each row for key c, so a key's importance is eight
// exponentials summed in the lane and one exchange across the halves, and
// lanes 0..31 own the keys in order.  K tiles of
// 32 keys stream through LDS with global_load_lds, shared by all 16 rows.
// Four passes over the keys:
//   1. lse_hi per (row, head): online max / sum in base 2, one exponential
//      per score;
//   2. importance of every candidate (probabilities summed over the 16
//      heads), a 2048-bin histogram of its bits 31..21 per row in LDS, then
//      the bin holding the max_sel-th largest;
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

namespace hswa {
namespace {

constexpr int D = 192;
constexpr int KS = D / 16;              // k-steps of the 32x32x16 MFMA
constexpr int GQ = 16;                   // query heads per kv head (one MFMA column block)
constexpr int NW = 8;                    // wavefronts per workgroup
constexpr int NB = 2;                    // rows per wavefront
constexpr int ROWS = NW * NB;            // 16 query rows per workgroup
static_assert(ROWS == 16, "select_scratch_bytes sizes slots of 16 rows");
constexpr int BK = 32;                   // keys per LDS tile
constexpr int KROW = D * 2;              // 384 B per key row
constexpr int KTILE = BK * KROW;         // 12 KB
constexpr int KINSTR = KTILE / 1024;     // 12 copies of 1 KB
constexpr int NBIN = 2048;               // histogram bins per level
constexpr int UNR = 8;                   // 16-byte scratch loads in flight per lane

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Max / sum over the 16 lanes of a DPP row, left in every lane: pairs
// within quads (quad_perm 1,0,3,2 and 2,3,0,1), then quad with quad
// (row_half_mirror), then half-row with half-row (row_mirror).  Each step
// pairs every lane with one partner, so all 16 lanes end with the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));    // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));   // row_mirror
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

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
__device__ __forceinline__ void find_bin(const unsigned* h, unsigned need, int lane, int* bin,
                                         unsigned* above) {
  constexpr int PER = NBIN / 64;          // 32 bins per lane
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The partner of v across DPP rows: v_permlane16_swap on two copies of v
// leaves rows (0, 0, 2, 2) in one and (1, 1, 3, 3) in the other;
// v_permlane32_swap leaves the lower half twice in one and the upper half
// twice in the other.  Both are VALU moves (no LDS round trip), and both
// lanes of a pair see the operands in the same order.
struct Pair {
  float a, b;
};
__device__ __forceinline__ Pair rows16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ Pair halves32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Max / sum over the 32 lanes of a wavefront half (two DPP rows).
__device__ __forceinline__ float max32(float v) {
  const Pair p = rows16(max16(v));
  return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float sum32(float v) {
  const Pair p = rows16(sum16(v));
  return p.a + p.b;
}

// The twelve K operands of one key row: k-step 4 u + b sits 128 u bytes on
// from ad[b].  In asm: for a plain read the compiler would also wait for the
// next tile's copies in flight; the copies of this tile have been waited for
// before the barrier.  The block waits for its own reads before it returns.
__device__ __forceinline__ void lds_k12(bf16x8 (&f)[KS], const uint32_t (&ad)[4]) {
  uint4 r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11;
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b128 %4, %12 offset:128\n\t"
      "ds_read_b128 %5, %13 offset:128\n\t"
      "ds_read_b128 %6, %14 offset:128\n\t"
      "ds_read_b128 %7, %15 offset:128\n\t"
      "ds_read_b128 %8, %12 offset:256\n\t"
      "ds_read_b128 %9, %13 offset:256\n\t"
      "ds_read_b128 %10, %14 offset:256\n\t"
      "ds_read_b128 %11, %15 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
        "=&v"(r7), "=&v"(r8), "=&v"(r9), "=&v"(r10), "=&v"(r11)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
  f[0] = as_bf16x8(r0);
  f[1] = as_bf16x8(r1);
  f[2] = as_bf16x8(r2);
  f[3] = as_bf16x8(r3);
  f[4] = as_bf16x8(r4);
  f[5] = as_bf16x8(r5);
  f[6] = as_bf16x8(r6);
  f[7] = as_bf16x8(r7);
  f[8] = as_bf16x8(r8);
  f[9] = as_bf16x8(r9);
  f[10] = as_bf16x8(r10);
  f[11] = as_bf16x8(r11);
}
static_assert(KS == 12, "twelve k-steps of 16 dims");

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
  __shared__ unsigned hist[ROWS][NBIN];
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

  // this wavefront's rows
  // mode: 0 keeps nothing, 1 keeps every candidate, 2 ranks them
  int row_i[NB], ncand[NB], kwant[NB], mode[NB];
  bool row_ok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    row_i[nb] = i0 + NB * wave + nb;
    row_ok[nb] = row_i[nb] < n;
    ncand[nb] = row_ok[nb] ? max(0, row_i[nb] - recent + 1) : 0;
    kwant[nb] = min(K, ncand[nb]);
    mode[nb] = (kwant[nb] == 0) ? 0 : (ncand[nb] <= kwant[nb]) ? 1 : 2;
  }
  const int ilast = min(n - 1, i0 + ROWS - 1);       // last row of the workgroup
  const int lse_keys = ilast + 1;                     // pass 1 covers keys 0 .. ilast
  const int cand_keys = max(0, ilast - recent + 1);   // passes 2-4 cover 0 .. ilast - recent
  // the selection needs importances only where a row has more candidates than it keeps
  const bool any_rank = __syncthreads_or((lane == 0) && (mode[0] == 2 || mode[1] == 2));

  const bf16_t* __restrict__ Qp = static_cast<const bf16_t*>(a.half > 0 ? a.qrot : a.q);
  const bf16_t* __restrict__ Kp = static_cast<const bf16_t*>(a.half > 0 ? a.krot : a.k);

  // q operand: M row c is head g*16 + c % 16 of the wavefront's row c / 16;
  // k-step ks holds dims 16 ks + 8 hi .. + 7
  bf16x8 qf[KS];
  {
    const int nb = c >> 4;
    const bf16_t* qrow =
        Qp + ((tokbase + min(row_i[nb], n - 1)) * a.hq + g * GQ + (c & 15)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }

  // ---- K tile copies: instruction ii (12 per tile) fills LDS bytes [1024 ii, +1024):
  // slot s = 64 ii + lane, key row s / 24, physical chunk pc = s % 24 holding
  // logical chunk pc ^ (row & 7) (within its aligned 128 B).  Wavefront w
  // issues ii = w and, for w < 4, ii = w + 8.
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(Kp + (tokbase * hkv + g) * D);
  const int kstride = hkv * KROW;
  int drow[2], doff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ii = wave + NW * u;
    const int sl = 64 * ii + lane;
    const int row = sl / 24, pc = sl - row * 24;
    drow[u] = row;
    doff[u] = 16 * (pc ^ (row & 7));
  }
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
  // K operand of key c, k-step ks = 4 u + b: logical chunk 2 ks + hi =
  // 8 u + (2 b + hi), so 128 u bytes on from the chunk of k-step b
  uint32_t koff[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) koff[bb] = c * KROW + 16 * ((2 * bb + hi) ^ (c & 7));
  // S = Q . K^T for the tile: element e of the lane is key c against M row
  // 8 (e / 4) + 4 hi + e % 4, i.e. row e / 8 of the wavefront, head
  // 8 ((e / 4) % 2) + 4 hi + e % 4
  auto scores = [&](const unsigned char* kc) {
    const uint32_t base = lds_addr(kc);
    uint32_t ad[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) ad[bb] = base + koff[bb];
    bf16x8 kf[KS];
    lds_k12(kf, ad);
    f32x16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = mfma32(qf[ks], kf[ks], sc);
    return sc;
  };

  // Stream keys 0 .. nkeys - 1 in tiles; body(kc, k0) sees each tile in order.
  auto stream = [&](int nkeys, auto&& body) {
    if (nkeys <= 0) return;
    const int ntile = (nkeys + BK - 1) / BK;
    __syncthreads();                       // the previous stream's tiles are consumed
    issue(0, nkeys, kst0);
    for (int t = 0; t < ntile; ++t) {
      unsigned char* cur = (t & 1) ? kst1 : kst0;
      unsigned char* nxt = (t & 1) ? kst0 : kst1;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's copies of tile t
      __syncthreads();                     // everyone's copies landed; tile t - 1 consumed
      if (t + 1 < ntile) issue((t + 1) * BK, nkeys, nxt);
      body(cur, t * BK);
    }
  };

  const float c2 = a.scale * kLog2e;

  // ---- pass 1: lse (base 2) of every (row, head) over keys 0 .. i -----------
  // lane (c, hi) runs a (max, sum) for each of its 16 (row, head) elements
  // over its key c of every tile, reduced over the 32 key lanes at the end.
  // One exponential per key: of the two rescaling factors, the one of the
  // larger operand is exactly 1.  The running max starts finite, so that a
  // masked key (-inf) leaves the sum unchanged without a special case.
  float m[16], l[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    m[e] = -__FLT_MAX__;
    l[e] = 0.f;
  }
  if (any_rank) {
    stream(lse_keys, [&](const unsigned char* kc, int k0) {
      const f32x16 sc = scores(kc);
      const int j = k0 + c;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = (j <= row_i[e >> 3]) ? sc[e] * c2 : kNegInf;
        const float d = x - m[e];
        const float f = fast_exp2(-fabsf(d));
        l[e] = (d > 0.f) ? fmaf(l[e], f, 1.f) : l[e] + f;
        m[e] = fmaxf(m[e], x);
      }
    });
  }
  float lse[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float M = max32(m[e]);
    const float L = sum32(l[e] * fast_exp2(m[e] - M));
    lse[e] = M + __log2f(L);
  }

  // importance of key c of the tile for row nb (both lane halves of column
  // c end with the sum over the 16 heads)
  auto importances = [&](const unsigned char* kc, float (&imp)[NB]) {
    const f32x16 sc = scores(kc);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float v = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) v += fast_exp2(fmaf(sc[8 * nb + r], c2, -lse[8 * nb + r]));
      const Pair p = halves32(v);
      imp[nb] = p.a + p.b;
    }
  };
  const bool owner = hi == 0;                    // lanes 0..31 own keys 0..31 of a tile

  // this wavefront's rows of the workgroup's scratch slot
  unsigned* scr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) scr[nb] = scr_wg + (size_t)(NB * wave + nb) * ncap;

  int bin1[NB], t22[NB];
  unsigned above1[NB], quota[NB];
  if (any_rank) {
    // ---- pass 2: level-1 histogram (bits 31..21) ---------------------------
    for (int nb = 0; nb < NB; ++nb)
      for (int t = lane; t < NBIN; t += 64) hist[NB * wave + nb][t] = 0u;
    stream(cand_keys, [&](const unsigned char* kc, int k0) {
      float imp[NB];
      importances(kc, imp);
      const int j = k0 + c;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const unsigned u = __float_as_uint(imp[nb]);
        // every lane stores (the two halves write the same word, and words
        // past the row's candidates, within its round64(n), are never read)
        scr[nb][j] = u;
        if (owner && j < ncand[nb] && mode[nb] == 2)
          lds_inc(lds_addr(&hist[NB * wave + nb][u >> 21]));
      }
    });
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bin1[nb] = 0;
      above1[nb] = 0;
      if (mode[nb] == 2) find_bin(hist[NB * wave + nb], (unsigned)kwant[nb], lane, &bin1[nb], &above1[nb]);
    }
    // ---- pass 3: level-2 histogram (bits 20..10) inside bin1, from the
    // importances pass 2 stored.  The rows are this wavefront's own, on this
    // compute unit: a workgroup-scope fence (the stores complete) makes them
    // visible to its loads.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    for (int nb = 0; nb < NB; ++nb)
      for (int t = lane; t < NBIN; t += 64) hist[NB * wave + nb][t] = 0u;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (mode[nb] != 2) continue;
      const uint4* row = reinterpret_cast<const uint4*>(scr[nb]);
      const int nc = ncand[nb], nc4 = (nc + 3) >> 2;
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
            if (j + e < nc && (int)(w[e] >> 21) == bin1[nb])
              lds_inc(lds_addr(&hist[NB * wave + nb][(w[e] >> 10) & (NBIN - 1)]));
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      t22[nb] = 0;
      quota[nb] = 0;
      if (mode[nb] == 2) {
        int bin2;
        unsigned above2;
        find_bin(hist[NB * wave + nb], (unsigned)kwant[nb] - above1[nb], lane, &bin2, &above2);
        t22[nb] = (bin1[nb] << 11) | bin2;
        quota[nb] = (unsigned)kwant[nb] - above1[nb] - above2;   // ties at t22 to take
      }
    }
  }

  // ---- pass 4: emit, ascending; lane l owns candidates 4 l .. 4 l + 3 of
  // each 256, ranks from ballots of the per-lane counts ----------------------
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (!row_ok[nb]) continue;
    int* out = a.sel_out + ((tokbase + row_i[nb]) * hkv + g) * (long long)K;
    const int nc = ncand[nb];
    unsigned emitted = 0;
    if (mode[nb] == 1) {                       // every candidate
      for (int t = lane; t < nc; t += 64) out[t] = t;
      emitted = (unsigned)nc;
    } else if (mode[nb] == 2) {
      const uint4* row = reinterpret_cast<const uint4*>(scr[nb]);
      const int nc4 = (nc + 3) >> 2;
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
            above[e] = j + e < nc && key > t22[nb];
            tie[e] = j + e < nc && key == t22[nb];
            ntie += tie[e] ? 1u : 0u;
          }
          unsigned tie_total;
          const unsigned tie_at = ties + prefix_before(ntie, below, &tie_total);
          bool take[4];
          unsigned ntake = 0, r = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            take[e] = above[e] || (tie[e] && tie_at + r < quota[nb]);
            r += tie[e] ? 1u : 0u;
            ntake += take[e] ? 1u : 0u;
          }
          unsigned take_total;
          unsigned at = emitted + prefix_before(ntake, below, &take_total);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (take[e]) {
              if (at < (unsigned)kwant[nb]) out[at] = j + e;
              ++at;
            }
          ties += tie_total;
          emitted += take_total;
        }
      }
    }
    for (int t = min((int)emitted, kwant[nb]) + lane; t < K; t += 64) out[t] = -1;
    if (lane == 0) a.cnt_out[(tokbase + row_i[nb]) * hkv + g] = (int)min(emitted, (unsigned)kwant[nb]);
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
  const unsigned grid = (unsigned)(items < kSelectSlots ? items : kSelectSlots);
  hipLaunchKernelGGL(select_tokens_kernel, dim3(grid), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hswa
