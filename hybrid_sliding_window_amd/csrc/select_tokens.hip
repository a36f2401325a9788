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
// offsets) belongs to one wavefront and needs no synchronisation.  A row's
// scores are S = Q . K^T on 16x16x32 MFMAs with the 16 heads on M and 16
// keys on N: lane (key c, group q) holds heads 4q .. 4q + 3 of key c, so a
// key's importance is four exponentials summed in the lane and two
// exchanges across the lane groups, and lanes 0..15 own the keys in order.  K tiles of
// 32 keys stream through LDS with global_load_lds, shared by all 16 rows.
// Four passes over the keys:
//   1. lse_hi per (row, head): online max / sum in base 2;
//   2. importance of every candidate (probabilities summed over the 16 head
//      lanes), a 2048-bin histogram of its bits 31..21 per row in LDS, then
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
constexpr int KS = D / 32;
constexpr int GQ = 16;                   // query heads per kv head (one MFMA column block)
constexpr int NW = 8;                    // wavefronts per workgroup
constexpr int NB = 2;                    // rows per wavefront
constexpr int ROWS = NW * NB;            // 16 query rows per workgroup
constexpr int BK = 32;                   // keys per LDS tile
constexpr int KROW = D * 2;              // 384 B per key row
constexpr int KTILE = BK * KROW;         // 12 KB
constexpr int KINSTR = KTILE / 1024;     // 12 copies of 1 KB
constexpr int NBIN = 2048;               // histogram bins per level

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

// The six K operands of key row r (or r + 16 with HI) at LDS addresses ad[].
// In asm: for a plain read the compiler would also wait for the next tile's
// copies in flight; the copies of this tile have been waited for before the
// barrier.  The block waits for its own reads before it returns.
template <bool HI>
__device__ __forceinline__ void lds_k6(bf16x8 (&f)[KS], const uint32_t (&ad)[KS]) {
  uint4 r0, r1, r2, r3, r4, r5;
  if (HI)
    asm volatile(
        "ds_read_b128 %0, %6 offset:6144\n\t"
        "ds_read_b128 %1, %7 offset:6144\n\t"
        "ds_read_b128 %2, %8 offset:6144\n\t"
        "ds_read_b128 %3, %9 offset:6144\n\t"
        "ds_read_b128 %4, %10 offset:6144\n\t"
        "ds_read_b128 %5, %11 offset:6144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5)
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5])
        : "memory");
  else
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5)
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5])
        : "memory");
  f[0] = as_bf16x8(r0);
  f[1] = as_bf16x8(r1);
  f[2] = as_bf16x8(r2);
  f[3] = as_bf16x8(r3);
  f[4] = as_bf16x8(r4);
  f[5] = as_bf16x8(r5);
}
static_assert(16 * KROW == 6144, "the second 16-key half sits 6144 bytes further on");

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
  const int lane = tid & 63, c = lane & 15, grp = lane >> 4;
  const int n = a.n, hkv = a.hkv, K = a.max_sel, recent = a.recent;
  const int nblk = (n + ROWS - 1) / ROWS;
  // heavy blocks (late rows, long key ranges) first
  const int item = (int)blockIdx.x;
  const int bg = item / nblk;
  const int blk = nblk - 1 - (item - bg * nblk);
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

  // q of row nb, head g*16 + c, k-step ks: dims 32 ks + 8 grp .. + 7
  bf16x8 qf[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bf16_t* qrow = Qp + ((tokbase + min(row_i[nb], n - 1)) * a.hq + g * GQ + c) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nb][ks] = as_bf16x8(ld16(qrow + 32 * ks));
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
  // K operands of key row (16 hf + c), k-step ks: logical chunk 4 ks + grp
  // (rows c and c + 16 share the swizzle, 6144 bytes apart)
  uint32_t koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = c * KROW + 16 * ((4 * ks + grp) ^ (c & 7));
  auto kops = [&](const unsigned char* kc, int hf, bf16x8 (&kf)[KS]) {
    const uint32_t base = lds_addr(kc);
    uint32_t ad[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ad[ks] = base + koff[ks];
    if (hf) lds_k6<true>(kf, ad);
    else lds_k6<false>(kf, ad);
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
  // lane (c, q) runs a (max, sum) for heads 4q + r over its keys c of each
  // 16-key half, reduced over the 16 key lanes at the end
  float m[NB][4], l[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[nb][r] = kNegInf;
      l[nb][r] = 0.f;
    }
  if (any_rank) {
    stream(lse_keys, [&](const unsigned char* kc, int k0) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 sc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kf[KS];
        kops(kc, hf, kf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) sc[nb] = mfma16(qf[nb][ks], kf[ks], sc[nb]);
        const int j = k0 + 16 * hf + c;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = (j <= row_i[nb]) ? sc[nb][r] * c2 : kNegInf;
            const float mn = fmaxf(m[nb][r], x);
            const float ms = (mn == kNegInf) ? 0.f : mn;
            l[nb][r] = l[nb][r] * fast_exp2(m[nb][r] - ms) + fast_exp2(x - ms);
            m[nb][r] = mn;
          }
      }
    });
  }
  float lse[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float M = max16(m[nb][r]);
      const float L =
          sum16(l[nb][r] * ((m[nb][r] == kNegInf) ? 0.f : fast_exp2(m[nb][r] - M)));
      lse[nb][r] = M + __log2f(L);
    }

  // importance of key c of the tile half for row nb (all four lane groups
  // of column c end with the sum over the 16 heads)
  auto importances = [&](const unsigned char* kc, int hf, float (&imp)[NB]) {
    f32x4 sc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 kf[KS];
    kops(kc, hf, kf);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sc[nb] = mfma16(qf[nb][ks], kf[ks], sc[nb]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float v = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) v += fast_exp2(fmaf(sc[nb][r], c2, -lse[nb][r]));
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      imp[nb] = v;
    }
  };
  auto owned = [&](const float (&imp)[NB], int nb) -> float { return imp[nb]; };
  const bool owner = grp == 0;                   // lanes 0..15 own keys 0..15 of a half
  const int kk_own = c;

  int bin1[NB], t22[NB];
  unsigned above1[NB], quota[NB];
  if (any_rank) {
    // ---- pass 2: level-1 histogram (bits 31..21) ---------------------------
    for (int nb = 0; nb < NB; ++nb)
      for (int t = lane; t < NBIN; t += 64) hist[NB * wave + nb][t] = 0u;
    stream(cand_keys, [&](const unsigned char* kc, int k0) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float imp[NB];
        importances(kc, hf, imp);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int j = k0 + 16 * hf + kk_own;
          if (owner && j < ncand[nb] && mode[nb] == 2)
            lds_inc(lds_addr(&hist[NB * wave + nb][__float_as_uint(owned(imp, nb)) >> 21]));
        }
      }
    });
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bin1[nb] = 0;
      above1[nb] = 0;
      if (mode[nb] == 2) find_bin(hist[NB * wave + nb], (unsigned)kwant[nb], lane, &bin1[nb], &above1[nb]);
    }
    // ---- pass 3: level-2 histogram (bits 20..10) inside bin1 ---------------
    for (int nb = 0; nb < NB; ++nb)
      for (int t = lane; t < NBIN; t += 64) hist[NB * wave + nb][t] = 0u;
    stream(cand_keys, [&](const unsigned char* kc, int k0) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float imp[NB];
        importances(kc, hf, imp);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int j = k0 + 16 * hf + kk_own;
          const unsigned u = __float_as_uint(owned(imp, nb));
          if (owner && j < ncand[nb] && mode[nb] == 2 && (int)(u >> 21) == bin1[nb])
            lds_inc(lds_addr(&hist[NB * wave + nb][(u >> 10) & (NBIN - 1)]));
        }
      }
    });
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

  // ---- pass 4: emit, ascending ----------------------------------------------
  int* sel_out[NB];
  unsigned emitted[NB], ties[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    sel_out[nb] = a.sel_out + ((tokbase + min(row_i[nb], n - 1)) * hkv + g) * (long long)K;
    emitted[nb] = 0;
    ties[nb] = 0;
  }
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  stream(cand_keys, [&](const unsigned char* kc, int k0) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float imp[NB];
      if (any_rank) importances(kc, hf, imp);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int j = k0 + 16 * hf + kk_own;
        const bool cand = owner && j < ncand[nb];
        bool take, tie = false;
        if (mode[nb] != 2) {
          take = cand && mode[nb] == 1;           // nothing, or every candidate
        } else {
          const int key = (int)(__float_as_uint(owned(imp, nb)) >> 10);
          tie = cand && key == t22[nb];
          const unsigned long long tm = __ballot(tie);
          const unsigned rank = ties[nb] + (unsigned)__builtin_popcountll(tm & below);
          take = cand && (key > t22[nb] || (tie && rank < quota[nb]));
          ties[nb] += (unsigned)__builtin_popcountll(tm);
        }
        const unsigned long long sm = __ballot(take);
        const unsigned at = emitted[nb] + (unsigned)__builtin_popcountll(sm & below);
        if (take && at < (unsigned)kwant[nb]) sel_out[nb][at] = j;
        emitted[nb] += (unsigned)__builtin_popcountll(sm);
      }
    }
  });
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (!row_ok[nb]) continue;
    for (int t = min((int)emitted[nb], kwant[nb]) + lane; t < K; t += 64) sel_out[nb][t] = -1;
    if (lane == 0) a.cnt_out[(tokbase + row_i[nb]) * hkv + g] = (int)min(emitted[nb], (unsigned)kwant[nb]);
  }
}

bool select_tokens_supported(const AttnArgs& a) {
  return a.d_qk == D && a.hq == GQ * a.hkv && 2 * a.half <= D;
}

hipError_t launch_select_tokens(const AttnArgs& a, hipStream_t stream) {
  const long long items = (long long)a.B * a.hkv * ((a.n + ROWS - 1) / ROWS);
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(select_tokens_kernel, dim3((unsigned)items), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hswa
