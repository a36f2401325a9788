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
// LDS serves all of them.  Each wavefront holds 32 rows as two 16-column
// MFMA operands.
//
// Orientation.  Scores are computed transposed, S^T = K . Q^T, so a lane
// owns one query row (column c) and four keys per 16-key sub-tile.  Two
// sub-tiles of that output are, lane for lane, the B operand of the next
// product O^T += V^T . P^T, so P never leaves registers.  The row max needs
// two cross-lane steps (lanes c, c+16, c+32, c+48); the row sum stays per
// lane until the end.
//
// Softmax in base 2.  The fp32 scores are scaled by scale * log2(e) inside
// the exp2 argument (one FMA), so q is rounded to bf16 only where RoPE
// changed it; the sink is multiplied by log2(e) only.  The state starts at
// m = sink, l = 1 (one lane per row): the sink's exp(sink - m) term.  The
// reference max m moves only when a row's max exceeds it by more than
// kLazy (in log2 units); until then P = exp2(s - m) <= 2^kLazy, which fp32
// sums and bf16 P hold as well as values below 1, and neither the row max
// nor the rescale of O is needed.  O and l always share the same m, so
// o = O / l is unchanged.  The row sum l is itself an MFMA output (P^T
// against a ones row), so it sums exactly the bf16 P that weight V.
//
// RoPE.  q is rotated in registers (pair r, r + R/2 sits in one lane when
// R/2 is a multiple of 32) from a cos/sin table; K's rotated dims were
// rotated once per call by the preparation kernel and are staged as is.
//
// Staging.  Two LDS stages: the global loads of tile t+1 are issued into
// registers before tile t is computed and written to the other stage after
// it, so their latency hides behind one tile of work (one barrier per tile).
// Rows are padded (K 400 B, V 288 B) so the MFMA operand reads hit distinct
// bank groups.  V stays row-major: the A operand of the PV product is read
// with ds_read_b64_tr_b16, whose 16-lane transpose hands lane i the values
// V[k0 + k][d0 + i], k = 0..3, when lane j points at V[k0 + j/4][d0 + 4 * (j % 4)].
#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

constexpr int D = 192;                 // q/k head dim
constexpr int DV = 128;                // v head dim
constexpr int KS = D / 32;             // k-steps of the 16x16x32 MFMA
constexpr int NT = DV / 16;            // 16-wide output tiles
constexpr int BK = 32;                 // keys per staged tile
constexpr int ROWS = 128;              // query rows per workgroup
constexpr int WG_ROWS = ROWS;
constexpr int KPITCH = D * 2 + 16;     // K row pitch in LDS (bytes)
constexpr int VPITCH = DV * 2 + 32;    // V row pitch in LDS (bytes)
constexpr int KBYTES = BK * KPITCH;    // 12800
constexpr int VBYTES = BK * VPITCH;    // 9216
constexpr int STAGE_BYTES = KBYTES + VBYTES;
constexpr int OPITCH = DV * 2 + 16;    // output row pitch in LDS (bytes) for the store transpose
constexpr int QSLOTS = D / 8 + 1;      // 16-byte slots per q row in LDS (400 B pitch, one pad)
constexpr int QBYTES_W = 13 * 1024;    // per-wavefront q region: 32 rows x 25 slots -> 13 x 1 KB
constexpr int SMEM_BYTES = (2 * STAGE_BYTES > 4 * QBYTES_W) ? 2 * STAGE_BYTES : 4 * QBYTES_W;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (lds_base uniform).
__device__ __forceinline__ void g2lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_base, 16, 0, 0);
}
constexpr int KCHUNKS = BK * (D / 8);   // 16-byte K chunks per tile: 768
constexpr int VCHUNKS = BK * (DV / 8);  // 16-byte V chunks per tile: 512
constexpr float kLazy = 8.f;
constexpr float kLazyPow = 256.f;      // 2^kLazy

// Rotate the rotary k-steps of q (pair (ka, ka + PK) sits in one lane) and
// round them to bf16; the other k-steps keep their exact input values.
template <int PK>
__device__ __forceinline__ void rotate_q(bf16x8 (&qf)[KS], const uint4 (&raw)[KS],
                                         const float2* __restrict__ trow, int grp) {
#pragma unroll
  for (int ka = 0; ka < PK; ++ka) {
    const float2* t = trow + 32 * ka + 8 * grp;
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

// CB = 16-row column blocks per wavefront.  2 is what runs: 4 wavefronts of
// 32 rows, 2 per SIMD.  CB = 1 (8 wavefronts of 16 rows, 4 per SIMD) hides
// more latency but reads every K/V operand twice as often from LDS, and
// measured slower on both the windowed and the causal workload.
template <int CB>
__global__ __launch_bounds__(512 / CB, 4 / CB) void prefill_bf16_kernel(AttnArgs a, int log2g,
                                                                        int nblk, int balance) {
  constexpr int NTHREADS = 512 / CB;
  constexpr int KPER = (KCHUNKS + NTHREADS - 1) / NTHREADS;
  constexpr int VPER = VCHUNKS / NTHREADS;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, grp = lane >> 4;

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

  // ---- staging: per-thread chunks, pointers advanced one tile per step ----
  // K chunk ch < R/8 of a row comes from the rotated copy (row pitch R),
  // the rest from K itself (row pitch D).
  const int rchunks = a.half >> 2;
  const bf16_t* kptr[KPER];
  int kkey[KPER], klds[KPER];
  long long kstep[KPER];
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int idx = min(tid + u * NTHREADS, KCHUNKS - 1);   // spare threads skip (see kown)
    const int key = idx / (D / 8), ch = idx - (idx / (D / 8)) * (D / 8);
    const bool rot = ch < rchunks;
    const int pitch = rot ? 2 * a.half : D;
    kptr[u] = (rot ? Kr : Kp) + ((tokbase + kstart + key) * hkv + g) * pitch + 8 * ch;
    kstep[u] = (long long)BK * hkv * pitch;
    kkey[u] = key;
    klds[u] = key * KPITCH + 16 * ch;
  }
  const bf16_t* vptr[VPER];
  int vkey[VPER], vlds[VPER];
#pragma unroll
  for (int u = 0; u < VPER; ++u) {
    const int idx = tid + u * NTHREADS;
    const int key = idx / (DV / 8), ch = idx - (idx / (DV / 8)) * (DV / 8);
    vptr[u] = Vp + ((tokbase + kstart + key) * hkv + g) * DV + 8 * ch;
    vkey[u] = key;
    vlds[u] = KBYTES + key * VPITCH + 16 * ch;
  }
  const long long vstep = (long long)BK * hkv * DV;
  uint4 kreg[KPER], vreg[VPER];

  auto kown = [&](int u) { return u * NTHREADS < KCHUNKS - tid; };   // wave-uniform
  auto load_tile = [&](int j0) {        // global -> registers, zero past kend
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
      if (!kown(u)) continue;
      kreg[u] = (j0 + kkey[u] < kend) ? ld16(kptr[u]) : make_uint4(0, 0, 0, 0);
      kptr[u] += kstep[u];
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      vreg[u] = (j0 + vkey[u] < kend) ? ld16(vptr[u]) : make_uint4(0, 0, 0, 0);
      vptr[u] += vstep;
    }
  };
  auto store_tile = [&](int stage) {    // registers -> LDS stage
    unsigned char* base = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int u = 0; u < KPER; ++u)
      if (kown(u)) st16(base + klds[u], kreg[u]);
#pragma unroll
    for (int u = 0; u < VPER; ++u) st16(base + vlds[u], vreg[u]);
  };

  // ---- the two query rows of this lane ---------------------------------
  int tok[CB], head[CB];
  bool rv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int r = wave * 16 * CB + cb * 16 + c;
    tok[cb] = i0 + (r >> log2g);
    head[cb] = g * G + (r & (G - 1));
    rv[cb] = tok[cb] < n;
  }
  const int tw0 = i0 + ((wave * 16 * CB) >> log2g);
  const int tw1 = min(n - 1, i0 + ((wave * 16 * CB + 16 * CB - 1) >> log2g));
  const bool wave_live = tw0 < n;

  // ---- q: straight into LDS, then tile 0, then operands and rotation ------
  // Each wavefront's 32 q rows are four runs of 3 KB (G heads of one token
  // are contiguous), so every 1 KB load instruction reads whole cache lines.
  // Slot s of the wavefront's region holds row s / 25, chunk s % 25 (chunk
  // 24 and slots past row 31 are padding, loaded from a valid address).
  static_assert(CB == 2, "the q staging assumes 32 rows per wavefront");
  unsigned char* qlds = smem + wave * QBYTES_W;
#pragma unroll
  for (int i = 0; i < QBYTES_W / 1024; ++i) {
    const int slot = 64 * i + lane;
    const int rr = min(slot / QSLOTS, 31);
    int ch = slot - (slot / QSLOTS) * QSLOTS;
    if (ch >= D / 8 || slot >= 32 * QSLOTS) ch = 0;
    const int r = wave * 32 + rr;
    const int tk = min(i0 + (r >> log2g), n - 1);
    const int hd = g * G + (r & (G - 1));
    g2lds16(Qp + ((tokbase + tk) * a.hq + hd) * D + 8 * ch, qlds + 1024 * i);
  }
  load_tile(kstart);

  bf16x8 qf[CB][KS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    uint4 qraw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qraw[ks] = ld16(qlds + (cb * 16 + c) * (QSLOTS * 16) + (4 * ks + grp) * 16);
      qf[cb][ks] = as_bf16x8(qraw[ks]);
    }
    if (a.half > 0 && rv[cb]) {
      const float2* trow = a.rope + (long long)tok[cb] * a.half;
      switch (a.half >> 5) {
        case 1: rotate_q<1>(qf[cb], qraw, trow, grp); break;
        case 2: rotate_q<2>(qf[cb], qraw, trow, grp); break;
        default: rotate_q<3>(qf[cb], qraw, trow, grp); break;
      }
    }
  }

  // ---- softmax state seeded with the sink -------------------------------
  // The row sum l rides in one more MFMA: an A operand whose row 0 is all
  // ones turns P^T into sum_keys P in element 0 of the lanes with grp == 0.
  const float c2 = a.scale * kLog2e;   // raw score -> base-2 units
  float m[CB];
  f32x4 acc[CB][NT], lacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float s2 = a.sink ? a.sink[head[cb]] * kLog2e : kNegInf;
    m[cb] = s2;
    lacc[cb] = f32x4{(grp == 0 && s2 > kNegInf) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[cb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = (c == 0) ? 0x3f803f80u : 0u;        // bf16 pair (1, 1) on row 0
  const bf16x8 ones = as_bf16x8(make_uint4(one2, one2, one2, one2));

  // per-lane LDS offsets of the MFMA operands
  const int koffA = c * KPITCH + grp * 16;                               // K row c, chunk grp
  const int voffA = KBYTES + (4 * grp + (c >> 2)) * VPITCH + 8 * (c & 3);  // transpose origin

  __syncthreads();   // every wavefront has its q operands; the region becomes stage 0
  store_tile(0);
  if (ntiles > 1) load_tile(kstart + BK);

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();   // stage t%2 is written; every wave is done with stage (t+1)%2
    const int j0 = kstart + t * BK;
    const unsigned char* kst = smem + (t & 1) * STAGE_BYTES;
    const unsigned char* vst = kst;
    if (!wave_live || j0 > tw1 || (W > 0 && j0 + BK - 1 < tw0 - W + 1)) {
      // nothing of this tile is visible to this wave's rows
    } else {
    const bool need_mask = (j0 + BK - 1 > tw0) || (W > 0 && j0 < tw1 - W + 1);

    // -- S^T = K . Q^T for two 16-key sub-tiles ---------------------------
    f32x4 s[2][CB];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) s[sub][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 kf = as_bf16x8(ld16(kst + koffA + sub * 16 * KPITCH + ks * 64));
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) s[sub][cb] = mfma16(kf, qf[cb][ks], s[sub][cb]);
      }
    }

    if (need_mask) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        // key j0 + 4*grp + kk (kk = sub*16 + r) is visible iff dlo <= kk <= dhi
        const int dhi = tok[cb] - (j0 + 4 * grp);
        const int dlo = (W > 0) ? dhi - (W - 1) : -0x7fffffff;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kk = sub * 16 + r;
            if (kk > dhi || kk < dlo) s[sub][cb][r] = kNegInf;
          }
      }
    }

    // -- online softmax (base 2, lazy reference max) and P in bf16 --------
    // Fast path: P against the current reference m, checked lane-locally.
    // A row with no reference yet, or with a P above 2^kLazy, sends the
    // whole wave through the slow path: exact row max across the four lanes
    // of each row, rescale of O and l, and P again.
    bf16x8 pb[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float p[8];
      float ms = (m[cb] == kNegInf) ? 0.f : m[cb];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[sub * 4 + r] = fast_exp2(fmaf(s[sub][cb][r], c2, -ms));
      const float pm = fmaxf(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])),
                             fmaxf(fmaxf(p[4], p[5]), fmaxf(p[6], p[7])));
      if (__any(m[cb] == kNegInf || pm > kLazyPow)) {
        float mx = fmaxf(fmaxf(fmaxf(s[0][cb][0], s[0][cb][1]), fmaxf(s[0][cb][2], s[0][cb][3])),
                         fmaxf(fmaxf(s[1][cb][0], s[1][cb][1]), fmaxf(s[1][cb][2], s[1][cb][3])));
        mx = max_across_groups(mx) * c2;
        const float mn = fmaxf(m[cb], mx);
        if (mn > m[cb]) {
          const float alpha = fast_exp2(m[cb] - mn);
          lacc[cb] *= alpha;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[cb][tt] *= alpha;
          m[cb] = mn;
        }
        ms = (m[cb] == kNegInf) ? 0.f : m[cb];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[sub * 4 + r] = fast_exp2(fmaf(s[sub][cb][r], c2, -ms));
      }
      pb[cb] = as_bf16x8(pack8(p));
    }

    // -- O^T += V^T . P^T, V^T read with the transpose loads ----------------
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint2 lo = lds_tr4(vst + voffA + 32 * tt);
      const uint2 hi = lds_tr4(vst + voffA + 16 * VPITCH + 32 * tt);
      const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb][tt] = mfma16(vf, pb[cb], acc[cb][tt]);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) lacc[cb] = mfma16(ones, pb[cb], lacc[cb]);
    }
    // write tile t+1 into the other stage and start loading tile t+2
    if (t + 1 < ntiles) {
      store_tile((t + 1) & 1);
      if (t + 2 < ntiles) load_tile(j0 + 2 * BK);
    }
  }

  // ---- epilogue: o = O / l, rounded to bf16 -----------------------------
  // The O^T fragments go through LDS (the staging buffers are free once
  // every wavefront has left the loop) so that the global stores are 16 bytes
  // per lane and each instruction covers four whole 256-byte rows.
  float inv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float lt = __shfl(lacc[cb][0], c);   // row sum sits in lane (grp 0, c)
    inv[cb] = (lt > 0.f) ? 1.f / lt : 0.f;
  }
  __syncthreads();
  unsigned char* obuf = smem + wave * (16 * CB) * OPITCH;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint2 w = make_uint2(pack_bf16x2(acc[cb][t][0] * inv[cb], acc[cb][t][1] * inv[cb]),
                                 pack_bf16x2(acc[cb][t][2] * inv[cb], acc[cb][t][3] * inv[cb]));
      st8(obuf + (cb * 16 + c) * OPITCH + (16 * t + 4 * grp) * 2, w);
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < CB * 16 * (DV / 8) / 64; ++i) {
    const int idx = lane + 64 * i;
    const int rr = idx >> 4, ch = idx & 15;       // row of this wavefront, 16-byte chunk
    const int r = wave * 16 * CB + rr;
    const int tk = i0 + (r >> log2g);
    if (tk < n) {
      const int hd = g * G + (r & (G - 1));
      st16(Op + ((tokbase + tk) * a.hq + hd) * DV + 8 * ch, ld16(obuf + rr * OPITCH + 16 * ch));
    }
  }
}

bool prefill_bf16_supported(const AttnArgs& a) {
  const int G = a.hq / a.hkv;
  return a.d_qk == D && a.d_v == DV && G >= 1 && G <= ROWS && (G & (G - 1)) == 0 &&
         (a.half % 32) == 0 && 2 * a.half <= D;
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
  hipLaunchKernelGGL(prefill_bf16_kernel<2>, dim3((unsigned)total), dim3(256), 0, stream, a,
                     log2g, nblk, balance);
  return hipGetLastError();
}

}  // namespace hswa
