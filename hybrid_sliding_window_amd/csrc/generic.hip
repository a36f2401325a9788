// Generic sink attention: one wavefront per query row, any head dims
// (d_qk, d_v <= 256), any GQA group, fp32 or bf16 storage, every key set.
//
// This is the fp32 path (exact to ~1e-6) and the path for shapes the
// matrix-core kernels do not cover.  Per key it forms the score with a
// wavefront reduction and updates a running (max, sum, output) triple; the
// result equals the two-pass definition of "MiMo-V2-Flash: Hybrid Sliding
// Window Attention Architecture" (rslog.cc) section 4.4 up to rounding:
// m starts at the sink and the sink's exp(sink - m) starts the sum.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace hswa {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, long long i) { return p[i]; }
  static __device__ __forceinline__ void put(float* p, long long i, float x) { p[i] = x; }
  static __device__ __forceinline__ void put_nan(float* p, long long i) {
    reinterpret_cast<uint32_t*>(p)[i] = 0x7fc00000u;
  }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float get(const bf16_t* p, long long i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void put(bf16_t* p, long long i, float x) {
    p[i] = f32_to_bf16_bits(x);
  }
  static __device__ __forceinline__ void put_nan(bf16_t* p, long long i) { p[i] = 0x7fc0u; }
};
// OCP E4M3 codes of an FP8 cache (read only); the hardware conversion is exact.
typedef uint8_t e4m3_t;
template <>
struct Elem<e4m3_t> {
  static __device__ __forceinline__ float get(const e4m3_t* p, long long i) {
    return __builtin_amdgcn_cvt_f32_fp8((int)p[i], 0);
  }
};

constexpr int kGenMaxPerLane = 4;  // dims per lane: 4 * 64 = 256

// Rotated value of dim d of a row: dim r < half pairs with r + half.
template <typename T>
__device__ __forceinline__ float rotated(const T* row, int d, int half, float c, float s) {
  if (d < half) return Elem<T>::get(row, d) * c - Elem<T>::get(row, d + half) * s;
  return Elem<T>::get(row, d) * c + Elem<T>::get(row, d - half) * s;
}

// T: storage of q and o; TKV: storage of k and v (T, or E4M3 codes whose
// values are code * kscale[g] / vscale[g]; decode and sparse modes).
template <typename T, typename TKV, int MODE>
__global__ __launch_bounds__(64) void generic_attn_kernel(AttnArgs a) {
  constexpr bool kFp8 = sizeof(TKV) == 1;
  const int lane = threadIdx.x;
  const long long row = blockIdx.x;
  const int h = (int)(row % a.hq);
  const long long outer = row / a.hq;          // prefill: b*nq + t; sparse: b*n + i; decode: b
  const int G = a.hq / a.hkv;
  const int g = h / G;
  const T* q = static_cast<const T*>(a.q);
  const TKV* k = static_cast<const TKV*>(a.k);
  const TKV* v = static_cast<const TKV*>(a.v);
  T* o = static_cast<T*>(a.o);
  const int R = 2 * a.half;

  long long b, i = 0;   // i: sequence position of the query (prefill / sparse)
  const T* qrow;
  if (MODE == MODE_PREFILL) {
    // query token t of a chunk sits at position qoff + t
    b = outer / a.nq;
    i = a.qoff + outer % a.nq;
    qrow = q + row * (long long)a.d_qk;
  } else if (MODE == MODE_SPARSE) {
    b = outer / a.n;
    i = outer % a.n;
    qrow = q + row * (long long)a.d_qk;
  } else {
    b = outer;
    qrow = q + (b * a.hq + h) * (long long)a.d_qk;
  }
  T* orow = o + row * (long long)a.d_v;

  // ---- key range of this row ------------------------------------------
  long long p = 0, kbase = 0, lo = 0, hi = -1;   // keys lo..hi (rows kbase + j)
  bool ok = true;
  if (MODE == MODE_PREFILL) {
    lo = (a.window > 0) ? (i - a.window + 1 > 0 ? i - a.window + 1 : 0) : 0;
    hi = i;
    kbase = b * a.n;
  } else if (MODE == MODE_SPARSE) {
    lo = (i - a.recent + 1 > 0) ? i - a.recent + 1 : 0;
    hi = i;
    kbase = b * a.n;
  } else if (MODE == MODE_DECODE_RING) {
    p = a.pos[b];
    ok = (p >= 0) && (p <= a.max_pos);
    lo = 0;
    hi = (p < a.window - 1) ? p : a.window - 1;      // slots written so far
    kbase = b * a.window;
  } else {
    p = a.pos[b];
    const long long off = a.seq_offsets[b], len = a.seq_offsets[b + 1] - off;
    ok = (p >= 0) && (p <= a.max_pos) && (p < len);
    lo = (a.window > 0) ? (p - a.window + 1 > 0 ? p - a.window + 1 : 0) : 0;
    hi = p;
    kbase = off;
  }
  if (!ok) {
    for (int d = lane; d < a.d_v; d += 64) Elem<T>::put_nan(orow, d);
    return;
  }

  // ---- rotated query in registers ------------------------------------
  float qd[kGenMaxPerLane];
#pragma unroll
  for (int u = 0; u < kGenMaxPerLane; ++u) {
    const int d = lane + 64 * u;
    qd[u] = 0.f;
    if (d >= a.d_qk) continue;
    if (d < R) {
      const int r = (d < a.half) ? d : d - a.half;
      float c, s;
      if (MODE == MODE_PREFILL || MODE == MODE_SPARSE) {
        const float2 cs = a.rope[i * a.half + r];
        c = cs.x;
        s = cs.y;
      } else {
        const double ang = (double)p * pow(a.rope_theta, -(double)r / (double)a.half);
        double sd, cd;
        sincos(ang, &sd, &cd);
        c = (float)cd;
        s = (float)sd;
      }
      qd[u] = rotated(qrow, d, a.half, c, s);
    } else {
      qd[u] = Elem<T>::get(qrow, d);
    }
  }

  // ---- running softmax state, seeded with the sink --------------------
  float m = a.sink ? a.sink[h] : kNegInf;
  float l = (m > kNegInf) ? 1.f : 0.f;
  float od[kGenMaxPerLane] = {0.f, 0.f, 0.f, 0.f};

  const float ksc = kFp8 ? a.kscale[g] : 1.f;
  const float vsc = kFp8 ? a.vscale[g] : 1.f;
  auto visit = [&](long long j) {
    const TKV* krow = k + ((kbase + j) * a.hkv + g) * (long long)a.d_qk;
    const TKV* vrow = v + ((kbase + j) * a.hkv + g) * (long long)a.d_v;
    const bool rot_k = (MODE == MODE_PREFILL || MODE == MODE_SPARSE) && R > 0 && !a.k_rotated;
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < kGenMaxPerLane; ++u) {
      const int d = lane + 64 * u;
      if (d >= a.d_qk) continue;
      float kv;
      if (rot_k && d < R) {
        const float2 cs = a.rope[j * a.half + ((d < a.half) ? d : d - a.half)];
        kv = rotated(krow, d, a.half, cs.x, cs.y);
      } else {
        kv = Elem<TKV>::get(krow, d);
      }
      part += qd[u] * kv;
    }
    const float sc = wave_sum(part) * (a.scale * ksc);
    const float mn = fmaxf(m, sc);
    const float alpha = expf(m - mn);           // m = -inf gives 0
    const float pj = expf(sc - mn);
    l = l * alpha + pj;
#pragma unroll
    for (int u = 0; u < kGenMaxPerLane; ++u) {
      const int d = lane + 64 * u;
      if (d < a.d_v) od[u] = od[u] * alpha + pj * Elem<TKV>::get(vrow, d);
    }
    m = mn;
  };

  if (MODE == MODE_SPARSE) {
    const long long li = (b * a.n + i) * a.hkv + g;
    int cnt = a.sel_count[li];
    cnt = cnt < 0 ? 0 : (cnt > a.max_sel ? a.max_sel : cnt);
    const int* sel = a.sel_idx + li * a.max_sel;
    for (int t = 0; t < cnt; ++t) {
      const long long j = sel[t];
      if (j >= 0 && j <= i - a.recent) visit(j);
    }
  }
  for (long long j = lo; j <= hi; ++j) visit(j);

  const float inv = (l > 0.f) ? vsc / l : 0.f;
#pragma unroll
  for (int u = 0; u < kGenMaxPerLane; ++u) {
    const int d = lane + 64 * u;
    if (d < a.d_v) Elem<T>::put(orow, d, od[u] * inv);
  }
}

template <typename T, typename TKV>
static hipError_t launch_t(const AttnArgs& a, int mode, hipStream_t stream) {
  long long rows = (mode == MODE_PREFILL)  ? (long long)a.B * a.nq * a.hq
                   : (mode == MODE_SPARSE) ? (long long)a.B * a.n * a.hq
                                           : (long long)a.B * a.hq;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)rows), block(64);
  switch (mode) {
    case MODE_PREFILL:
      hipLaunchKernelGGL((generic_attn_kernel<T, TKV, MODE_PREFILL>), grid, block, 0, stream, a);
      break;
    case MODE_SPARSE:
      hipLaunchKernelGGL((generic_attn_kernel<T, TKV, MODE_SPARSE>), grid, block, 0, stream, a);
      break;
    case MODE_DECODE_RING:
      hipLaunchKernelGGL((generic_attn_kernel<T, TKV, MODE_DECODE_RING>), grid, block, 0, stream,
                         a);
      break;
    default:
      hipLaunchKernelGGL((generic_attn_kernel<T, TKV, MODE_DECODE_CONTIG>), grid, block, 0,
                         stream, a);
      break;
  }
  return hipGetLastError();
}

// E4M3 K/V: the decode modes and sparse attention are built for them.
template <typename T>
static hipError_t launch_fp8(const AttnArgs& a, int mode, hipStream_t stream) {
  const long long rows = (mode == MODE_SPARSE) ? (long long)a.B * a.n * a.hq : (long long)a.B * a.hq;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)rows), block(64);
  if (mode == MODE_SPARSE)
    hipLaunchKernelGGL((generic_attn_kernel<T, e4m3_t, MODE_SPARSE>), grid, block, 0, stream, a);
  else if (mode == MODE_DECODE_RING)
    hipLaunchKernelGGL((generic_attn_kernel<T, e4m3_t, MODE_DECODE_RING>), grid, block, 0,
                       stream, a);
  else if (mode == MODE_DECODE_CONTIG)
    hipLaunchKernelGGL((generic_attn_kernel<T, e4m3_t, MODE_DECODE_CONTIG>), grid, block, 0,
                       stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_generic(const AttnArgs& a, int mode, bool bf16, bool kv_fp8, hipStream_t stream) {
  if (kv_fp8) return bf16 ? launch_fp8<bf16_t>(a, mode, stream) : launch_fp8<float>(a, mode, stream);
  return bf16 ? launch_t<bf16_t, bf16_t>(a, mode, stream) : launch_t<float, float>(a, mode, stream);
}

}  // namespace hswa
