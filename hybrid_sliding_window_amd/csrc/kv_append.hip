// Appending new tokens' keys and values to a decode cache.
//
// A decode (or MTP verification) step first writes the K/V of its new
// tokens into the cache the attention then reads: the ring of an SWA layer
// (token j in slot j mod S: "MiMo v2.5 inference optimisation"
// (youngju.dev), the SWA pool bounded by the window) or the contiguous pool
// of a GA layer.  The cache holds keys already rotated, so the append
// applies the partial RoPE at each token's position, then stores the row in
// the cache's format: bf16 / fp32 like the input, or E4M3 codes of
// value / scale (per kv head) rounded to nearest even and saturated to the
// largest finite code.
//
// 16- or 32-byte reads and writes, each byte moved once; the cos/sin of a
// rotated pair are evaluated once per token, all of a block's in parallel.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

// Cache row of token t of sequence b (layout 0: ring slot; 1: contiguous).
__device__ __forceinline__ long long append_row(const AttnArgs& a, int layout, int b, long long p) {
  if (layout == 0) return (long long)b * a.slots + p % a.slots;
  return a.seq_offsets[b] + p;
}

// fp32 -> E4M3 code: round to nearest, ties to even, |x| >= 448 saturates
// to +-448 (0x7E).  Written on the bit pattern so that the result does not
// depend on the conversion hardware.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (!(ax < 448.f)) return sign | 0x7Eu;
  if (ax < 0.015625f) {                            // below 2^-6: subnormal step 2^-9
    const float m = rintf(ax * 512.f);             // exact scaling; rint is ties-to-even
    return sign | (uint32_t)m;                     // m = 8 is the smallest normal, 0x08
  }
  int e = (int)((u >> 23) & 0xffu) - 127;          // -6 .. 8
  const uint32_t mant = u & 0x7fffffu;
  uint32_t m3 = mant >> 20;
  const uint32_t rem = mant & 0xfffffu;
  m3 += (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ? 1u : 0u;
  if (m3 == 8u) {
    m3 = 0u;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | m3;
}

// Rotation of the pair (x0, x1) by (c, s) in plain fp32 steps: each product
// and the difference / sum rounded on its own (no fused multiply-add), so
// that a quantised result is reproducible bit for bit.
__device__ __forceinline__ void rotate_pair(float& x0, float& x1, float c, float s) {
#pragma clang fp contract(off)
  const float a0 = x0 * c, b0 = x1 * s, a1 = x1 * c, b1 = x0 * s;
  x0 = a0 - b0;
  x1 = a1 + b1;
}

template <typename TIN>
__device__ __forceinline__ void load8(const TIN* p, float* f) {
  if constexpr (sizeof(TIN) == 2) {
    unpack8(ld16(p), f);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// OUT: 0 = same type as the input, 1 = E4M3 codes.
template <typename TIN, int OUT>
__device__ __forceinline__ void store8(void* base, long long elem, const float* f) {
  if constexpr (OUT == 1) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w0 |= e4m3_code(f[e]) << (8 * e);
#pragma unroll
    for (int e = 0; e < 4; ++e) w1 |= e4m3_code(f[4 + e]) << (8 * e);
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(base) + elem) = make_uint2(w0, w1);
  } else if constexpr (sizeof(TIN) == 2) {
    st16(static_cast<bf16_t*>(base) + elem, pack8(f));
  } else {
    float* o = static_cast<float*>(base) + elem;
    *reinterpret_cast<float4*>(o) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
}

}  // namespace

// A block serves TPB tokens.  First every (token, rotated pair) evaluates
// its cos/sin once, one per thread, into LDS; then the threads take the
// (token, kv head, 8-dim chunk) items: K chunks c < R/16 rotate a pair (dims
// 8c.. and their partners R/2 further on), the other K chunks and all V
// chunks are copied or quantised.
constexpr int TPB = 4;
constexpr int kMaxPairs = 64;

template <typename TIN, int OUT>
__global__ __launch_bounds__(256) void kv_append_kernel(AttnArgs a, int layout) {
  __shared__ float2 csn[TPB][kMaxPairs];
  const int half = a.half;
  const long long ntok = (long long)a.B * a.nq;
  const long long tok0 = (long long)blockIdx.x * TPB;
  for (int e = threadIdx.x; e < TPB * half; e += blockDim.x) {
    const int tl = e / half, r = e - tl * half;
    const long long bt = tok0 + tl;
    if (bt >= ntok) continue;
    const long long p = a.pos[bt / a.nq] + bt % a.nq;
    const double ang = (double)p * pow(a.rope_theta, -(double)r / (double)half);
    double sd, cd;
    sincos(ang, &sd, &cd);
    csn[tl][r] = make_float2((float)cd, (float)sd);
  }
  __syncthreads();
  const int kch = a.d_qk / 8 - half / 8;           // K items per head (pairs count once)
  const int vch = a.d_v / 8;
  const int per_head = kch + vch;
  const int per_tok = per_head * a.hkv;
  for (int it = threadIdx.x; it < TPB * per_tok; it += blockDim.x) {
    const int tl = it / per_tok;
    const int rem = it - tl * per_tok;
    const int g = rem / per_head;
    const int w = rem - g * per_head;
    const long long bt = tok0 + tl;
    if (bt >= ntok) continue;
    const int t = (int)(bt % a.nq);
    const int b = (int)(bt / a.nq);
    const long long p = a.pos[b] + t;
    if (p < 0 || p > a.max_pos) continue;          // contract broken: nothing is written
    if (layout == 1 && p >= a.seq_offsets[b + 1] - a.seq_offsets[b]) continue;
    const long long crow = append_row(a, layout, b, p) * a.hkv + g;
    if (w < kch) {
      const TIN* kin = static_cast<const TIN*>(a.k) + (bt * a.hkv + g) * a.d_qk;
      const float s = (OUT == 1) ? a.kscale[g] : 1.f;
      if (8 * w < half) {                          // rotated pair: dims 8w.. and 8w + half..
        const int d0 = 8 * w;
        float f0[8], f1[8];
        load8(kin + d0, f0);
        load8(kin + d0 + half, f1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = csn[tl][d0 + e];
          rotate_pair(f0[e], f1[e], cs.x, cs.y);
        }
        if (OUT == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            f0[e] = __fdiv_rn(f0[e], s);
            f1[e] = __fdiv_rn(f1[e], s);
          }
        }
        store8<TIN, OUT>(a.kout, crow * a.d_qk + d0, f0);
        store8<TIN, OUT>(a.kout, crow * a.d_qk + d0 + half, f1);
      } else {                                     // unrotated dims past the first R
        const int d0 = 8 * w + half;
        float f0[8];
        load8(kin + d0, f0);
        if (OUT == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) f0[e] = __fdiv_rn(f0[e], s);
        }
        store8<TIN, OUT>(a.kout, crow * a.d_qk + d0, f0);
      }
    } else {
      const int d0 = 8 * (w - kch);
      const TIN* vin = static_cast<const TIN*>(a.v) + (bt * a.hkv + g) * a.d_v;
      float f[8];
      load8(vin + d0, f);
      if (OUT == 1) {
        const float s = a.vscale[g];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = __fdiv_rn(f[e], s);
      }
      store8<TIN, OUT>(a.vout, crow * a.d_v + d0, f);
    }
  }
}

hipError_t launch_kv_append(const AttnArgs& a, int layout, bool bf16_in, bool e4m3_out,
                            hipStream_t stream) {
  const long long ntok = (long long)a.B * a.nq;
  if (ntok == 0) return hipSuccess;
  if (a.half > kMaxPairs) return hipErrorInvalidValue;
  const long long blocks = (ntok + TPB - 1) / TPB;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  if (bf16_in) {
    if (e4m3_out) hipLaunchKernelGGL((kv_append_kernel<bf16_t, 1>), grid, block, 0, stream, a, layout);
    else hipLaunchKernelGGL((kv_append_kernel<bf16_t, 0>), grid, block, 0, stream, a, layout);
  } else {
    if (e4m3_out) hipLaunchKernelGGL((kv_append_kernel<float, 1>), grid, block, 0, stream, a, layout);
    else hipLaunchKernelGGL((kv_append_kernel<float, 0>), grid, block, 0, stream, a, layout);
  }
  return hipGetLastError();
}

}  // namespace hswa
