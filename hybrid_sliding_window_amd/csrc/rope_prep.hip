// Partial-RoPE preparation for a run of consecutive positions.
//
// "MiMo-V2.6-Flash hybrid SWA" (pwwt.cn), section 5: about a third of the
// q/k dims rotate (partial_rotary_factor 0.334), with base 1e4 in SWA layers
// and 1e7 in GA layers.  Pair r of R/2 turns by pos * theta^(-2r/R).
//
// Two kernels, run once per call:
//  * rope_table_kernel: cos/sin of every (position, pair).  Angles reach
//    2.6e5 rad for long contexts, where an fp32 product alone loses ~1e-2
//    rad, so the angle is formed and evaluated in fp64 and rounded once.
//  * rope_k_kernel: the first R dims of every K row, rotated and rounded to
//    bf16 once.  Attention kernels read these instead of re-rotating a key
//    for every query block whose window covers it.
#include "common.h"
#include "launch.h"

namespace hswa {

__global__ void rope_table_kernel(float2* __restrict__ table, long long pos0, int npos, int half,
                                  double theta) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)npos * half) return;
  const int r = (int)(idx % half);
  const long long t = idx / half;
  const double inv_freq = pow(theta, -(double)r / (double)half);
  const double angle = (double)(pos0 + t) * inv_freq;
  double s, c;
  sincos(angle, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

// Row `u` of the rows of tokens first..n-1 of every sequence (B * (n -
// first) * hkv of them) is row kv_row of K and krot, of token j.
__device__ __forceinline__ void tail_row(long long u, int n, int first, int hkv,
                                         long long* kv_row, long long* j) {
  const long long per_seq = (long long)(n - first) * hkv;
  const long long b = u / per_seq;
  const long long rem = u - b * per_seq;
  *kv_row = (b * n + first) * hkv + rem;
  *j = first + rem / hkv;
}

// One thread per (K row, 8-dim chunk c < R/16): rotates dims 8c..8c+7 with
// their partners R/2 further on and writes both to the rotated-K buffer
// krot [B * n * hkv, R].  Only the rows of tokens first..n-1 are written
// (rows = B * (n - first) * hkv); token j uses table row j.
__global__ void rope_k_kernel(const bf16_t* __restrict__ k, const float2* __restrict__ table,
                              bf16_t* __restrict__ krot, long long rows, int n, int first,
                              int hkv, int d, int half) {
  const int cpr = half >> 3;                   // chunk pairs per row
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cpr) return;
  const long long u = idx / cpr;
  const int c = (int)(idx - u * cpr);
  long long row, j;
  tail_row(u, n, first, hkv, &row, &j);
  const bf16_t* src = k + row * d;
  float f0[8], f1[8];
  unpack8(ld16(src + 8 * c), f0);
  unpack8(ld16(src + 8 * c + half), f1);
  const float2* t = table + j * half + 8 * c;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 cs = t[e];
    const float y0 = f0[e] * cs.x - f1[e] * cs.y;
    const float y1 = f1[e] * cs.x + f0[e] * cs.y;
    f0[e] = y0;
    f1[e] = y1;
  }
  bf16_t* dst = krot + row * (2 * half);
  st16(dst + 8 * c, pack8(f0));
  st16(dst + 8 * c + half, pack8(f1));
}

// The same for K stored as E4M3 codes: the codes' values (exact in fp32)
// are rotated and rounded to bf16 once.  The per-head scale is not applied:
// rotation is linear, so the attention kernel multiplies the whole score by
// it instead.
__global__ void rope_k_e4m3_kernel(const uint8_t* __restrict__ k, const float2* __restrict__ table,
                                   bf16_t* __restrict__ krot, long long rows, int n, int first,
                                   int hkv, int d, int half) {
  const int cpr = half >> 3;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cpr) return;
  const long long u = idx / cpr;
  const int c = (int)(idx - u * cpr);
  long long row, j;
  tail_row(u, n, first, hkv, &row, &j);
  const uint8_t* src = k + row * d;
  const uint2 w0 = *reinterpret_cast<const uint2*>(src + 8 * c);
  const uint2 w1 = *reinterpret_cast<const uint2*>(src + 8 * c + half);
  float f0[8], f1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f0[e] = __builtin_amdgcn_cvt_f32_fp8((int)((e < 4 ? w0.x : w0.y) >> (8 * (e & 3))), 0);
    f1[e] = __builtin_amdgcn_cvt_f32_fp8((int)((e < 4 ? w1.x : w1.y) >> (8 * (e & 3))), 0);
  }
  const float2* t = table + j * half + 8 * c;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 cs = t[e];
    const float y0 = f0[e] * cs.x - f1[e] * cs.y;
    const float y1 = f1[e] * cs.x + f0[e] * cs.y;
    f0[e] = y0;
    f1[e] = y1;
  }
  bf16_t* dst = krot + row * (2 * half);
  st16(dst + 8 * c, pack8(f0));
  st16(dst + 8 * c + half, pack8(f1));
}

// The same rotation of K without a table, for attention kernels that also
// rotate q without one: the pair's frequency theta^(-r/half) (fp64, once per
// block into LDS) times the position gives the angle in revolutions in fp64,
// which is reduced to [0, 1) before the hardware sine and cosine (which take
// revolutions) evaluate it in fp32.
constexpr int kMaxHalf = 64;
__global__ void rope_k_direct_kernel(const bf16_t* __restrict__ k, bf16_t* __restrict__ krot,
                                     long long rows, int n, int first, int hkv, int d, int half,
                                     long long pos0, double theta) {
  __shared__ double rev[kMaxHalf];
  if ((int)threadIdx.x < half)
    rev[threadIdx.x] = pow(theta, -(double)threadIdx.x / (double)half) * 0.15915494309189535;
  __syncthreads();
  const int cpr = half >> 3;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cpr) return;
  const long long u = idx / cpr;
  const int c = (int)(idx - u * cpr);
  long long row, j;
  tail_row(u, n, first, hkv, &row, &j);
  const double pos = (double)(pos0 + j);
  const bf16_t* src = k + row * d;
  float f0[8], f1[8];
  unpack8(ld16(src + 8 * c), f0);
  unpack8(ld16(src + 8 * c + half), f1);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double turns = pos * rev[8 * c + e];
    const float f = (float)(turns - floor(turns));
    const float co = __builtin_amdgcn_cosf(f), si = __builtin_amdgcn_sinf(f);
    const float y0 = f0[e] * co - f1[e] * si;
    const float y1 = f1[e] * co + f0[e] * si;
    f0[e] = y0;
    f1[e] = y1;
  }
  bf16_t* dst = krot + row * (2 * half);
  st16(dst + 8 * c, pack8(f0));
  st16(dst + 8 * c + half, pack8(f1));
}

// Full rows with their first R dims rotated (the direct cos/sin of
// rope_k_direct_kernel) and the other dims copied: one thread per 8-dim
// chunk of the first half (rotated pair) or of the unrotated tail.
__global__ void rope_rows_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                 long long rows, int n, int heads, int d, int half, long long pos0,
                                 double theta) {
  __shared__ double rev[kMaxHalf];
  if ((int)threadIdx.x < half)
    rev[threadIdx.x] = pow(theta, -(double)threadIdx.x / (double)half) * 0.15915494309189535;
  __syncthreads();
  const int per = (d - half) >> 3;           // chunks: half/8 rotated pairs + (d - 2 half)/8 copies
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * per) return;
  const long long row = idx / per;
  const int c = (int)(idx - row * per);
  const bf16_t* s = src + row * d;
  bf16_t* o = dst + row * d;
  if (8 * c < half) {
    const double pos = (double)(pos0 + (row / heads) % n);
    float f0[8], f1[8];
    unpack8(ld16(s + 8 * c), f0);
    unpack8(ld16(s + 8 * c + half), f1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double turns = pos * rev[8 * c + e];
      const float f = (float)(turns - floor(turns));
      const float co = __builtin_amdgcn_cosf(f), si = __builtin_amdgcn_sinf(f);
      const float y0 = f0[e] * co - f1[e] * si;
      const float y1 = f1[e] * co + f0[e] * si;
      f0[e] = y0;
      f1[e] = y1;
    }
    st16(o + 8 * c, pack8(f0));
    st16(o + 8 * c + half, pack8(f1));
  } else {
    const int d0 = 8 * c + half;             // past the rotated 2 * half dims
    st16(o + d0, ld16(s + d0));
  }
}

hipError_t launch_rope_rows(const uint16_t* src, uint16_t* dst, int B, int n, int heads, int d,
                            int half, long long pos0, double theta, hipStream_t stream) {
  const long long rows = (long long)B * n * heads;
  const long long total = rows * ((d - half) >> 3);
  if (total == 0) return hipSuccess;
  if (half > kMaxHalf || (half & 7) || (d & 7)) return hipErrorInvalidValue;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     reinterpret_cast<const bf16_t*>(src), reinterpret_cast<bf16_t*>(dst), rows,
                     n, heads, d, half, pos0, theta);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* table, long long pos0, int npos, int half, double theta,
                             hipStream_t stream) {
  const long long total = (long long)npos * half;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, table,
                     pos0, npos, half, theta);
  return hipGetLastError();
}

hipError_t launch_rope_k(const uint16_t* k, const float2* table, uint16_t* krot, int B, int n,
                         int first, int hkv, int d, int half, hipStream_t stream) {
  const long long rows = (long long)B * (n - first) * hkv;
  const long long total = rows * (half >> 3);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_k_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, k, table,
                     krot, rows, n, first, hkv, d, half);
  return hipGetLastError();
}

hipError_t launch_rope_k_e4m3(const uint8_t* k, const float2* table, uint16_t* krot, int B, int n,
                              int first, int hkv, int d, int half, hipStream_t stream) {
  const long long rows = (long long)B * (n - first) * hkv;
  const long long total = rows * (half >> 3);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_k_e4m3_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, k,
                     table, krot, rows, n, first, hkv, d, half);
  return hipGetLastError();
}

hipError_t launch_rope_k_direct(const uint16_t* k, uint16_t* krot, int B, int n, int first,
                                int hkv, int d, int half, long long pos0, double theta,
                                hipStream_t stream) {
  const long long rows = (long long)B * (n - first) * hkv;
  const long long total = rows * (half >> 3);
  if (total == 0) return hipSuccess;
  if (half > kMaxHalf) return hipErrorInvalidValue;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_k_direct_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, k,
                     krot, rows, n, first, hkv, d, half, pos0, theta);
  return hipGetLastError();
}

}  // namespace hswa
