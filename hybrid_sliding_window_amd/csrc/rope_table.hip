// cos/sin table of partial RoPE for a run of consecutive positions.
//
// "MiMo-V2.6-Flash hybrid SWA" (pwwt.cn), section 5: about a third of the
// q/k dims rotate (partial_rotary_factor 0.334), with base 1e4 in SWA layers
// and 1e7 in GA layers.  Pair r of R/2 turns by pos * theta^(-2r/R).
//
// Angles reach pos * 1 = 2.6e5 rad for long contexts, where an fp32
// product alone loses ~1e-2 rad.  The angle is therefore formed and its
// sine and cosine evaluated in fp64, then rounded once to fp32.
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

}  // namespace hswa
