// Streaming read/write bandwidth at a chosen mix of read and written bytes.
//
// The windowed prefill ("MiMo-V2-Flash: Hybrid Sliding Window Attention
// Architecture" (rslog.cc) sections 2.1 and 4.4) reads q, K and V once and
// writes the output once; at a 128-token window that traffic, not the
// matrix work, bounds it.  The chip's rate for such traffic is not the
// published HBM peak: it depends on the mix of reads and writes.  This probe
// moves the same bytes with no arithmetic: every wavefront owns a
// contiguous share of the source and of the destination and walks both
// together, eight 1 KB reads (16 bytes per lane, coalesced) and the
// writes that keep its written share in step with its read share, per
// iteration.  The loaded words are folded into one checksum per wavefront
// so that nothing is optimised away; the written words are a pattern that
// depends on no load, so the writes never wait for the reads.
#include "../../include/hswa_measure.h"
#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

constexpr int SP_WAVES = 4;     // wavefronts per workgroup
constexpr int SP_BURST = 8;     // 1 KB chunks per iteration and wavefront

__global__ __launch_bounds__(64 * SP_WAVES) void stream_probe_kernel(const uint4* __restrict__ src,
                                                                     long long rchunks,
                                                                     uint4* __restrict__ dst,
                                                                     long long wchunks,
                                                                     unsigned* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const long long nw = (long long)gridDim.x * SP_WAVES;
  const long long w = (long long)blockIdx.x * SP_WAVES + (threadIdx.x >> 6);
  const long long r0 = rchunks * w / nw, r1 = rchunks * (w + 1) / nw;
  const long long q0 = wchunks * w / nw, q1 = wchunks * (w + 1) / nw;
  unsigned sum = 0;
  long long r = r0, q = q0;
  while (r < r1 || q < q1) {   // wave-uniform
    const long long rn = min((long long)SP_BURST, r1 - r);
    uint4 x[SP_BURST];
    if (rn > 0) {
#pragma unroll
      for (int p = 0; p < SP_BURST; ++p) x[p] = src[min(r + p, r1 - 1) * 64 + lane];
      r += rn;
    }
    // written chunks due once r of the share's reads are issued
    const long long due = (r >= r1) ? q1 : q0 + (q1 - q0) * (r - r0) / (r1 - r0);
    const long long wn = min((long long)SP_BURST, due - q);
#pragma unroll
    for (int p = 0; p < SP_BURST; ++p)
      if (p < wn) dst[(q + p) * 64 + lane] = make_uint4((unsigned)(q + p), (unsigned)w, p, lane);
    if (wn > 0) q += wn;
    if (rn > 0) {
#pragma unroll
      for (int p = 0; p < SP_BURST; ++p) sum ^= x[p].x ^ x[p].y ^ x[p].z ^ x[p].w;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum ^= __shfl_xor(sum, m);
  if (lane == 0) out[w] = sum;
}

}  // namespace
}  // namespace hswa

extern "C" int hswa_stream_probe(const void* src, long long read_bytes, void* dst,
                                 long long write_bytes, int blocks, unsigned* out, void* stream) {
  if (!out || blocks <= 0 || read_bytes < 0 || write_bytes < 0 || read_bytes + write_bytes == 0)
    return hswa::api_fail(1, "hswa_stream_probe: null output, non-positive block count or no bytes");
  if ((read_bytes > 0 && !src) || (write_bytes > 0 && !dst))
    return hswa::api_fail(1, "hswa_stream_probe: null buffer for a non-zero byte count");
  if ((read_bytes | write_bytes) & 1023)
    return hswa::api_fail(1, "hswa_stream_probe: byte counts must be multiples of 1024");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
    return hswa::api_fail(1, "hswa_stream_probe: buffers must be 16-byte aligned");
  if ((long long)blocks * hswa::SP_WAVES > 0x7fffffffLL)
    return hswa::api_fail(1, "hswa_stream_probe: too many blocks");
  hipLaunchKernelGGL(hswa::stream_probe_kernel, dim3((unsigned)blocks), dim3(64 * hswa::SP_WAVES), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     read_bytes / 1024, static_cast<uint4*>(dst), write_bytes / 1024, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hswa::api_fail(3, hipGetErrorString(e));
  return 0;
}
