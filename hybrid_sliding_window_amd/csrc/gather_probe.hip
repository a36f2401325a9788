// Random-row gather bandwidth of the token-level sparse attention's loads.
//
// "MiMo-V3 HySparse2" (aideepthink.cn), section 4: each query of a kv head
// reads up to 1024 selected rows plus 128 recent rows of one shared K/V
// cache.  At the sparse workload the cache (65536 tokens x 4 kv heads, K
// rows of 384 B, V rows of 256 B: 168 MB) fits in the 256 MB last-level
// cache, so the rate that bounds the sparse kernel is neither HBM's nor
// L2's but that of random-row gathers over a cache of that size.  This probe
// measures it with the sparse kernel's own access pattern: one wavefront per
// workgroup, tiles of 32 rows whose indices lanes 0..31 read, K rows loaded
// as six 16-byte pieces per lane group (lane (c, grp) reads bytes
// 16 grp + 64 ks of row c), V rows as four 16-byte pieces per lane (row
// 4 (u & 7) + q4, bytes 16 (u >> 3)), every load of a tile issued before
// any is used.  The loaded words are folded into one checksum per wavefront
// so that nothing is optimised away.
#include "../../include/hswa_measure.h"
#include "common.h"
#include "launch.h"

namespace hswa {
namespace {

constexpr int D = 192;
constexpr int DV = 128;
constexpr int KS = D / 32;
constexpr int BK = 32;

__global__ __launch_bounds__(64) void gather_probe_kernel(const bf16_t* __restrict__ K,
                                                          const bf16_t* __restrict__ V,
                                                          const int* __restrict__ idx, int rows,
                                                          int tiles, unsigned* __restrict__ out) {
  const int lane = threadIdx.x, c = lane & 15, grp = lane >> 4;
  const long long base = (long long)blockIdx.x * tiles * BK;
  unsigned sum = 0;
  for (int t = 0; t < tiles; ++t) {
    int myj = idx[base + t * BK + (lane & 31)];
    myj = min(max(myj, 0), rows - 1);   // every access stays inside the buffers
    uint4 kr[2][KS], vr[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int j = __shfl(myj, sub * 16 + c);
      const bf16_t* kp = K + (long long)j * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[sub][ks] = ld16(kp + 32 * ks);
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int u = lane + 64 * w;
      const int kq = u & 7, dc = u >> 3;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = __shfl(myj, 4 * kq + q4);
        vr[w][q4] = ld16(V + (long long)j * DV + 8 * dc);
      }
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sum ^= kr[sub][ks].x ^ kr[sub][ks].y ^ kr[sub][ks].z ^ kr[sub][ks].w;
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) sum ^= vr[w][q4].x ^ vr[w][q4].y ^ vr[w][q4].z ^ vr[w][q4].w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum ^= __shfl_xor(sum, m);
  if (lane == 0) out[blockIdx.x] = sum;
}

}  // namespace
}  // namespace hswa

extern "C" int hswa_gather_probe(const void* k, const void* v, int rows, const int* idx,
                                 int nwaves, int tiles_per_wave, unsigned* out, void* stream) {
  if (!k || !v || !idx || !out || rows <= 0 || nwaves <= 0 || tiles_per_wave <= 0)
    return hswa::api_fail(1, "hswa_gather_probe: null pointer or non-positive size");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15u)
    return hswa::api_fail(1, "hswa_gather_probe: k and v must be 16-byte aligned");
  if ((long long)nwaves * tiles_per_wave * 32 > 0x7fffffffLL)
    return hswa::api_fail(1, "hswa_gather_probe: index list too long");
  hipLaunchKernelGGL(hswa::gather_probe_kernel, dim3((unsigned)nwaves), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const hswa::bf16_t*>(k),
                     static_cast<const hswa::bf16_t*>(v), idx, rows, tiles_per_wave, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hswa::api_fail(3, hipGetErrorString(e));
  return 0;
}
