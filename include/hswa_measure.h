/*
 * hswa_measure.h - measurement support of libhswa.so (not part of the
 * attention ABI in hswa.h).
 */
#ifndef HSWA_MEASURE_H
#define HSWA_MEASURE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Random-row gather probe: the access pattern of token-level sparse
 * attention ("MiMo-V3 HySparse2" (aideepthink.cn), section 4: each query
 * gathers its selected rows of one shared K/V cache) without its
 * arithmetic, to measure the gather bandwidth that bounds that kernel.
 *   k: bf16 [rows, 192], v: bf16 [rows, 128] DEVICE arrays (16-byte
 *   aligned); idx: int32 [nwaves * tiles_per_wave * 32] DEVICE array of row
 *   numbers (entries outside [0, rows) are clamped into it);
 *   out: uint32 [nwaves] DEVICE array receiving one checksum per wavefront.
 * Wavefront w reads the K and V rows idx[w * tiles_per_wave * 32 ...] in
 * tiles of 32 rows, each load 16 bytes wide, as the sparse kernel does.
 * Returns 0 (HSWA_OK), 1 (invalid argument, nothing enqueued) or 3 (launch
 * error); hswa_last_error() describes a failure.  Asynchronous on stream
 * (a hipStream_t as void*).
 */
int hswa_gather_probe(const void* k, const void* v, int rows, const int* idx, int nwaves,
                      int tiles_per_wave, unsigned* out, void* stream);

/*
 * Streaming probe: the traffic of the windowed prefill ("MiMo-V2-Flash:
 * Hybrid Sliding Window Attention Architecture" (rslog.cc) sections 2.1 and
 * 4.4: q, K and V read once, the output written once) without its
 * arithmetic, to measure the rate at which the chip moves a given mix of
 * read and written bytes.
 *   src: DEVICE array of read_bytes bytes, read once; dst: DEVICE array of
 *   write_bytes bytes, overwritten with a pattern; both 16-byte aligned,
 *   both counts multiples of 1024 (either may be 0, not both).
 *   blocks: workgroups of 4 wavefronts; out: uint32 [blocks * 4] DEVICE
 *   array receiving one checksum of the read words per wavefront.
 * Each wavefront reads and writes a contiguous share of each array,
 * interleaving its reads and writes in proportion.  Returns 0 (HSWA_OK),
 * 1 (invalid argument, nothing enqueued) or 3 (launch error);
 * hswa_last_error() describes a failure.  Asynchronous on stream (a
 * hipStream_t as void*).
 */
int hswa_stream_probe(const void* src, long long read_bytes, void* dst, long long write_bytes,
                      int blocks, unsigned* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSWA_MEASURE_H */
