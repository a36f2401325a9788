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

#ifdef __cplusplus
}
#endif

#endif /* HSWA_MEASURE_H */
