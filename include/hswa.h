/*
 * hswa.h - sliding-window attention with a learnable per-head sink, its
 * full-causal sibling, single-token decode and token-level sparse attention,
 * as a C ABI for AMD Instinct MI355X (gfx950).
 *
 * The operation (all entry points) is the one written out in
 * "MiMo-V2-Flash: Hybrid Sliding Window Attention Architecture" (rslog.cc):
 * for query row i of query head h with key set J_i,
 *     a_ij = (q~_i . k~_j) * scale                        (section 1.2 / 2.3)
 *     m_i  = max(max_j a_ij, sink_h)                      (section 4.4)
 *     s_ij = exp(a_ij - m_i) / (exp(sink_h - m_i) + sum_j' exp(a_ij' - m_i))
 *     o_i  = sum_j s_ij v_j                               (section 4.4)
 * where q~, k~ carry partial RoPE on the first R dims and V is not rotated.
 * The sink has no value vector: it only enlarges the denominator.
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller, dense
 *    (row-major, no padding) and 16-byte aligned.  The library never
 *    allocates, frees or synchronises, and keeps no state between calls
 *    except the thread-local text behind hswa_last_error().
 *  - dtype selects the element type of q, k, v and o (HSWA_F32 or
 *    HSWA_BF16).  Arithmetic accumulates in fp32.  sink is always fp32.
 *  - sink: fp32 [hq] device pointer, one value per QUERY head, in the units
 *    of the scaled scores a_ij; NULL means no sink (the -inf limit, i.e.
 *    the ordinary softmax).  A -inf entry disables the sink for that head.
 *    Entries must be finite or -inf.
 *  - scale: the factor on q.k; pass 0 for the default 1/sqrt(d_qk).
 *  - Partial RoPE: R = largest even integer <= rotary_fraction * d_qk.
 *    Dim r (r < R/2) pairs with dim r + R/2 and turns by the angle
 *    pos * rope_theta^(-2r/R); dims >= R are untouched.  rotary_fraction 0
 *    disables RoPE.  ("MiMo-V2.6-Flash hybrid SWA" (pwwt.cn), section 5,
 *    gives the fraction 0.334 and the bases 1e4 / 1e7; the pairing is a
 *    reading, the pages do not fix it.)
 *  - GQA: query head h reads kv head h / (hq / hkv); hq % hkv == 0.
 *  - stream: a hipStream_t passed as void*; NULL is the null stream.  Every
 *    call only enqueues work on it and returns.
 *  - workspace: caller-owned device scratch of at least the size the
 *    matching *_workspace_size() query returns (may be NULL when that size
 *    is 0).  Its contents on entry do not matter; it must not be shared by
 *    calls that may run at the same time.
 *  - Errors: every argument is validated before anything is enqueued.  On
 *    a non-OK status nothing has been enqueued and the outputs are
 *    untouched; hswa_last_error() describes the problem.  HSWA_ERR_HIP means
 *    the HIP runtime reported an error at launch.
 */
#ifndef HSWA_H
#define HSWA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSWA_OK = 0,
  HSWA_ERR_INVALID_ARGUMENT = 1,
  HSWA_ERR_UNSUPPORTED = 2,
  HSWA_ERR_HIP = 3
} hswa_status_t;

typedef enum { HSWA_F32 = 0, HSWA_BF16 = 1 } hswa_dtype_t;

typedef enum { HSWA_KV_RING = 0, HSWA_KV_CONTIGUOUS = 1 } hswa_kv_layout_t;

/* Bytes of workspace swa_sink_prefill / ga_prefill need: the cos/sin table
 * of the seqlen positions (seqlen * R/2 * 8 bytes) followed by a rotated copy
 * of K's first R dims (batch * seqlen * hkv * R * 2 bytes), each rounded up
 * to 256 bytes; 0 without RoPE. */
size_t hswa_prefill_workspace_size(int batch, int seqlen, int hkv, int d_qk,
                                   float rotary_fraction);

/*
 * Sliding-window prefill with a sink: the SWA layer of rslog.cc section 4.4.
 *   q [batch, seqlen, hq, d_qk], k [batch, seqlen, hkv, d_qk],
 *   v [batch, seqlen, hkv, d_v]  ->  o [batch, seqlen, hq, d_v].
 * Query token i (0-based) attends to keys max(0, i - window + 1) .. i, the
 * causal window of section 2.1 (W tokens including itself).  window <= 0
 * means the full causal prefix.  Token i has RoPE position pos_offset + i.
 */
hswa_status_t swa_sink_prefill(const void* q, const void* k, const void* v, const float* sink,
                               void* o, int batch, int seqlen, int hq, int hkv, int d_qk,
                               int d_v, int window, float scale, float rope_theta,
                               float rotary_fraction, long long pos_offset, hswa_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Global-attention prefill: the GA layer of rslog.cc sections 1 and 5 (full
 * causal key set, no sink term).  Same layouts as swa_sink_prefill; it is
 * that call with window = 0 and sink = NULL.
 */
hswa_status_t ga_prefill(const void* q, const void* k, const void* v, void* o, int batch,
                         int seqlen, int hq, int hkv, int d_qk, int d_v, float scale,
                         float rope_theta, float rotary_fraction, long long pos_offset,
                         hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Chunked prefill: the last q_len tokens of sequences of kv_len tokens whose
 * earlier tokens (a cached prefix) already have K and V: the fixed-size
 * prefill chunks of "MiMo v2.5 inference optimisation" (youngju.dev), section
 * on KV-cache restructuring and scheduling (16K-token chunks, throughput falling
 * as the prefix grows).  The same operation as swa_sink_prefill restricted to
 * those query rows.
 *   q [batch, q_len, hq, d_qk] (query token t is sequence position
 *   kv_len - q_len + t), k [batch, kv_len, hkv, d_qk],
 *   v [batch, kv_len, hkv, d_v]  ->  o [batch, q_len, hq, d_v].
 * Position p attends to keys max(0, p - window + 1) .. p (window <= 0 or
 * >= kv_len: the full causal prefix, the GA layer with sink = NULL).
 * RoPE position of sequence position p is pos_offset + p, for q and k.
 * Requires 0 <= q_len <= kv_len; q_len == kv_len is swa_sink_prefill.
 * Workspace: hswa_prefill_workspace_size(batch, kv_len, hkv, d_qk,
 * rotary_fraction).
 */
hswa_status_t swa_sink_prefill_chunk(const void* q, const void* k, const void* v,
                                     const float* sink, void* o, int batch, int q_len,
                                     int kv_len, int hq, int hkv, int d_qk, int d_v, int window,
                                     float scale, float rope_theta, float rotary_fraction,
                                     long long pos_offset, hswa_dtype_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * swa_sink_prefill_chunk over a cache whose keys are stored already rotated
 * at their positions (the convention of the decode caches and of
 * kv_cache_append): the prefill chunk of "MiMo v2.5 inference optimisation"
 * (youngju.dev), KV-cache restructuring and scheduling, reading its cached
 * prefix where it lives.  k_cache [batch, kv_len, hkv, d_qk] holds the
 * prefix and the chunk's own keys (appended first), v_cache the values; only
 * the queries are rotated.  Same operation, arguments, workspace and errors
 * as swa_sink_prefill_chunk otherwise.
 */
hswa_status_t swa_sink_prefill_chunk_cached(const void* q, const void* k_cache, const void* v_cache,
                                            const float* sink, void* o, int batch, int q_len,
                                            int kv_len, int hq, int hkv, int d_qk, int d_v,
                                            int window, float scale, float rope_theta,
                                            float rotary_fraction, long long pos_offset,
                                            hswa_dtype_t dtype, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* Bytes of workspace swa_sink_decode needs for `batch` sequences whose
 * positions are all <= max_pos: split partial results (fp32), then the
 * query rotated to its position (bf16, 192 dims per head). */
size_t hswa_decode_workspace_size(hswa_kv_layout_t layout, int batch, int hq, int d_v,
                                  int window, long long max_pos);

/*
 * Single-token decode: one new query per sequence against its KV cache.
 *   q [batch, hq, d_qk] (RoPE at position pos[b] is applied in the call; the
 *   cache holds keys already rotated when they were written), o [batch, hq, d_v].
 *   pos: int64 [batch] DEVICE array, the position of each sequence's query;
 *   the caller has already written that token's key and value into the cache.
 *   max_pos: host-side upper bound on every pos[b] (sizes the launch).
 * HSWA_KV_RING ("MiMo v2.5 inference optimisation" (youngju.dev): the SWA pool
 *   holds only the window):
 *   k_cache [batch, window, hkv, d_qk], v_cache [batch, window, hkv, d_v];
 *   token t lives in slot t mod window; slots not yet written (pos < window-1)
 *   are ignored.  seq_offsets must be NULL and window > 0.
 * HSWA_KV_CONTIGUOUS (the full-attention pool, O(sequence length)):
 *   k_cache [total_rows, hkv, d_qk], v_cache [total_rows, hkv, d_v];
 *   sequence b owns rows seq_offsets[b] .. seq_offsets[b+1]-1 (int64 [batch+1]
 *   DEVICE array) and its token t is row seq_offsets[b] + t.  The query
 *   attends to tokens max(0, pos-window+1) .. pos (window > 0) or 0 .. pos
 *   (window == 0: a GA layer).
 * A sequence whose pos is negative, above max_pos, or (contiguous) not below
 * its row count gets NaN outputs; nothing outside the cache is read.
 */
hswa_status_t swa_sink_decode(const void* q, const void* k_cache, const void* v_cache,
                              hswa_kv_layout_t layout, const long long* seq_offsets,
                              const long long* pos, const float* sink, void* o, int batch,
                              int hq, int hkv, int d_qk, int d_v, int window, long long max_pos,
                              float scale, float rope_theta, float rotary_fraction,
                              hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Bytes of the static device scratch behind swa_sink_decode_noalloc. */
#define HSWA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * swa_sink_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same operation, arguments, contract and
 * errors as swa_sink_decode; the scratch it needs comes from a device array
 * inside the library of HSWA_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held
 * from the first call on that GPU until the process ends.  A call whose
 * hswa_decode_workspace_size() exceeds that maximum fails with
 * HSWA_ERR_INVALID_ARGUMENT before anything is enqueued.  The call allocates
 * and frees nothing.  All calls on one GPU share its array: calls that may
 * run at the same time on one GPU (different streams or host threads) race
 * and must not be issued.
 */
hswa_status_t swa_sink_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      hswa_kv_layout_t layout, const long long* seq_offsets,
                                      const long long* pos, const float* sink, void* o, int batch,
                                      int hq, int hkv, int d_qk, int d_v, int window,
                                      long long max_pos, float scale, float rope_theta,
                                      float rotary_fraction, hswa_dtype_t dtype, void* stream);

/*
 * Appending q_len new tokens per sequence to a decode cache, ahead of the
 * decode (or multi-token decode) call that reads them: the ring of an SWA
 * layer, whose pool is bounded by the window ("MiMo v2.5 inference
 * optimisation" (youngju.dev): token j in slot j mod ring_slots), or the
 * contiguous pool of a GA layer (row seq_offsets[b] + j).
 *   k_new [batch, q_len, hkv, d_qk], v_new [batch, q_len, hkv, d_v] (dtype):
 *   token t of sequence b is position pos[b] + t (pos: int64 [batch] DEVICE
 *   array; max_pos: host bound on every pos[b] + q_len - 1).
 *   Caches: as swa_sink_decode (ring [batch, ring_slots, hkv, d]; contiguous
 *   [rows, hkv, d] with seq_offsets, ring_slots 0), of type dtype.
 * Keys are stored rotated: the partial RoPE at the token's position, in
 * float32 steps (cos/sin of the float64 angle rounded to float32, each
 * product and the difference / sum rounded on its own), then rounded to the
 * cache type.  Values are copied.  Tokens whose position is negative, above
 * max_pos or (contiguous) not below their sequence's row count are not
 * written.  d_qk, d_v and the rotated half-width R/2 must be multiples of 8,
 * and R/2 at most 64.
 */
hswa_status_t kv_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              hswa_kv_layout_t layout, int ring_slots,
                              const long long* seq_offsets, const long long* pos, int batch,
                              int q_len, int hkv, int d_qk, int d_v, long long max_pos,
                              float rope_theta, float rotary_fraction, hswa_dtype_t dtype,
                              void* stream);

/*
 * The same into E4M3 caches (one byte per element, as swa_sink_decode_fp8):
 * each stored value is the E4M3 code of the float32 quotient value /
 * k_scale[g] (rotated key) or value / v_scale[g], rounded to nearest with
 * ties to the even code and saturated to +-448.  dtype is the type of k_new
 * and v_new; k_scale, v_scale: fp32 [hkv] DEVICE arrays.
 */
hswa_status_t kv_cache_append_fp8(const void* k_new, const void* v_new, void* k_cache,
                                  void* v_cache, const float* k_scale, const float* v_scale,
                                  hswa_kv_layout_t layout, int ring_slots,
                                  const long long* seq_offsets, const long long* pos, int batch,
                                  int q_len, int hkv, int d_qk, int d_v, long long max_pos,
                                  float rope_theta, float rotary_fraction, hswa_dtype_t dtype,
                                  void* stream);

/* Bytes of workspace swa_sink_decode_multi needs: as hswa_decode_workspace_size
 * with batch * q_len query rows and the key range of the longest query. */
size_t hswa_decode_multi_workspace_size(hswa_kv_layout_t layout, int batch, int q_len, int hq,
                                        int d_v, int window, int ring_slots, long long max_pos);

/*
 * Multi-token decode: one verification step of multi-token prediction, the
 * last accepted token and its drafts checked in one pass ("visual reading:
 * MiMo MTP/SWA, not MLA" (syt-nju.github.io), MTP section).
 *   q [batch, q_len, hq, d_qk]: query t of sequence b is the token at
 *   position pos[b] + t; o [batch, q_len, hq, d_v].  RoPE rotates query t at
 *   its position in the call; the cache holds keys already rotated.
 *   pos: int64 [batch] DEVICE array; the caller has written the keys and
 *   values of positions up to pos[b] + q_len - 1.  max_pos: host-side bound
 *   on every pos[b] + q_len - 1.
 * Query t attends to positions max(0, p - window + 1) .. p, p = pos[b] + t
 * (window == 0: 0 .. p): causal among the drafts too.
 * HSWA_KV_RING: k_cache [batch, ring_slots, hkv, d_qk], v_cache
 *   [batch, ring_slots, hkv, d_v], token j in slot j mod ring_slots;
 *   window > 0 and ring_slots >= window + q_len - 1, so that the drafts have
 *   not overwritten a key the first query sees.  seq_offsets must be NULL.
 * HSWA_KV_CONTIGUOUS: as swa_sink_decode (seq_offsets [batch+1]);
 *   ring_slots must be 0; every pos[b] + q_len - 1 must be below its row count.
 * A sequence breaking the contract gets NaN outputs; nothing outside the
 * cache is read.  q_len == 1 with ring_slots == window is swa_sink_decode.
 */
hswa_status_t swa_sink_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                                    hswa_kv_layout_t layout, int ring_slots,
                                    const long long* seq_offsets, const long long* pos,
                                    const float* sink, void* o, int batch, int q_len, int hq,
                                    int hkv, int d_qk, int d_v, int window, long long max_pos,
                                    float scale, float rope_theta, float rotary_fraction,
                                    hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * Single-token decode over an FP8 KV cache: a cache narrowed by the window
 * and stored in FP8 ("MiMo v2.5 inference optimisation" (youngju.dev),
 * closing section: the two savings stack; "MiMo-V3 HySparse2"
 * (aideepthink.cn), section 5, sizes its KV cache in FP8).  Same operation,
 * layouts, pos / max_pos / seq_offsets contract, workspace
 * (hswa_decode_workspace_size) and error behaviour as swa_sink_decode,
 * except:
 *   k_cache, v_cache hold one byte per element, an OCP FP8 E4M3 code
 *   (sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 *   S.1111.111 is NaN and must not occur);
 *   k_scale, v_scale: fp32 [hkv] DEVICE arrays: element d of kv head g's key
 *   has the value e4m3(code) * k_scale[g], of its value vector
 *   e4m3(code) * v_scale[g].
 * dtype selects q and o (HSWA_BF16 or HSWA_F32).  E4M3 values are exact in
 * bf16, so the cache enters the products unrounded.
 */
hswa_status_t swa_sink_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale,
                                  hswa_kv_layout_t layout, const long long* seq_offsets,
                                  const long long* pos, const float* sink, void* o, int batch,
                                  int hq, int hkv, int d_qk, int d_v, int window,
                                  long long max_pos, float scale, float rope_theta,
                                  float rotary_fraction, hswa_dtype_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of workspace sparse_sink_attn needs: same layout and size as
 * hswa_prefill_workspace_size (0 without RoPE). */
size_t hswa_sparse_workspace_size(int batch, int seqlen, int hkv, int d_qk,
                                  float rotary_fraction);

/*
 * Token-level sparse attention on one shared cache ("MiMo-V3 HySparse2"
 * (aideepthink.cn), section 4): query i of kv group g attends to the
 * recent_window most recent tokens max(0, i-recent_window+1) .. i plus the
 * selected tokens sel_idx[b, i, g, 0 : sel_count[b, i, g]].
 *   q [batch, seqlen, hq, d_qk], k/v [batch, seqlen, hkv, d_qk / d_v],
 *   sel_idx int32 [batch, seqlen, hkv, max_sel], sel_count int32 [batch, seqlen, hkv],
 *   o [batch, seqlen, hq, d_v].  Token i has RoPE position pos_offset + i.
 * Caller contract: each list is sorted ascending and distinct, and every
 * entry lies in [0, i - recent_window].  Entries outside that range are
 * skipped (so nothing outside k/v is read); counts are clamped to
 * [0, max_sel].
 */
hswa_status_t sparse_sink_attn(const void* q, const void* k, const void* v, const int* sel_idx,
                               const int* sel_count, int max_sel, int recent_window,
                               const float* sink, void* o, int batch, int seqlen, int hq,
                               int hkv, int d_qk, int d_v, float scale, float rope_theta,
                               float rotary_fraction, long long pos_offset, hswa_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_sink_attn over FP8 K/V: the sparse attention of "MiMo-V3
 * HySparse2" (aideepthink.cn), section 4, on one shared cache kept in FP8
 * (the same page, section 5, sizes its KV cache in FP8).  Same operation,
 * layouts, selection contract, workspace (hswa_sparse_workspace_size) and
 * error behaviour as sparse_sink_attn, except:
 *   k, v hold one byte per element, an OCP FP8 E4M3 code (as
 *   swa_sink_decode_fp8; NaN codes must not occur);
 *   k_scale, v_scale: fp32 [hkv] DEVICE arrays; element d of token j's key in
 *   kv head g is e4m3(code) * k_scale[g], of its value e4m3(code) * v_scale[g].
 * RoPE (rotary_fraction > 0) rotates those key values at their positions, as
 * for sparse_sink_attn.  dtype selects q and o (HSWA_BF16 or HSWA_F32).
 */
hswa_status_t sparse_sink_attn_fp8(const void* q, const void* k, const void* v,
                                   const float* k_scale, const float* v_scale, const int* sel_idx,
                                   const int* sel_count, int max_sel, int recent_window,
                                   const float* sink, void* o, int batch, int seqlen, int hq,
                                   int hkv, int d_qk, int d_v, float scale, float rope_theta,
                                   float rotary_fraction, long long pos_offset,
                                   hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Bytes of workspace sparse_select_tokens needs: rotated copies of q and k
 * (bf16, full rows) when RoPE is on, each rounded up to 256 bytes, then the
 * log-sum-exp rows (fp32 [batch, seqlen, hq], rounded up to 256 bytes), then
 * the importance scratch: 256 slots (one per resident workgroup) of 32 rows,
 * each row round64(seqlen) 4-byte words plus a 4096-entry list of 8 bytes.
 * The scratch grows linearly in seqlen and not with batch: about 2.4 GB at
 * seqlen = 65536.  0 for invalid arguments. */
size_t hswa_select_workspace_size(int batch, int seqlen, int hq, int hkv, int d_qk,
                                  float rotary_fraction);

/*
 * Token selection for the sparse layers: the selection indices the sparse
 * layers reuse from the preceding full-attention layer ("MiMo-V3 HySparse2"
 * (aideepthink.cn), section 4).  For query i (position pos_offset + i) and
 * kv head g the importance of token j is the full-attention layer's softmax
 * probability summed over the group's query heads,
 *     I_j = sum_{h in g} exp(a_hij - lse_hi),   a as swa_sink_prefill, over 0 .. i,
 * (no sink: a full-attention layer); the candidates are 0 .. i -
 * recent_window, and the min(max_sel, i - recent_window + 1) of largest
 * importance are kept, equal importances going to the lower position.
 * Importances are compared at 22 bits of their fp32 pattern (exponent and 13
 * mantissa bits): keys that agree to that resolution count as equal.
 *   q [batch, seqlen, hq, d_qk], k [batch, seqlen, hkv, d_qk] (bf16; d_qk =
 *   192 and hq = 16 * hkv);  sel_idx int32 [batch, seqlen, hkv, max_sel]
 *   (ascending, padded with -1), sel_count int32 [batch, seqlen, hkv]: the
 *   layout sparse_sink_attn reads.  RoPE as swa_sink_prefill (half-width a
 *   multiple of 8, at most 64); workspace: hswa_select_workspace_size().
 */
hswa_status_t sparse_select_tokens(const void* q, const void* k, int* sel_idx, int* sel_count,
                                   int max_sel, int recent_window, int batch, int seqlen, int hq,
                                   int hkv, int d_qk, float scale, float rope_theta,
                                   float rotary_fraction, long long pos_offset,
                                   hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Text for the last non-OK status returned on this thread ("" if none). */
const char* hswa_last_error(void);

/* Library version string. */
const char* hswa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HSWA_H */
