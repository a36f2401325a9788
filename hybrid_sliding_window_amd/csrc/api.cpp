// C ABI of the library: argument validation, workspace layout and dispatch
// to the kernels.  Every check happens before anything is enqueued, so a
// non-OK status leaves the outputs and the stream untouched.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "../../include/hswa.h"
#include "launch.h"

using hswa::AttnArgs;

namespace {

thread_local std::string g_last_error;

hswa_status_t fail(hswa_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

hswa_status_t ok() {
  g_last_error.clear();
  return HSWA_OK;
}

hswa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HSWA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Half the number of rotated dims: R/2 = floor(fraction * d / 2).
int rotary_half(int d_qk, float rotary_fraction) {
  return (int)std::floor((double)rotary_fraction * (double)d_qk / 2.0);
}

const int kMaxGenericDim = 256;

// Checks common to every entry point.  Returns HSWA_OK or the failing status.
hswa_status_t check_common(int batch, int hq, int hkv, int d_qk, int d_v, float scale,
                           float rope_theta, float rotary_fraction, hswa_dtype_t dtype) {
  if (batch < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "batch must be >= 0");
  if (hq <= 0 || hkv <= 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "head counts must be > 0");
  if (hq % hkv != 0)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "hq must be a multiple of hkv (GQA groups)");
  if (d_qk <= 0 || d_v <= 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "head dims must be > 0");
  if (!(scale >= 0.f) || std::isinf(scale))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "scale must be finite and >= 0 (0 = 1/sqrt(d_qk))");
  if (!(rotary_fraction >= 0.f && rotary_fraction <= 1.f))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "rotary_fraction must lie in [0, 1]");
  if (rotary_half(d_qk, rotary_fraction) > 0 && !(rope_theta > 0.f && std::isfinite(rope_theta)))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 0 when RoPE is on");
  if (dtype != HSWA_F32 && dtype != HSWA_BF16)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "dtype must be HSWA_F32 or HSWA_BF16");
  return HSWA_OK;
}

AttnArgs base_args(int batch, int n, int hq, int hkv, int d_qk, int d_v, float scale,
                   float rope_theta, float rotary_fraction) {
  AttnArgs a{};
  a.B = batch;
  a.n = n;
  a.nq = n;
  a.qoff = 0;
  a.hq = hq;
  a.hkv = hkv;
  a.d_qk = d_qk;
  a.d_v = d_v;
  a.half = rotary_half(d_qk, rotary_fraction);
  a.scale = (scale > 0.f) ? scale : (float)(1.0 / std::sqrt((double)d_qk));
  a.rope_theta = (double)rope_theta;
  return a;
}

bool generic_fits(int d_qk, int d_v) { return d_qk <= kMaxGenericDim && d_v <= kMaxGenericDim; }

size_t table_bytes(int seqlen, int d_qk, float rotary_fraction) {
  if (seqlen <= 0 || d_qk <= 0 || !(rotary_fraction >= 0.f && rotary_fraction <= 1.f)) return 0;
  const int half = rotary_half(d_qk, rotary_fraction);
  return round256((size_t)seqlen * (size_t)half * sizeof(float2));
}

// Rotated copy of K's first R dims (bf16), read by the matrix-core kernels.
size_t krot_bytes(int batch, int seqlen, int hkv, int d_qk, float rotary_fraction) {
  if (batch <= 0 || seqlen <= 0 || hkv <= 0 || d_qk <= 0) return 0;
  if (!(rotary_fraction >= 0.f && rotary_fraction <= 1.f)) return 0;
  const int half = rotary_half(d_qk, rotary_fraction);
  return round256((size_t)batch * seqlen * hkv * (size_t)(2 * half) * 2);
}

// Workspace of prefill and sparse calls: [cos/sin table][rotated K rows].
size_t rope_workspace_bytes(int batch, int seqlen, int hkv, int d_qk, float rotary_fraction) {
  const size_t t = table_bytes(seqlen, d_qk, rotary_fraction);
  return t == 0 ? 0 : t + krot_bytes(batch, seqlen, hkv, d_qk, rotary_fraction);
}

// Builds the table (and, for the matrix-core kernels, the rotated K rows) on
// the stream ahead of the attention kernel.  Without need_table (kernels that
// rotate q themselves) only the rotated K rows are built, by one kernel that
// evaluates its own cos/sin.  Only positions first..n-1 are prepared: no
// query of the call reads a key before `first` (a chunk behind a long
// prefix in a windowed layer).
hipError_t launch_rope_prep(AttnArgs& a, void* workspace, long long pos_offset, int first,
                            bool rotate_k, bool need_table, hipStream_t s, bool k_e4m3 = false) {
  if (a.half == 0 || (!rotate_k && !need_table)) return hipSuccess;
  float2* table = static_cast<float2*>(workspace);
  const size_t tb = round256((size_t)a.n * a.half * sizeof(float2));
  uint16_t* krot = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + tb);
  a.rope = table;
  a.krot = krot;
  if (rotate_k && !need_table) {
    return hswa::launch_rope_k_direct(static_cast<const uint16_t*>(a.k), krot, a.B, a.n, first,
                                      a.hkv, a.d_qk, a.half, pos_offset, a.rope_theta, s);
  }
  hipError_t e = hswa::launch_rope_table(table + (size_t)first * a.half, pos_offset + first,
                                         a.n - first, a.half, a.rope_theta, s);
  if (e != hipSuccess || !rotate_k) return e;
  if (k_e4m3)
    return hswa::launch_rope_k_e4m3(static_cast<const uint8_t*>(a.k), table, krot, a.B, a.n, first,
                                    a.hkv, a.d_qk, a.half, s);
  return hswa::launch_rope_k(static_cast<const uint16_t*>(a.k), table, krot, a.B, a.n, first,
                             a.hkv, a.d_qk, a.half, s);
}

// Prefill of the last q_len tokens of sequences of kv_len tokens (q_len ==
// kv_len: the whole sequence).  Query token t sits at sequence position
// kv_len - q_len + t.
hswa_status_t prefill_impl(const void* q, const void* k, const void* v, const float* sink, void* o,
                           int batch, int q_len, int kv_len, int hq, int hkv, int d_qk, int d_v,
                           int window, float scale, float rope_theta, float rotary_fraction,
                           long long pos_offset, hswa_dtype_t dtype, void* workspace,
                           size_t workspace_bytes, void* stream, bool k_rotated = false) {
  hswa_status_t st =
      check_common(batch, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction, dtype);
  if (st != HSWA_OK) return st;
  if (kv_len < 0 || q_len < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "lengths must be >= 0");
  if (q_len > kv_len) return fail(HSWA_ERR_INVALID_ARGUMENT, "q_len must not exceed kv_len");
  if (window < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "window must be >= 0 (0 = full causal)");
  if (batch == 0 || q_len == 0) return ok();
  if (!q || !k || !v || !o) return fail(HSWA_ERR_INVALID_ARGUMENT, "q, k, v and o must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");
  if ((long long)batch * kv_len * hq * (long long)(d_qk > d_v ? d_qk : d_v) > (1LL << 56))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "tensor too large");
  const size_t need = rope_workspace_bytes(batch, kv_len, hkv, d_qk, rotary_fraction);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace smaller than hswa_prefill_workspace_size()");
    if (!aligned16(workspace)) return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }

  AttnArgs a = base_args(batch, kv_len, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction);
  a.nq = q_len;
  a.qoff = kv_len - q_len;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.sink = sink;
  a.window = (window >= kv_len) ? 0 : window;
  a.pos_offset = pos_offset;
  a.k_rotated = k_rotated ? 1 : 0;

  // windowed layers: the kernel that keeps the window's K/V tiles resident;
  // the per-block bf16 kernel covers whole sequences only, chunks of the
  // shapes it serves run on the generic kernel
  const bool seq = (dtype == HSWA_BF16) && hswa::prefill_seq_supported(a);
  const bool causal = !seq && (dtype == HSWA_BF16) && hswa::prefill_causal_supported(a);
  const bool own_q = seq || causal;   // kernels that rotate q themselves
  const bool per_block = !own_q && (dtype == HSWA_BF16) && q_len == kv_len && !k_rotated &&
                         hswa::prefill_bf16_supported(a);
  const bool use_mfma = own_q || per_block;
  if (!use_mfma && !generic_fits(d_qk, d_v))
    return fail(HSWA_ERR_UNSUPPORTED, "head dims above 256 are not supported");

  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    // first key position any query of the call reads
    const int first = (a.window > 0 && a.qoff - a.window + 1 > 0) ? a.qoff - a.window + 1 : 0;
    // (the windowed kernel rotates its K tiles in LDS itself)
    hipError_t e = launch_rope_prep(a, workspace, pos_offset, first, use_mfma && !k_rotated && !seq,
                                    !own_q, s);
    if (e != hipSuccess) return hip_status(e, "rope preparation launch");
  }
  hipError_t e = seq         ? hswa::launch_prefill_seq(a, s)
                 : causal      ? hswa::launch_prefill_causal(a, s)
                 : per_block ? hswa::launch_prefill_bf16(a, s)
                             : hswa::launch_generic(a, hswa::MODE_PREFILL, dtype == HSWA_BF16, false, s);
  return hip_status(e, "prefill launch");
}

// Decode over bf16 / fp32 caches (kv_fp8 false) or E4M3 caches with per-kv-head
// scales (kv_fp8 true).
hswa_status_t decode_impl(const void* q, const void* k_cache, const void* v_cache, bool kv_fp8,
                          const float* k_scale, const float* v_scale, hswa_kv_layout_t layout,
                          const long long* seq_offsets, const long long* pos, const float* sink,
                          void* o, int batch, int hq, int hkv, int d_qk, int d_v, int window,
                          long long max_pos, float scale, float rope_theta, float rotary_fraction,
                          hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  hswa_status_t st =
      check_common(batch, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction, dtype);
  if (st != HSWA_OK) return st;
  if (layout != HSWA_KV_RING && layout != HSWA_KV_CONTIGUOUS)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "layout must be HSWA_KV_RING or HSWA_KV_CONTIGUOUS");
  if (window < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "window must be >= 0");
  if (layout == HSWA_KV_RING && window == 0)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "a ring cache needs window > 0 (its slot count)");
  if (layout == HSWA_KV_RING && seq_offsets)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "seq_offsets must be NULL for a ring cache");
  if (layout == HSWA_KV_CONTIGUOUS && !seq_offsets)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "seq_offsets is required for a contiguous cache");
  if (max_pos < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "max_pos must be >= 0");
  if (batch == 0) return ok();
  if (!q || !k_cache || !v_cache || !o || !pos)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, caches, pos and o must be non-null");
  if (kv_fp8 && (!k_scale || !v_scale))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "FP8 caches need k_scale and v_scale");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, caches and o must be 16-byte aligned");
  if (batch > 65535) return fail(HSWA_ERR_UNSUPPORTED, "batch above 65535");

  AttnArgs a = base_args(batch, 0, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction);
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.sink = sink;
  a.seq_offsets = seq_offsets;
  a.pos = pos;
  a.window = window;
  a.max_pos = max_pos;
  a.kscale = k_scale;
  a.vscale = v_scale;
  const int lay = (layout == HSWA_KV_RING) ? 0 : 1;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool mfma = dtype == HSWA_BF16 && (kv_fp8 ? hswa::decode_fp8_supported(a)
                                                  : hswa::decode_bf16_supported(a));
  if (mfma) {
    const size_t need = hswa_decode_workspace_size(layout, batch, hq, d_v, window, max_pos);
    if (!workspace || workspace_bytes < need)
      return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace smaller than hswa_decode_workspace_size()");
    if (!aligned16(workspace)) return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    hswa::decode_split_plan(lay, window, max_pos, &a.split_keys, &a.nsplit);
    a.ws = static_cast<float*>(workspace);
    // the (m, l) pairs follow the partial outputs directly: with d_v = 128 each
    // entry is 512 bytes, so the output region is already 256-byte aligned;
    // the rotated queries follow the (m, l) region
    const size_t per = (size_t)batch * hq * (size_t)a.nsplit;
    a.qrot = static_cast<unsigned char*>(workspace) + round256(per * (size_t)d_v * sizeof(float)) +
             round256(per * 2 * sizeof(float));
    return hip_status(kv_fp8 ? hswa::launch_decode_fp8(a, lay, s) : hswa::launch_decode_bf16(a, lay, s),
                      "decode launch");
  }
  if (!generic_fits(d_qk, d_v)) return fail(HSWA_ERR_UNSUPPORTED, "head dims above 256 are not supported");
  return hip_status(hswa::launch_generic(a, lay == 0 ? hswa::MODE_DECODE_RING
                                                     : hswa::MODE_DECODE_CONTIG,
                                         dtype == HSWA_BF16, kv_fp8, s),
                    "decode launch");
}

// Token-level sparse attention over bf16 / fp32 K/V (kv_fp8 false) or E4M3
// K/V codes with per-kv-head scales (kv_fp8 true).
hswa_status_t sparse_impl(const void* q, const void* k, const void* v, bool kv_fp8,
                          const float* k_scale, const float* v_scale, const int* sel_idx,
                          const int* sel_count, int max_sel, int recent_window, const float* sink,
                          void* o, int batch, int seqlen, int hq, int hkv, int d_qk, int d_v,
                          float scale, float rope_theta, float rotary_fraction,
                          long long pos_offset, hswa_dtype_t dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  hswa_status_t st =
      check_common(batch, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction, dtype);
  if (st != HSWA_OK) return st;
  if (seqlen < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "seqlen must be >= 0");
  if (max_sel < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "max_sel must be >= 0");
  if (recent_window < 1) return fail(HSWA_ERR_INVALID_ARGUMENT, "recent_window must be >= 1");
  if (batch == 0 || seqlen == 0) return ok();
  if (!q || !k || !v || !o || !sel_count || (max_sel > 0 && !sel_idx))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, k, v, o, sel_idx and sel_count must be non-null");
  if (kv_fp8 && (!k_scale || !v_scale))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "FP8 K/V need k_scale and v_scale");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");
  const size_t need = rope_workspace_bytes(batch, seqlen, hkv, d_qk, rotary_fraction);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace smaller than hswa_sparse_workspace_size()");
    if (!aligned16(workspace)) return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }

  AttnArgs a = base_args(batch, seqlen, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.sink = sink;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.max_sel = max_sel;
  a.recent = recent_window;
  a.pos_offset = pos_offset;
  a.kscale = k_scale;
  a.vscale = v_scale;

  const bool use_mfma = (dtype == HSWA_BF16) && (kv_fp8 ? hswa::sparse_fp8_supported(a)
                                                         : hswa::sparse_bf16_supported(a));
  if (!use_mfma && !generic_fits(d_qk, d_v))
    return fail(HSWA_ERR_UNSUPPORTED, "head dims above 256 are not supported");
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    hipError_t e = launch_rope_prep(a, workspace, pos_offset, 0, use_mfma, true, s, kv_fp8);
    if (e != hipSuccess) return hip_status(e, "rope preparation launch");
  }
  hipError_t e = !use_mfma ? hswa::launch_generic(a, hswa::MODE_SPARSE, dtype == HSWA_BF16, kv_fp8, s)
                 : kv_fp8  ? hswa::launch_sparse_fp8(a, s)
                           : hswa::launch_sparse_bf16(a, s);
  return hip_status(e, "sparse launch");
}

// Split plan of a multi-token decode: the longest key range is min(last + 1,
// S) slots of a ring, or W + q_len - 1 (W > 0) or last + 1 rows of a
// contiguous cache, where last = max_pos is the largest query position.
void multi_split_plan(hswa_kv_layout_t layout, int q_len, int window, int ring_slots,
                      long long max_pos, int* split_keys, int* nsplit) {
  if (layout == HSWA_KV_RING)
    hswa::decode_split_plan(0, ring_slots, max_pos, split_keys, nsplit);
  else
    hswa::decode_split_plan(1, window > 0 ? window + q_len - 1 : 0, max_pos, split_keys, nsplit);
}

// Cache append for bf16 / fp32 caches (e4m3 false) or E4M3 caches with
// per-kv-head scales (e4m3 true).
hswa_status_t append_impl(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          bool e4m3, const float* k_scale, const float* v_scale,
                          hswa_kv_layout_t layout, int ring_slots, const long long* seq_offsets,
                          const long long* pos, int batch, int q_len, int hkv, int d_qk, int d_v,
                          long long max_pos, float rope_theta, float rotary_fraction,
                          hswa_dtype_t dtype, void* stream) {
  hswa_status_t st =
      check_common(batch, hkv, hkv, d_qk, d_v, 0.f, rope_theta, rotary_fraction, dtype);
  if (st != HSWA_OK) return st;
  if (layout != HSWA_KV_RING && layout != HSWA_KV_CONTIGUOUS)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "layout must be HSWA_KV_RING or HSWA_KV_CONTIGUOUS");
  if (q_len < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "q_len must be >= 0");
  if (layout == HSWA_KV_RING) {
    if (ring_slots <= 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "a ring cache needs ring_slots > 0");
    if (seq_offsets) return fail(HSWA_ERR_INVALID_ARGUMENT, "seq_offsets must be NULL for a ring cache");
  } else {
    if (ring_slots != 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "ring_slots must be 0 for a contiguous cache");
    if (!seq_offsets) return fail(HSWA_ERR_INVALID_ARGUMENT, "seq_offsets is required for a contiguous cache");
  }
  if (max_pos < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "max_pos must be >= 0");
  const int half = rotary_half(d_qk, rotary_fraction);
  if (d_qk % 8 != 0 || d_v % 8 != 0 || half % 8 != 0 || half > 64)
    return fail(HSWA_ERR_UNSUPPORTED,
                "head dims and the rotated half-width must be multiples of 8 (half-width at most 64)");
  if (batch == 0 || q_len == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !pos)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "k_new, v_new, caches and pos must be non-null");
  if (e4m3 && (!k_scale || !v_scale))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "FP8 caches need k_scale and v_scale");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "k_new, v_new and the caches must be 16-byte aligned");
  AttnArgs a = base_args(batch, 0, hkv, hkv, d_qk, d_v, 0.f, rope_theta, rotary_fraction);
  a.k = k_new;
  a.v = v_new;
  a.kout = k_cache;
  a.vout = v_cache;
  a.kscale = k_scale;
  a.vscale = v_scale;
  a.seq_offsets = seq_offsets;
  a.pos = pos;
  a.max_pos = max_pos;
  a.nq = q_len;
  a.slots = ring_slots;
  return hip_status(hswa::launch_kv_append(a, layout == HSWA_KV_RING ? 0 : 1, dtype == HSWA_BF16,
                                           e4m3, static_cast<hipStream_t>(stream)),
                    "cache append launch");
}

}  // namespace

namespace hswa {
// Status and message for entry points defined outside this file.
int api_fail(int status, const char* msg) { return (int)fail((hswa_status_t)status, msg); }
}  // namespace hswa

extern "C" {

const char* hswa_last_error(void) { return g_last_error.c_str(); }

const char* hswa_version(void) { return "hswa 0.1.0 (gfx950)"; }

size_t hswa_prefill_workspace_size(int batch, int seqlen, int hkv, int d_qk,
                                   float rotary_fraction) {
  return rope_workspace_bytes(batch, seqlen, hkv, d_qk, rotary_fraction);
}

size_t hswa_sparse_workspace_size(int batch, int seqlen, int hkv, int d_qk,
                                  float rotary_fraction) {
  return rope_workspace_bytes(batch, seqlen, hkv, d_qk, rotary_fraction);
}

hswa_status_t swa_sink_prefill(const void* q, const void* k, const void* v, const float* sink,
                               void* o, int batch, int seqlen, int hq, int hkv, int d_qk,
                               int d_v, int window, float scale, float rope_theta,
                               float rotary_fraction, long long pos_offset, hswa_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (seqlen < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "seqlen must be >= 0");
  return prefill_impl(q, k, v, sink, o, batch, seqlen, seqlen, hq, hkv, d_qk, d_v, window, scale,
                      rope_theta, rotary_fraction, pos_offset, dtype, workspace, workspace_bytes,
                      stream);
}

hswa_status_t swa_sink_prefill_chunk(const void* q, const void* k, const void* v,
                                     const float* sink, void* o, int batch, int q_len,
                                     int kv_len, int hq, int hkv, int d_qk, int d_v, int window,
                                     float scale, float rope_theta, float rotary_fraction,
                                     long long pos_offset, hswa_dtype_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, sink, o, batch, q_len, kv_len, hq, hkv, d_qk, d_v, window, scale,
                      rope_theta, rotary_fraction, pos_offset, dtype, workspace, workspace_bytes,
                      stream);
}

hswa_status_t swa_sink_prefill_chunk_cached(const void* q, const void* k_cache, const void* v_cache,
                                            const float* sink, void* o, int batch, int q_len,
                                            int kv_len, int hq, int hkv, int d_qk, int d_v,
                                            int window, float scale, float rope_theta,
                                            float rotary_fraction, long long pos_offset,
                                            hswa_dtype_t dtype, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k_cache, v_cache, sink, o, batch, q_len, kv_len, hq, hkv, d_qk, d_v,
                      window, scale, rope_theta, rotary_fraction, pos_offset, dtype, workspace,
                      workspace_bytes, stream, true);
}

hswa_status_t ga_prefill(const void* q, const void* k, const void* v, void* o, int batch,
                         int seqlen, int hq, int hkv, int d_qk, int d_v, float scale,
                         float rope_theta, float rotary_fraction, long long pos_offset,
                         hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return swa_sink_prefill(q, k, v, nullptr, o, batch, seqlen, hq, hkv, d_qk, d_v, 0, scale,
                          rope_theta, rotary_fraction, pos_offset, dtype, workspace,
                          workspace_bytes, stream);
}

// Query dims the bf16 decode kernel handles (its rotated-q buffer size).
constexpr size_t kDecodeQDims = 192;

size_t hswa_decode_workspace_size(hswa_kv_layout_t layout, int batch, int hq, int d_v, int window,
                                  long long max_pos) {
  if (batch <= 0 || hq <= 0 || d_v <= 0 || max_pos < 0) return 0;
  if (layout != HSWA_KV_RING && layout != HSWA_KV_CONTIGUOUS) return 0;
  if (layout == HSWA_KV_RING && window <= 0) return 0;
  int split_keys = 0, nsplit = 0;
  hswa::decode_split_plan(layout == HSWA_KV_RING ? 0 : 1, window, max_pos, &split_keys, &nsplit);
  const size_t per = (size_t)batch * hq * (size_t)nsplit;
  return round256(per * (size_t)d_v * sizeof(float)) + round256(per * 2 * sizeof(float)) +
         round256((size_t)batch * hq * kDecodeQDims * 2);
}

size_t hswa_decode_multi_workspace_size(hswa_kv_layout_t layout, int batch, int q_len, int hq,
                                        int d_v, int window, int ring_slots, long long max_pos) {
  if (batch <= 0 || q_len <= 0 || hq <= 0 || d_v <= 0 || max_pos < 0) return 0;
  if (layout != HSWA_KV_RING && layout != HSWA_KV_CONTIGUOUS) return 0;
  if (layout == HSWA_KV_RING && ring_slots <= 0) return 0;
  int split_keys = 0, nsplit = 0;
  multi_split_plan(layout, q_len, window, ring_slots, max_pos, &split_keys, &nsplit);
  const size_t rows = (size_t)batch * q_len * hq;
  const size_t per = rows * (size_t)nsplit;
  return round256(per * (size_t)d_v * sizeof(float)) + round256(per * 2 * sizeof(float)) +
         round256(rows * kDecodeQDims * 2);
}

hswa_status_t swa_sink_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                                    hswa_kv_layout_t layout, int ring_slots,
                                    const long long* seq_offsets, const long long* pos,
                                    const float* sink, void* o, int batch, int q_len, int hq,
                                    int hkv, int d_qk, int d_v, int window, long long max_pos,
                                    float scale, float rope_theta, float rotary_fraction,
                                    hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  hswa_status_t st =
      check_common(batch, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction, dtype);
  if (st != HSWA_OK) return st;
  if (layout != HSWA_KV_RING && layout != HSWA_KV_CONTIGUOUS)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "layout must be HSWA_KV_RING or HSWA_KV_CONTIGUOUS");
  if (q_len < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "q_len must be >= 0");
  if (window < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "window must be >= 0");
  if (layout == HSWA_KV_RING) {
    if (window == 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "a ring cache serves a window > 0");
    if ((long long)ring_slots < (long long)window + q_len - 1)
      return fail(HSWA_ERR_INVALID_ARGUMENT, "ring_slots must be >= window + q_len - 1");
    if (seq_offsets) return fail(HSWA_ERR_INVALID_ARGUMENT, "seq_offsets must be NULL for a ring cache");
  } else {
    if (ring_slots != 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "ring_slots must be 0 for a contiguous cache");
    if (!seq_offsets) return fail(HSWA_ERR_INVALID_ARGUMENT, "seq_offsets is required for a contiguous cache");
  }
  if (max_pos < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "max_pos must be >= 0");
  if (batch == 0 || q_len == 0) return ok();
  if (!q || !k_cache || !v_cache || !o || !pos)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, caches, pos and o must be non-null");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, caches and o must be 16-byte aligned");
  if (batch > 65535 || q_len > 65535 || hq > 65535)
    return fail(HSWA_ERR_UNSUPPORTED, "batch, q_len and hq must be at most 65535");

  AttnArgs a = base_args(batch, 0, hq, hkv, d_qk, d_v, scale, rope_theta, rotary_fraction);
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.sink = sink;
  a.seq_offsets = seq_offsets;
  a.pos = pos;
  a.window = window;
  a.max_pos = max_pos;
  a.nq = q_len;
  a.slots = ring_slots;
  const int lay = (layout == HSWA_KV_RING) ? 0 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == HSWA_BF16 && hswa::decode_multi_supported(a)) {
    const size_t need = hswa_decode_multi_workspace_size(layout, batch, q_len, hq, d_v, window,
                                                         ring_slots, max_pos);
    if (!workspace || workspace_bytes < need)
      return fail(HSWA_ERR_INVALID_ARGUMENT,
                  "workspace smaller than hswa_decode_multi_workspace_size()");
    if (!aligned16(workspace)) return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    multi_split_plan(layout, q_len, window, ring_slots, max_pos, &a.split_keys, &a.nsplit);
    a.ws = static_cast<float*>(workspace);
    const size_t per = (size_t)batch * q_len * hq * (size_t)a.nsplit;
    a.qrot = static_cast<unsigned char*>(workspace) + round256(per * (size_t)d_v * sizeof(float)) +
             round256(per * 2 * sizeof(float));
    return hip_status(hswa::launch_decode_multi(a, lay, s), "multi-token decode launch");
  }
  if (!generic_fits(d_qk, d_v)) return fail(HSWA_ERR_UNSUPPORTED, "head dims above 256 are not supported");
  return hip_status(hswa::launch_decode_multi_generic(a, lay, dtype == HSWA_BF16, s),
                    "multi-token decode launch");
}

hswa_status_t kv_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              hswa_kv_layout_t layout, int ring_slots,
                              const long long* seq_offsets, const long long* pos, int batch,
                              int q_len, int hkv, int d_qk, int d_v, long long max_pos,
                              float rope_theta, float rotary_fraction, hswa_dtype_t dtype,
                              void* stream) {
  return append_impl(k_new, v_new, k_cache, v_cache, false, nullptr, nullptr, layout, ring_slots,
                     seq_offsets, pos, batch, q_len, hkv, d_qk, d_v, max_pos, rope_theta,
                     rotary_fraction, dtype, stream);
}

hswa_status_t kv_cache_append_fp8(const void* k_new, const void* v_new, void* k_cache,
                                  void* v_cache, const float* k_scale, const float* v_scale,
                                  hswa_kv_layout_t layout, int ring_slots,
                                  const long long* seq_offsets, const long long* pos, int batch,
                                  int q_len, int hkv, int d_qk, int d_v, long long max_pos,
                                  float rope_theta, float rotary_fraction, hswa_dtype_t dtype,
                                  void* stream) {
  return append_impl(k_new, v_new, k_cache, v_cache, true, k_scale, v_scale, layout, ring_slots,
                     seq_offsets, pos, batch, q_len, hkv, d_qk, d_v, max_pos, rope_theta,
                     rotary_fraction, dtype, stream);
}

hswa_status_t swa_sink_decode(const void* q, const void* k_cache, const void* v_cache,
                              hswa_kv_layout_t layout, const long long* seq_offsets,
                              const long long* pos, const float* sink, void* o, int batch,
                              int hq, int hkv, int d_qk, int d_v, int window, long long max_pos,
                              float scale, float rope_theta, float rotary_fraction,
                              hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_impl(q, k_cache, v_cache, false, nullptr, nullptr, layout, seq_offsets, pos, sink,
                     o, batch, hq, hkv, d_qk, d_v, window, max_pos, scale, rope_theta,
                     rotary_fraction, dtype, workspace, workspace_bytes, stream);
}

hswa_status_t swa_sink_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale,
                                  hswa_kv_layout_t layout, const long long* seq_offsets,
                                  const long long* pos, const float* sink, void* o, int batch,
                                  int hq, int hkv, int d_qk, int d_v, int window,
                                  long long max_pos, float scale, float rope_theta,
                                  float rotary_fraction, hswa_dtype_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, true, k_scale, v_scale, layout, seq_offsets, pos, sink,
                     o, batch, hq, hkv, d_qk, d_v, window, max_pos, scale, rope_theta,
                     rotary_fraction, dtype, workspace, workspace_bytes, stream);
}

size_t hswa_select_workspace_size(int batch, int seqlen, int hq, int hkv, int d_qk,
                                  float rotary_fraction) {
  if (batch <= 0 || seqlen <= 0 || hq <= 0 || hkv <= 0 || d_qk <= 0) return 0;
  if (!(rotary_fraction >= 0.f && rotary_fraction <= 1.f)) return 0;
  // [rotated q][rotated k] (RoPE only), then the log-sum-exp rows, then the
  // importance scratch
  const size_t tail = round256(hswa::select_lse_bytes(batch, seqlen, hq)) +
                      hswa::select_scratch_bytes(seqlen);
  if (rotary_half(d_qk, rotary_fraction) == 0) return tail;
  const size_t rows = (size_t)batch * seqlen;
  return round256(rows * hq * (size_t)d_qk * 2) + round256(rows * hkv * (size_t)d_qk * 2) + tail;
}

hswa_status_t sparse_select_tokens(const void* q, const void* k, int* sel_idx, int* sel_count,
                                   int max_sel, int recent_window, int batch, int seqlen, int hq,
                                   int hkv, int d_qk, float scale, float rope_theta,
                                   float rotary_fraction, long long pos_offset,
                                   hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  hswa_status_t st =
      check_common(batch, hq, hkv, d_qk, d_qk, scale, rope_theta, rotary_fraction, dtype);
  if (st != HSWA_OK) return st;
  if (seqlen < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "seqlen must be >= 0");
  if (max_sel < 0) return fail(HSWA_ERR_INVALID_ARGUMENT, "max_sel must be >= 0");
  if (recent_window < 1) return fail(HSWA_ERR_INVALID_ARGUMENT, "recent_window must be >= 1");
  AttnArgs a = base_args(batch, seqlen, hq, hkv, d_qk, d_qk, scale, rope_theta, rotary_fraction);
  if (dtype != HSWA_BF16 || !hswa::select_tokens_supported(a))
    return fail(HSWA_ERR_UNSUPPORTED, "token selection takes bf16 q/k with d_qk = 192 and 16 query heads per kv head");
  if (a.half > 0 && (a.half % 8 != 0 || a.half > 64))
    return fail(HSWA_ERR_UNSUPPORTED, "the rotated half-width must be a multiple of 8, at most 64");
  if (batch == 0 || seqlen == 0) return ok();
  if (!q || !k || !sel_count || (max_sel > 0 && !sel_idx))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "q, k, sel_idx and sel_count must be non-null");
  if (!aligned16(q) || !aligned16(k)) return fail(HSWA_ERR_INVALID_ARGUMENT, "q and k must be 16-byte aligned");
  if ((long long)batch * seqlen * hq * (long long)d_qk > (1LL << 56))
    return fail(HSWA_ERR_INVALID_ARGUMENT, "tensor too large");
  const size_t need = hswa_select_workspace_size(batch, seqlen, hq, hkv, d_qk, rotary_fraction);
  if (!workspace || workspace_bytes < need)
    return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace smaller than hswa_select_workspace_size()");
  if (!aligned16(workspace)) return fail(HSWA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  a.q = q;
  a.k = k;
  a.max_sel = max_sel;
  a.recent = recent_window;
  a.pos_offset = pos_offset;
  a.sel_out = sel_idx;
  a.cnt_out = sel_count;
  a.sel_ws = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + need -
                                         hswa::select_scratch_bytes(seqlen));
  a.sel_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(a.sel_ws) -
                                       round256(hswa::select_lse_bytes(batch, seqlen, hq)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.half > 0) {
    const size_t rows = (size_t)batch * seqlen;
    uint16_t* qr = static_cast<uint16_t*>(workspace);
    uint16_t* kr = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                               round256(rows * hq * (size_t)d_qk * 2));
    hipError_t e = hswa::launch_rope_rows(static_cast<const uint16_t*>(q), qr, batch, seqlen, hq,
                                          d_qk, a.half, pos_offset, a.rope_theta, s);
    if (e == hipSuccess)
      e = hswa::launch_rope_rows(static_cast<const uint16_t*>(k), kr, batch, seqlen, hkv, d_qk,
                                 a.half, pos_offset, a.rope_theta, s);
    if (e != hipSuccess) return hip_status(e, "rope preparation launch");
    a.qrot = qr;
    a.krot = kr;
  }
  return hip_status(hswa::launch_select_tokens(a, s), "token selection launch");
}

hswa_status_t sparse_sink_attn(const void* q, const void* k, const void* v, const int* sel_idx,
                               const int* sel_count, int max_sel, int recent_window,
                               const float* sink, void* o, int batch, int seqlen, int hq,
                               int hkv, int d_qk, int d_v, float scale, float rope_theta,
                               float rotary_fraction, long long pos_offset, hswa_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_impl(q, k, v, false, nullptr, nullptr, sel_idx, sel_count, max_sel, recent_window,
                     sink, o, batch, seqlen, hq, hkv, d_qk, d_v, scale, rope_theta,
                     rotary_fraction, pos_offset, dtype, workspace, workspace_bytes, stream);
}

hswa_status_t sparse_sink_attn_fp8(const void* q, const void* k, const void* v,
                                   const float* k_scale, const float* v_scale, const int* sel_idx,
                                   const int* sel_count, int max_sel, int recent_window,
                                   const float* sink, void* o, int batch, int seqlen, int hq,
                                   int hkv, int d_qk, int d_v, float scale, float rope_theta,
                                   float rotary_fraction, long long pos_offset,
                                   hswa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return sparse_impl(q, k, v, true, k_scale, v_scale, sel_idx, sel_count, max_sel, recent_window,
                     sink, o, batch, seqlen, hq, hkv, d_qk, d_v, scale, rope_theta,
                     rotary_fraction, pos_offset, dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
