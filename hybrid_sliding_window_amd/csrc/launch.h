// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hswa {

// Which key set a query row reads.
enum Mode { MODE_PREFILL = 0, MODE_SPARSE = 1, MODE_DECODE_RING = 2, MODE_DECODE_CONTIG = 3 };

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sink;              // [hq] or null
  void* o;
  const int* sel_idx;             // sparse: [B, n, hkv, max_sel]
  const int* sel_count;           // sparse: [B, n, hkv]
  const long long* seq_offsets;   // decode contiguous: [B + 1]
  const long long* pos;           // decode: [B]
  const float2* rope;             // prefill / sparse: cos/sin table [n][half]
  const void* krot;               // prefill / sparse bf16: K's first R dims, rotated [B, n, hkv, R]
  void* qrot;                     // decode bf16: q rotated to pos[b] [B, hq, d_qk] (workspace)
  int* sel_out;                   // token selection: lists [B, n, hkv, max_sel]
  int* cnt_out;                   // and counts [B, n, hkv]
  unsigned* sel_ws;               // token selection: importance scratch (select_scratch_bytes)
  float* sel_lse;                 // token selection: log2-sum-exp2 per (b, i, query head)
  void* kout;                     // cache append: the K and V caches written
  void* vout;
  const float* kscale;            // decode FP8 caches: per-kv-head value of one K code unit [hkv]
  const float* vscale;            // the same for V
  int B, n, hq, hkv, d_qk, d_v;   // n: tokens of K/V (and q unless chunked)
  int nq;                         // prefill: query tokens per sequence (n unless chunked);
                                  // multi-token decode: queries per sequence
  int slots;                      // multi-token decode, ring cache: slot count S
  int qoff;                       // prefill: sequence position of query token 0 (n - nq)
  int window;                     // prefill: 0 = full causal; decode: ring size or window
  int k_rotated;                  // prefill: K rows are stored already rotated (a cache)
  int half;                       // R / 2 (0 = no RoPE)
  int max_sel, recent;            // sparse
  float scale;                    // factor on q.k (natural-log units)
  double rope_theta;
  long long pos_offset;           // RoPE position of token 0 (prefill / sparse)
  long long max_pos;              // decode: host bound on pos[b]
  float* ws;                      // decode: split partials
  int split_keys, nsplit;         // decode: keys per split, splits per (b, kv head)
};

// cos/sin table: table[t][r] = (cos, sin)((pos0 + t) * theta^(-r/half)).
hipError_t launch_rope_table(float2* table, long long pos0, int npos, int half, double theta,
                             hipStream_t stream);

// krot[row][0:R] = RoPE of k[row][0:R] (bf16) for the rows [B, n, hkv] of
// tokens first..n-1 (token (row / hkv) % n); other rows are not written.
hipError_t launch_rope_k(const uint16_t* k, const float2* table, uint16_t* krot, int B, int n,
                         int first, int hkv, int d, int half, hipStream_t stream);

// The same for K stored as E4M3 codes (krot = bf16 rotation of the codes'
// values, no scale applied).
hipError_t launch_rope_k_e4m3(const uint8_t* k, const float2* table, uint16_t* krot, int B, int n,
                              int first, int hkv, int d, int half, hipStream_t stream);

// The same without a table: cos/sin evaluated per element (fp64 angle in
// revolutions, reduced, hardware sine/cosine).  Requires half <= 64.
hipError_t launch_rope_k_direct(const uint16_t* k, uint16_t* krot, int B, int n, int first,
                                int hkv, int d, int half, long long pos0, double theta,
                                hipStream_t stream);

// Any shape, any key set, fp32 or bf16 storage: one wavefront per query row.
// kv_fp8 (decode and sparse modes): K/V are E4M3 codes scaled by kscale / vscale.
hipError_t launch_generic(const AttnArgs& a, int mode, bool bf16, bool kv_fp8, hipStream_t stream);

// bf16 matrix-core kernels for d_qk = 192, d_v = 128.
bool prefill_bf16_supported(const AttnArgs& a);
hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream);

// Windowed layers (G >= 8, d 192 / 128, rotary half-width 0, 16 or 32, at
// most 256 q heads) with W + 2 * (256 / G) small enough for a 7-tile K/V
// ring (prefill_seq.hip).
bool prefill_seq_supported(const AttnArgs& a);
hipError_t launch_prefill_seq(const AttnArgs& a, hipStream_t stream);
// The same shapes for full causal layers and wider windows, one workgroup
// barrier per two key tiles (prefill_causal.hip).
bool prefill_causal_supported(const AttnArgs& a);
hipError_t launch_prefill_causal(const AttnArgs& a, hipStream_t stream);

bool decode_bf16_supported(const AttnArgs& a);
void decode_split_plan(int layout, int window, long long max_pos, int* split_keys, int* nsplit);
hipError_t launch_decode_bf16(const AttnArgs& a, int layout, hipStream_t stream);
// Rings of at most 128 slots (and head shapes the matrix-core decode takes)
// run in one launch, without split partials.
bool decode_ring_supported(const AttnArgs& a, int layout);
// The two kernels around a decode split kernel: q rotated to its position
// (no-op without RoPE) and the combine of the split partials with the sink.
hipError_t launch_decode_rope_q(const AttnArgs& a, int layout, hipStream_t stream);
hipError_t launch_decode_combine(const AttnArgs& a, int layout, hipStream_t stream);

// Multi-token decode (nq queries per sequence at pos[b] .. pos[b] + nq - 1):
// bf16 matrix-core kernels for d_qk = 192, d_v = 128, hkv % 4 == 0 and
// nq * G <= 64 (workspace as the single-token decode with B * nq rows), and
// a generic kernel for any shape, bf16 or fp32 (no workspace).
bool decode_multi_supported(const AttnArgs& a);
hipError_t launch_decode_multi(const AttnArgs& a, int layout, hipStream_t stream);
hipError_t launch_decode_multi_generic(const AttnArgs& a, int layout, bool bf16,
                                       hipStream_t stream);

// Append nq new tokens per sequence (k, v: [B, nq, hkv, d]) at positions
// pos[b] .. pos[b] + nq - 1 to a ring (slots) or contiguous cache (kout,
// vout): RoPE on K at each position, then a copy in the input type or E4M3
// codes of value / kscale[g] (vscale[g]).  d_qk, d_v and half multiples of 8.
hipError_t launch_kv_append(const AttnArgs& a, int layout, bool bf16_in, bool e4m3_out,
                            hipStream_t stream);

// Token selection (bf16, d_qk = 192, 16 query heads per kv head): for every
// (b, i, g) the max_sel candidates 0 .. i - recent of largest importance into
// sel_out / cnt_out.  With RoPE (half > 0) q and k are read from qrot / krot,
// full rotated rows [B, n, hq | hkv, 192] made by launch_rope_rows.
// A first kernel writes sel_lse [B, n, hq] (fp32, base 2) for the rows that
// rank their candidates; the selection kernel runs at most kSelectSlots
// workgroups, each looping over (row block, kv head) items; workgroup w keeps
// the importances of its current item's kSelectRows rows in slot w of sel_ws
// (kSelectRows rows of round64(n) words), then, after all slots, a list of
// kSelectListCap (position, key) pairs per row and slot.
constexpr int kSelectSlots = 256;
constexpr int kSelectRows = 32;
constexpr int kSelectListCap = 4096;
inline size_t select_scratch_bytes(int n) {
  return (size_t)kSelectSlots * kSelectRows *
         ((((size_t)n + 63) & ~(size_t)63) * 4 + (size_t)kSelectListCap * 8);
}
inline size_t select_lse_bytes(int B, int n, int hq) { return (size_t)B * n * hq * 4; }
bool select_tokens_supported(const AttnArgs& a);
hipError_t launch_select_tokens(const AttnArgs& a, hipStream_t stream);
// The first of the two: sel_lse for the rows that rank their candidates,
// on up to two workgroups per compute unit (cus of them).
hipError_t launch_select_lse(const AttnArgs& a, int cus, hipStream_t stream);

// dst[row] = src[row] with its first 2 * half dims rotated at position
// pos0 + (row / heads) % n (cos/sin as launch_rope_k_direct), the rest copied;
// rows = B * n * heads bf16 rows of d dims.  half <= 64.
hipError_t launch_rope_rows(const uint16_t* src, uint16_t* dst, int B, int n, int heads, int d,
                            int half, long long pos0, double theta, hipStream_t stream);

// Decode over E4M3 caches (same shapes as the bf16 decode kernel).
bool decode_fp8_supported(const AttnArgs& a);
hipError_t launch_decode_fp8(const AttnArgs& a, int layout, hipStream_t stream);

bool sparse_bf16_supported(const AttnArgs& a);
hipError_t launch_sparse_bf16(const AttnArgs& a, hipStream_t stream);
// The same over E4M3 K/V codes with per-kv-head scales (kscale, vscale);
// rotary half-widths 0 or 32.
bool sparse_fp8_supported(const AttnArgs& a);
hipError_t launch_sparse_fp8(const AttnArgs& a, hipStream_t stream);

// Records msg as the text of hswa_last_error() and returns status (api.cpp).
int api_fail(int status, const char* msg);

}  // namespace hswa
