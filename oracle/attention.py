"""Plain float64 definition of sink attention, its GA sibling, decode and sparse form.

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the CPU-baseline
leg of the benchmark; never by the product path.

Notation follows "MiMo-V2-Flash: Hybrid Sliding Window Attention Architecture"
(rslog.cc).  Indices here are 0-based; the page counts from 1.  For query row
i of head h with key set J_i:

    a_ij = q~_i . k~_j * scale                       (section 1.2 / 2.3)
    m_i  = max(max_{j in J_i} a_ij, sink_h)          (section 4.4)
    s_ij = exp(a_ij - m_i) / (exp(sink_h - m_i) + sum_{j' in J_i} exp(a_ij' - m_i))
    o_i  = sum_{j in J_i} s_ij v_j                   (section 4.4, final output)

sink_h = -inf means "no sink" (section 4.3 table: the -inf limit is the
ordinary softmax; section 5: GA layers have no sink term).  q~ and k~ carry
partial RoPE (pwwt.cn article, section 5); V is never rotated.

Each query row is evaluated on its own with a two-pass sum: first the max,
then the exponentials, the denominator and the weighted sum of values.  No
online rescaling, no tiling: library matrix products are the only steps
borrowed.
"""

import math

import numpy as np

NEG_INF = float("-inf")


# ----------------------------------------------------------------------------
# Partial rotary position embedding
# ----------------------------------------------------------------------------

def rotary_dims(d_qk, rotary_fraction):
    """Number of rotated dims R: the largest even integer <= fraction * d_qk.

    The pwwt.cn article (section 5) gives partial_rotary_factor 0.334 and
    head_dim 192: 0.334 * 192 = 64.13, so R = 64, i.e. about a third of the
    dims rotate.  Reading: the rotated dims are the first R.
    """
    if not (0.0 <= rotary_fraction <= 1.0):
        raise ValueError("rotary_fraction must lie in [0, 1]")
    return 2 * int(math.floor(rotary_fraction * d_qk / 2.0))


def rope(x, pos, theta, rotary_fraction):
    """Rotate the first R dims of x by position.

    x: float64 array [..., n, H, d]; pos: n integer positions.
    Pairing reading (the pages are silent): dim r pairs with dim r + R/2 for
    r < R/2, angle pos * theta^(-2r/R).  Written here as one complex product
    per pair: (x_r + i x_{r+R/2}) * exp(i * angle).  Dims >= R are untouched.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    rot = rotary_dims(d, rotary_fraction)
    out = x.copy()
    if rot == 0:
        return out
    half = rot // 2
    r = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(theta), -(2.0 * r) / rot)
    angle = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]  # [n, half]
    turn = np.exp(1j * angle)[:, None, :]                                    # [n, 1, half]
    z = (x[..., :half] + 1j * x[..., half:rot]) * turn
    out[..., :half] = z.real
    out[..., half:rot] = z.imag
    return out


# ----------------------------------------------------------------------------
# Key sets J_i
# ----------------------------------------------------------------------------

def window_keys(i, window):
    """Causal window of query i (0-based): keys max(0, i-W+1) .. i inclusive.

    rslog.cc section 2.1 defines W(i) = {j : max(1, i-W+1) <= j <= i} on
    1-based indices: W tokens including the query itself.  window None or
    <= 0 means the full causal set 0 .. i (section 1, the GA layer).
    """
    lo = 0 if (window is None or window <= 0) else max(0, i - window + 1)
    return np.arange(lo, i + 1, dtype=np.int64)


def ring_slot_positions(p, window):
    """Positions held by the W slots of a ring cache when the newest token is p.

    Slot s holds the token at position p - ((p - s) mod W), i.e. the cache
    writes token t into slot t mod W (youngju.dev article: the SWA pool is
    bounded by the window).  A negative entry marks a slot that has not been
    written yet (p < W - 1).
    """
    s = np.arange(window, dtype=np.int64)
    return p - np.mod(p - s, window)


def sparse_keys(i, selected, count, recent):
    """Key set of token-level sparse attention for query i.

    aideepthink.cn article, section 4: the most recent `recent` tokens
    (including i) plus the selected tokens outside that window, merged into
    one attention.  Set union of the two parts.
    """
    lo = max(0, i - recent + 1)
    rec = np.arange(lo, i + 1, dtype=np.int64)
    sel = np.asarray(selected[:count], dtype=np.int64)
    return np.union1d(sel, rec)


# ----------------------------------------------------------------------------
# One query row
# ----------------------------------------------------------------------------

def attend_row(qg, kj, vj, sink, scale):
    """Sink softmax attention of G query heads against one key set.

    qg: [G, d] (already rotated), kj: [m, d] (rotated), vj: [m, dv],
    sink: [G] (use -inf for no sink).  Returns [G, dv].
    Two passes, as rslog.cc section 4.4 writes it: m first, then the sums.
    """
    qg = np.asarray(qg, dtype=np.float64)
    kj = np.asarray(kj, dtype=np.float64)
    vj = np.asarray(vj, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64).reshape(-1)
    G = qg.shape[0]
    dv = vj.shape[-1]
    if kj.shape[0] == 0:
        # No key at all: only the sink is in the denominator, nothing in the
        # numerator.  With no sink either the row is undefined; return 0.
        return np.zeros((G, dv), dtype=np.float64)
    a = (qg @ kj.T) * scale                       # [G, m]   a_ij
    m = np.maximum(a.max(axis=1), sink)           # m_i
    out = np.zeros((G, dv), dtype=np.float64)
    for g in range(G):
        if m[g] == NEG_INF:
            continue
        e = np.exp(a[g] - m[g])                   # exp(a_ij - m_i)
        den = math.exp(sink[g] - m[g]) if sink[g] != NEG_INF else 0.0
        den += e.sum()
        out[g] = (e @ vj) / den                   # sum_j s_ij v_j
    return out


def _sink_vector(sink, hq):
    if sink is None:
        return np.full(hq, NEG_INF)
    s = np.asarray(sink, dtype=np.float64).reshape(-1)
    if s.shape[0] != hq:
        raise ValueError("sink must hold one value per query head")
    return s


def _check_heads(hq, hkv):
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    return hq // hkv


# ----------------------------------------------------------------------------
# Prefill (SWA with sink, and the GA sibling)
# ----------------------------------------------------------------------------

def prefill_rows(q, k, v, rows, sink=None, window=128, scale=None,
                 rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0, q_rows=None):
    """Prefill outputs for the query rows listed in `rows` only.

    q: [B, n, Hq, d_qk], k: [B, n, Hkv, d_qk], v: [B, n, Hkv, d_v].
    Token i sits at RoPE position pos_offset + i.  Query head h reads kv head
    h // (Hq/Hkv) (reading: contiguous GQA groups).  Returns [B, len(rows), Hq, d_v].
    q_rows, when given, is q[:, rows] already (q itself may then be None).
    """
    k = np.asarray(k)
    v = np.asarray(v)
    rows = np.asarray(rows, dtype=np.int64)
    q_sel = np.asarray(q_rows) if q_rows is not None else np.asarray(q)[:, rows]
    B, _, hq, d = q_sel.shape
    n = k.shape[1]
    hkv = k.shape[2]
    G = _check_heads(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_all = _sink_vector(sink, hq)
    qr = rope(q_sel, pos_offset + rows, rope_theta, rotary_fraction)
    kr = rope(k, pos_offset + np.arange(n), rope_theta, rotary_fraction)
    vv = np.asarray(v, dtype=np.float64)
    out = np.zeros((B, len(rows), hq, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for t, i in enumerate(rows):
            J = window_keys(int(i), window)
            for g in range(hkv):
                hs = slice(g * G, (g + 1) * G)
                out[b, t, hs] = attend_row(qr[b, t, hs], kr[b, J, g], vv[b, J, g],
                                           s_all[hs], scale)
    return out


def swa_sink_prefill(q, k, v, sink, window=128, scale=None, rope_theta=10000.0,
                     rotary_fraction=0.0, pos_offset=0):
    """SWA layer with a learnable sink (rslog.cc section 4.4): every row."""
    n = np.asarray(q).shape[1]
    return prefill_rows(q, k, v, np.arange(n), sink=sink, window=window, scale=scale,
                        rope_theta=rope_theta, rotary_fraction=rotary_fraction,
                        pos_offset=pos_offset)


def swa_sink_prefill_chunk(q, k, v, sink, window=128, scale=None, rope_theta=10000.0,
                           rotary_fraction=0.0, pos_offset=0):
    """Chunked prefill ("MiMo v2.5 inference optimisation" (youngju.dev),
    section on KV-cache restructuring and scheduling: long prefills run in
    fixed-size chunks behind the tokens already cached).

    q: [B, q_len, Hq, d_qk], the last q_len tokens; k, v: [B, kv_len, ...],
    the cached prefix followed by the chunk.  Query token t sits at sequence
    position kv_len - q_len + t and attends exactly as that row of the whole
    prefill does (window=0 or None with sink=None: the GA layer).
    """
    q = np.asarray(q)
    q_len, n = q.shape[1], np.asarray(k).shape[1]
    if q_len > n:
        raise ValueError("a chunk cannot be longer than its sequence")
    rows = n - q_len + np.arange(q_len)
    return prefill_rows(None, k, v, rows, sink=sink, window=window, scale=scale,
                        rope_theta=rope_theta, rotary_fraction=rotary_fraction,
                        pos_offset=pos_offset, q_rows=q)


def swa_sink_prefill_chunk_cached(q, k_cached, v, sink, window=128, scale=None,
                                  rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0):
    """swa_sink_prefill_chunk over a cache whose keys are stored already
    rotated (the decode caches' convention, written by kv_append): the
    chunk's queries are rotated at their positions, the keys are used as
    they are.  k_cached: [B, kv_len, Hkv, d_qk] rotated keys (prefix and
    chunk, the chunk's appended first)."""
    q = np.asarray(q)
    k_cached = np.asarray(k_cached, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, q_len, hq, d = q.shape
    n, hkv = k_cached.shape[1], k_cached.shape[2]
    if q_len > n:
        raise ValueError("a chunk cannot be longer than its sequence")
    G = _check_heads(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_all = _sink_vector(sink, hq)
    rows = n - q_len + np.arange(q_len)
    qr = rope(q, pos_offset + rows, rope_theta, rotary_fraction)
    out = np.zeros((B, q_len, hq, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for t, i in enumerate(rows):
            J = window_keys(int(i), window)
            for g in range(hkv):
                hs = slice(g * G, (g + 1) * G)
                out[b, t, hs] = attend_row(qr[b, t, hs], k_cached[b, J, g], v[b, J, g], s_all[hs],
                                           scale)
    return out


def ga_prefill(q, k, v, scale=None, rope_theta=1.0e7, rotary_fraction=0.0, pos_offset=0):
    """GA layer (rslog.cc section 1 and section 5): full causal set, no sink."""
    n = np.asarray(q).shape[1]
    return prefill_rows(q, k, v, np.arange(n), sink=None, window=None, scale=scale,
                        rope_theta=rope_theta, rotary_fraction=rotary_fraction,
                        pos_offset=pos_offset)


# ----------------------------------------------------------------------------
# Decode: one new token per sequence
# ----------------------------------------------------------------------------

def swa_sink_decode_ring(q, k_ring, v_ring, pos, sink, scale=None, rope_theta=10000.0,
                         rotary_fraction=0.0, seqs=None):
    """Decode against a W-slot ring cache.

    q: [B, Hq, d_qk] (RoPE at position pos[b] is applied here; the cache is
    taken to hold keys already rotated when they were written);
    k_ring: [B, W, Hkv, d_qk], v_ring: [B, W, Hkv, d_v], pos: [B] >= 0.
    The key set is every written slot (ring_slot_positions >= 0); the token
    at pos[b] itself is in the cache (the window includes the query).
    `seqs` restricts the evaluation to some sequences; returns [len(seqs), Hq, d_v].
    """
    q = np.asarray(q)
    B, hq, d = q.shape
    W = k_ring.shape[1]
    hkv = k_ring.shape[2]
    G = _check_heads(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_all = _sink_vector(sink, hq)
    seqs = np.arange(B) if seqs is None else np.asarray(seqs, dtype=np.int64)
    out = np.zeros((len(seqs), hq, v_ring.shape[-1]), dtype=np.float64)
    for t, b in enumerate(seqs):
        p = int(pos[b])
        qb = rope(q[b][None], np.array([p]), rope_theta, rotary_fraction)[0]
        slots = np.nonzero(ring_slot_positions(p, W) >= 0)[0]
        kb = np.asarray(k_ring[b], dtype=np.float64)
        vb = np.asarray(v_ring[b], dtype=np.float64)
        for g in range(hkv):
            hs = slice(g * G, (g + 1) * G)
            out[t, hs] = attend_row(qb[hs], kb[slots, g], vb[slots, g], s_all[hs], scale)
    return out


def swa_sink_decode_contiguous(q, k, v, seq_offsets, pos, sink=None, window=None,
                               scale=None, rope_theta=1.0e7, rotary_fraction=0.0,
                               seqs=None, kv_loader=None):
    """Decode against a contiguous per-sequence cache (the O(N) pool).

    k: [sum_b len_b, Hkv, d_qk], v: [sum_b len_b, Hkv, d_v]; sequence b owns
    rows seq_offsets[b] .. seq_offsets[b+1]-1 and its query sits at pos[b].
    Keys are rows seq_offsets[b] + window_keys(pos[b], window): the full
    prefix when window is None (GA layer, no sink), the last W otherwise.
    `kv_loader(b)` may supply (k_b, v_b) for one sequence instead of k, v, so
    that a cache too large for host memory is read one sequence at a time.
    """
    q = np.asarray(q)
    B, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_all = _sink_vector(sink, hq)
    seqs = np.arange(B) if seqs is None else np.asarray(seqs, dtype=np.int64)
    out = None
    for t, b in enumerate(seqs):
        p = int(pos[b])
        if kv_loader is not None:
            kb, vb = kv_loader(int(b))
        else:
            lo, hi = int(seq_offsets[b]), int(seq_offsets[b + 1])
            kb, vb = k[lo:hi], v[lo:hi]
        if p >= kb.shape[0]:
            raise ValueError("pos[b] must index a row inside sequence b's cache")
        hkv = kb.shape[1]
        G = _check_heads(hq, hkv)
        if out is None:
            out = np.zeros((len(seqs), hq, vb.shape[-1]), dtype=np.float64)
        qb = rope(q[b][None], np.array([p]), rope_theta, rotary_fraction)[0]
        J = window_keys(p, window)
        kJ = np.asarray(kb[J], dtype=np.float64)
        vJ = np.asarray(vb[J], dtype=np.float64)
        for g in range(hkv):
            hs = slice(g * G, (g + 1) * G)
            out[t, hs] = attend_row(qb[hs], kJ[:, g], vJ[:, g], s_all[hs], scale)
    return out


# ----------------------------------------------------------------------------
# Multi-token decode: the last accepted token and its drafts (MTP verification)
# ----------------------------------------------------------------------------

def decode_multi_ring(q, k_ring, v_ring, pos, sink, window, scale=None, rope_theta=10000.0,
                      rotary_fraction=0.0):
    """One verification step of multi-token prediction against a ring cache.

    The MTP drafts are checked by the main model in one forward pass ("visual
    reading: MiMo MTP/SWA, not MLA" (syt-nju.github.io), MTP section: three
    draft tokens verified at almost no extra cost; youngju.dev, architecture
    section: the 3-layer MTP).  q: [B, T, Hq, d]: query t of sequence b is
    the token at position pos[b] + t (the last accepted one, then T - 1
    drafts); each attends causally, also among the drafts, to positions
    max(0, p - W + 1) .. p.  k_ring: [B, S, Hkv, d], v_ring: [B, S, Hkv, dv]
    hold token j in slot j mod S, written up to position pos[b] + T - 1.
    Reading: the ring needs S >= W + T - 1 slots, or the drafts would have
    overwritten keys the first queries still see; checked here.
    Returns [B, T, Hq, dv].
    """
    q = np.asarray(q)
    B, T, hq, d = q.shape
    S = k_ring.shape[1]
    hkv = k_ring.shape[2]
    G = _check_heads(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_all = _sink_vector(sink, hq)
    out = np.zeros((B, T, hq, v_ring.shape[-1]), dtype=np.float64)
    for b in range(B):
        newest = int(pos[b]) + T - 1
        held = ring_slot_positions(newest, S)
        kb = np.asarray(k_ring[b], dtype=np.float64)
        vb = np.asarray(v_ring[b], dtype=np.float64)
        for t in range(T):
            p = int(pos[b]) + t
            J = window_keys(p, window)
            slots = np.mod(J, S)
            if not np.array_equal(held[slots], J):
                raise ValueError("the ring no longer holds every key of query t: S < W + T - 1")
            qt = rope(q[b, t][None], np.array([p]), rope_theta, rotary_fraction)[0]
            for g in range(hkv):
                hs = slice(g * G, (g + 1) * G)
                out[b, t, hs] = attend_row(qt[hs], kb[slots, g], vb[slots, g], s_all[hs], scale)
    return out


def decode_multi_contiguous(q, k, v, seq_offsets, pos, sink=None, window=None, scale=None,
                            rope_theta=1.0e7, rotary_fraction=0.0):
    """decode_multi_ring's step against a contiguous per-sequence cache:
    sequence b owns rows seq_offsets[b] .. seq_offsets[b+1]-1, its token j is
    row seq_offsets[b] + j, and rows up to position pos[b] + T - 1 are
    written.  window None: the full causal prefix (a GA layer)."""
    q = np.asarray(q)
    B, T, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_all = _sink_vector(sink, hq)
    out = None
    for b in range(B):
        lo, hi = int(seq_offsets[b]), int(seq_offsets[b + 1])
        kb = np.asarray(k[lo:hi], dtype=np.float64)
        vb = np.asarray(v[lo:hi], dtype=np.float64)
        if int(pos[b]) + T - 1 >= kb.shape[0]:
            raise ValueError("every query position must index a row of its sequence")
        hkv = kb.shape[1]
        G = _check_heads(hq, hkv)
        if out is None:
            out = np.zeros((B, T, hq, vb.shape[-1]), dtype=np.float64)
        for t in range(T):
            p = int(pos[b]) + t
            J = window_keys(p, window)
            qt = rope(q[b, t][None], np.array([p]), rope_theta, rotary_fraction)[0]
            for g in range(hkv):
                hs = slice(g * G, (g + 1) * G)
                out[b, t, hs] = attend_row(qt[hs], kb[J, g], vb[J, g], s_all[hs], scale)
    return out


# ----------------------------------------------------------------------------
# FP8 KV cache: E4M3 codes with one scale per kv head
# ----------------------------------------------------------------------------

def e4m3_value(codes):
    """Value of FP8 E4M3 codes (uint8), in float64.

    The pages store the KV cache in "FP8" (youngju.dev "MiMo v2.5 inference
    optimisation", closing section; aideepthink.cn "MiMo-V3 HySparse2",
    section 5) without naming the encoding.  Reading: the OCP E4M3 format:
    sign bit 7, exponent e in bits 6-3 with bias 7, mantissa m in bits 2-0;
    e > 0 is (1 + m/8) * 2^(e-7), e = 0 is the subnormal m * 2^-9; there are
    no infinities and exponent 15 with mantissa 7 is NaN.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def dequantise_kv(codes, scale):
    """Cache values from codes [..., Hkv, d] and per-kv-head scales [Hkv]."""
    return e4m3_value(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def swa_sink_decode_ring_fp8(q, k_codes, v_codes, k_scale, v_scale, pos, sink, scale=None,
                             rope_theta=10000.0, rotary_fraction=0.0, seqs=None):
    """Ring-cache decode over E4M3 caches: the ring decode on the cache values."""
    return swa_sink_decode_ring(q, dequantise_kv(k_codes, k_scale),
                                dequantise_kv(v_codes, v_scale), pos, sink, scale=scale,
                                rope_theta=rope_theta, rotary_fraction=rotary_fraction,
                                seqs=seqs)


def swa_sink_decode_contiguous_fp8(q, k_codes, v_codes, k_scale, v_scale, seq_offsets, pos,
                                   sink=None, window=None, scale=None, rope_theta=1.0e7,
                                   rotary_fraction=0.0, seqs=None, kv_loader=None):
    """Contiguous-cache decode over E4M3 caches.  `kv_loader(b)`, if given,
    returns the codes (k_b, v_b) of one sequence."""
    loader = None
    if kv_loader is not None:
        def loader(b):
            kb, vb = kv_loader(b)
            return dequantise_kv(kb, k_scale), dequantise_kv(vb, v_scale)
        k = v = None
    else:
        k, v = dequantise_kv(k_codes, k_scale), dequantise_kv(v_codes, v_scale)
    return swa_sink_decode_contiguous(q, k, v, seq_offsets, pos, sink=sink, window=window,
                                      scale=scale, rope_theta=rope_theta,
                                      rotary_fraction=rotary_fraction, seqs=seqs,
                                      kv_loader=loader)


# ----------------------------------------------------------------------------
# Token-level sparse attention on one shared cache
# ----------------------------------------------------------------------------

def sparse_rows(q, k, v, sel_idx, sel_count, rows, sink, recent=128, scale=None,
                rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0, restricted=False):
    """Sparse attention outputs for the query rows listed in `rows`.

    q: [B, n, Hq, d_qk]; k: [B, n, Hkv, d_qk]; v: [B, n, Hkv, d_v];
    sel_idx: [B, n, Hkv, max_sel] int; sel_count: [B, n, Hkv] int.
    Query i of kv group g attends to sparse_keys(i, sel_idx[b,i,g], count, recent).
    With restricted=True, q, sel_idx and sel_count hold only the listed rows
    (their second axis runs over `rows`).
    """
    rows = np.asarray(rows, dtype=np.int64)
    q_sel = np.asarray(q) if restricted else np.asarray(q)[:, rows]
    if not restricted:
        sel_idx = np.asarray(sel_idx)[:, rows]
        sel_count = np.asarray(sel_count)[:, rows]
    B, _, hq, d = q_sel.shape
    n = k.shape[1]
    hkv = k.shape[2]
    G = _check_heads(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_all = _sink_vector(sink, hq)
    qr = rope(q_sel, pos_offset + rows, rope_theta, rotary_fraction)
    kr = rope(k, pos_offset + np.arange(n), rope_theta, rotary_fraction)
    vv = np.asarray(v, dtype=np.float64)
    out = np.zeros((B, len(rows), hq, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for t, i in enumerate(rows):
            for g in range(hkv):
                J = sparse_keys(int(i), sel_idx[b, t, g], int(sel_count[b, t, g]), recent)
                hs = slice(g * G, (g + 1) * G)
                out[b, t, hs] = attend_row(qr[b, t, hs], kr[b, J, g], vv[b, J, g],
                                           s_all[hs], scale)
    return out


def sparse_sink_attn(q, k, v, sel_idx, sel_count, sink, recent=128, scale=None,
                     rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0):
    """Every row of token-level sparse attention with a sink."""
    n = np.asarray(q).shape[1]
    return sparse_rows(q, k, v, sel_idx, sel_count, np.arange(n), sink, recent=recent,
                       scale=scale, rope_theta=rope_theta, rotary_fraction=rotary_fraction,
                       pos_offset=pos_offset)


def sparse_rows_fp8(q, k_codes, v_codes, k_scale, v_scale, sel_idx, sel_count, rows, sink,
                    recent=128, scale=None, rope_theta=10000.0, rotary_fraction=0.0,
                    pos_offset=0, restricted=False):
    """Sparse attention over E4M3 K/V codes: sparse_rows on the cache values
    (RoPE rotates those values)."""
    return sparse_rows(q, dequantise_kv(k_codes, k_scale), dequantise_kv(v_codes, v_scale),
                       sel_idx, sel_count, rows, sink, recent=recent, scale=scale,
                       rope_theta=rope_theta, rotary_fraction=rotary_fraction,
                       pos_offset=pos_offset, restricted=restricted)


# ----------------------------------------------------------------------------
# Appending new tokens' keys and values to a decode cache
# ----------------------------------------------------------------------------

def e4m3_encode(x):
    """E4M3 code (uint8) nearest to each value of x: ties go to the code with
    an even mantissa, magnitudes of 448 and above saturate to 448 (reading:
    a saturating cast, so that no finite value becomes NaN), the sign is
    kept (a negative value that rounds to zero gives the negative-zero code).
    By search over the 127 finite non-negative values of e4m3_value."""
    x = np.asarray(x, dtype=np.float64)
    finite = e4m3_value(np.arange(127, dtype=np.uint8))          # codes 0x00 .. 0x7E, ascending
    a = np.abs(x)
    hi = np.clip(np.searchsorted(finite, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - finite[lo]
    d_hi = finite[hi] - a
    pick = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(a >= 448.0, 126, pick)
    return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def rope_f32_steps(x, pos, theta, rotary_fraction):
    """The partial RoPE of `rope`, evaluated in float32 the way a quantised
    cache entry is decided: cos and sin of the float64 angle rounded to
    float32, then each product and the difference / sum rounded to float32
    on its own.  x: [..., n, H, d] float32; pos: n positions."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    rot = rotary_dims(d, rotary_fraction)
    out = x.copy()
    if rot == 0:
        return out
    half = rot // 2
    r = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta ** (-(2.0 * r) / rot)   # [n, half]
    c = np.cos(ang).astype(np.float32)[:, None, :]
    sn = np.sin(ang).astype(np.float32)[:, None, :]
    x0, x1 = x[..., :half], x[..., half:rot]
    out[..., :half] = (x0 * c) - (x1 * sn)
    out[..., half:rot] = (x1 * c) + (x0 * sn)
    return out


def kv_append(k_cache, v_cache, k_new, v_new, pos, rope_theta, rotary_fraction, ring_slots=None,
              seq_offsets=None, k_scale=None, v_scale=None, store="same"):
    """Caches after writing T new tokens per sequence.

    k_new [B, T, Hkv, d_qk], v_new [B, T, Hkv, d_v] (float32 values); token t of
    sequence b is position pos[b] + t.  Ring (ring_slots = S): cache
    [B, S, Hkv, d], position j in slot j mod S (youngju.dev: the SWA pool is
    bounded by the window).  Contiguous (seq_offsets): row seq_offsets[b] + j.
    Keys are stored rotated (rope_f32_steps); store = "bf16" rounds to
    bfloat16 (to nearest even), "f32" keeps float32, "e4m3" stores
    e4m3_encode(value / scale[g]) with the quotient rounded to float32.
    Returns new (k_cache, v_cache) arrays; the inputs are not modified.
    """
    import torch
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    k_new = np.asarray(k_new, dtype=np.float32)
    v_new = np.asarray(v_new, dtype=np.float32)
    B, T = k_new.shape[:2]
    for b in range(B):
        ps = int(pos[b]) + np.arange(T)
        kr = rope_f32_steps(k_new[b], ps, rope_theta, rotary_fraction)          # [T, Hkv, d]
        vr = v_new[b]
        if ring_slots is not None:
            rows = (b, np.mod(ps, ring_slots))
        else:
            rows = (int(seq_offsets[b]) + ps,)
        if store == "e4m3":
            ks = np.asarray(k_scale, dtype=np.float32)[:, None]
            vs = np.asarray(v_scale, dtype=np.float32)[:, None]
            kc[rows] = e4m3_encode((kr / ks).astype(np.float32))
            vc[rows] = e4m3_encode((vr / vs).astype(np.float32))
        elif store == "bf16":
            kc[rows] = torch.from_numpy(kr).to(torch.bfloat16).float().numpy()
            vc[rows] = torch.from_numpy(vr).to(torch.bfloat16).float().numpy()
        else:
            kc[rows] = kr
            vc[rows] = vr
    return kc, vc


# ----------------------------------------------------------------------------
# Token selection for the sparse layers (HySparse2)
# ----------------------------------------------------------------------------

def selection_importance(q, k, b, i, g, recent, scale=None, rope_theta=1.0e7,
                         rotary_fraction=0.0, pos_offset=0):
    """Importance of every candidate token for query i, kv head g of sequence b.

    "MiMo-V3 HySparse2" (aideepthink.cn), section 4: the sparse layers reuse
    the token-selection indices of the preceding full-attention layer, with
    no separately trained retrieval module.  Reading: the importance of token
    j is the attention the full-attention layer gives it, summed over the
    group's query heads: I_j = sum_{h in g} exp(a_hij - lse_hi), the softmax
    over the full causal set 0 .. i (no sink: a GA layer).  Candidates are
    the tokens outside the recent window, 0 .. i - recent.
    Returns the float64 importances of tokens 0 .. i - recent (may be empty).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    hq, d = q.shape[2], q.shape[3]
    hkv = k.shape[2]
    G = _check_heads(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    last = i - recent
    if last < 0:
        return np.zeros(0)
    qi = rope(q[b, i][None], np.array([pos_offset + i]), rope_theta, rotary_fraction)[0]
    kr = rope(k[b, :i + 1], pos_offset + np.arange(i + 1), rope_theta, rotary_fraction)
    imp = np.zeros(last + 1)
    for h in range(g * G, (g + 1) * G):
        a = (kr[:, g] @ qi[h]) * scale                       # a_hij, j = 0 .. i
        m = a.max()
        lse = m + math.log(np.exp(a - m).sum())
        imp += np.exp(a[:last + 1] - lse)
    return imp


def select_tokens(q, k, rows, recent, max_sel, scale=None, rope_theta=1.0e7,
                  rotary_fraction=0.0, pos_offset=0):
    """Selected-token lists of the query rows listed in `rows`.

    For each (b, i, g): the min(max_sel, i - recent + 1) candidates of
    selection_importance with the largest importance, equal importances
    going to the lower position, listed in ascending order and padded with
    -1.  Returns idx int32 [B, len(rows), Hkv, max_sel] and count int32
    [B, len(rows), Hkv] (the layout sparse attention reads).
    """
    B, hkv = np.asarray(q).shape[0], np.asarray(k).shape[2]
    rows = np.asarray(rows, dtype=np.int64)
    idx = np.full((B, len(rows), hkv, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, len(rows), hkv), dtype=np.int32)
    for b in range(B):
        for t, i in enumerate(rows):
            for g in range(hkv):
                imp = selection_importance(q, k, b, int(i), g, recent, scale, rope_theta,
                                           rotary_fraction, pos_offset)
                take = min(max_sel, imp.size)
                order = np.lexsort((np.arange(imp.size), -imp))    # importance desc, then position
                chosen = np.sort(order[:take])
                idx[b, t, g, :take] = chosen
                cnt[b, t, g] = take
    return idx, cnt
