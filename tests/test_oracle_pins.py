"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin checks the oracle against something other than itself: library
routines (torch SDPA in float64, scipy), closed forms, a scalar brute force
with a different RoPE formulation, and invariants the pages state.  The
mutant tests plant plausible mistakes in a copy of the oracle and require
that at least one pin catches each of them.

Pages: "MiMo-V2-Flash: Hybrid Sliding Window Attention Architecture"
(rslog.cc), "MiMo-V2.6-Flash hybrid SWA" (pwwt.cn), "MiMo-V3 HySparse2"
(aideepthink.cn), "MiMo v2.5 inference optimisation" (youngju.dev).
"""

import inspect
import json
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit, logsumexp

import oracle.attention as OA
import synthetic

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))
NEG_INF = float("-inf")


def _inputs(B, n, hq, hkv, d=192, dv=128, seed=0, sink=(-2.0, 2.0)):
    x = synthetic.prefill_inputs(B, n, hq, hkv, d, dv, "f32", seed, sink_range=sink)
    q, k, v = (x[t].double().numpy() for t in "qkv")
    s = None if x["sink"] is None else x["sink"].double().numpy()
    return q, k, v, s


# ---------------------------------------------------------------------------
# Independent references
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, allowed, sink, scale):
    """torch SDPA (float64) with a boolean key mask and the sink as an extra key.

    The sink becomes one appended key with zero vector and zero value whose
    additive mask is sink_h: its score is 0 + sink_h and it adds nothing to
    the output, which is exactly the extra denominator term of the sink
    softmax (rslog.cc section 4.2).  allowed: [B or 1, n_q, n_k] bool.
    """
    B, n, hq, d = q.shape
    G = hq // k.shape[2]
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    K = torch.from_numpy(np.repeat(k, G, axis=2)).permute(0, 2, 1, 3)
    V = torch.from_numpy(np.repeat(v, G, axis=2)).permute(0, 2, 1, 3)
    mask = torch.where(torch.from_numpy(allowed), 0.0, NEG_INF).double()[:, None]  # [B,1,nq,nk]
    mask = mask.expand(B, hq, *mask.shape[2:])
    if sink is not None:
        K = torch.cat([K, torch.zeros(B, hq, 1, d, dtype=torch.float64)], dim=2)
        V = torch.cat([V, torch.zeros(B, hq, 1, V.shape[-1], dtype=torch.float64)], dim=2)
        col = torch.from_numpy(np.asarray(sink, dtype=np.float64))[None, :, None, None]
        col = col.expand(B, hq, mask.shape[2], 1)
        mask = torch.cat([mask, col], dim=3)
    o = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _window_mask(n, W):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    ok = j <= i
    if W is not None:
        ok &= j >= i - W + 1
    return ok[None]


def _brute_rope(x, p, theta, R):
    """Real-arithmetic statement of the RoPE reading: pair (r, r+R/2)."""
    out = list(x)
    half = R // 2
    for r in range(half):
        ang = p * theta ** (-2.0 * r / R)
        c, s = math.cos(ang), math.sin(ang)
        out[r] = x[r] * c - x[r + half] * s
        out[r + half] = x[r + half] * c + x[r] * s
    return out


def _brute_prefill(q, k, v, sink, W, theta, frac):
    """Scalar loops with math.fsum: a third formulation of the definition."""
    B, n, hq, d = q.shape
    hkv = k.shape[2]
    G = hq // hkv
    R = 2 * int(math.floor(frac * d / 2))
    out = np.zeros((B, n, hq, v.shape[-1]))
    for b in range(B):
        kr = [[_brute_rope(list(k[b, j, g]), j, theta, R) for g in range(hkv)] for j in range(n)]
        for i in range(n):
            keys = [j for j in range(i + 1) if W is None or j >= i - W + 1]
            for h in range(hq):
                g = h // G
                qi = _brute_rope(list(q[b, i, h]), i, theta, R)
                a = {j: math.fsum(qi[t] * kr[j][g][t] for t in range(d)) / math.sqrt(d) for j in keys}
                sh = NEG_INF if sink is None else float(sink[h])
                m = max(max(a.values()), sh)
                terms = [math.exp(a[j] - m) for j in keys]
                den = math.fsum(terms + ([math.exp(sh - m)] if sh != NEG_INF else []))
                for c in range(v.shape[-1]):
                    out[b, i, h, c] = math.fsum(terms[t] * v[b, j, g, c] for t, j in enumerate(keys)) / den
    return out


# ---------------------------------------------------------------------------
# Pins.  Each takes the oracle module so that mutants can be run through them.
# ---------------------------------------------------------------------------

def pin_p1_no_sink_is_masked_softmax(O):
    """sink -> -inf gives the ordinary softmax over the window (rslog.cc 4.3)."""
    q, k, v, _ = _inputs(1, 40, 4, 2, seed=11)
    for W in (1, 5, 16):
        got = O.swa_sink_prefill(q, k, v, None, window=W)
        ref = _sdpa(q, k, v, _window_mask(40, W), None, 1 / math.sqrt(192))
        assert np.abs(got - ref).max() < 1e-12, W


def pin_p2_wide_window_is_causal(O):
    """W >= n with no sink is full causal attention (rslog.cc section 5, GA row)."""
    q, k, v, _ = _inputs(2, 24, 4, 1, seed=12)
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    K = torch.from_numpy(np.repeat(k, 4, axis=2)).permute(0, 2, 1, 3)
    V = torch.from_numpy(np.repeat(v, 4, axis=2)).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=1 / math.sqrt(192))
    ref = ref.permute(0, 2, 1, 3).numpy()
    for got in (O.swa_sink_prefill(q, k, v, None, window=24),
                O.swa_sink_prefill(q, k, v, None, window=1000),
                O.ga_prefill(q, k, v)):
        assert np.abs(got - ref).max() < 1e-12


def pin_p3_sink_as_extra_key(O):
    """The sink term equals one extra zero-valued key scored sink_h (rslog.cc 4.2, 4.4)."""
    q, k, v, s = _inputs(1, 36, 8, 2, seed=13)
    for W in (1, 3, 16, 36):
        got = O.swa_sink_prefill(q, k, v, s, window=W)
        ref = _sdpa(q, k, v, _window_mask(36, W), s, 1 / math.sqrt(192))
        assert np.abs(got - ref).max() < 1e-12, W


def pin_p4_weights_sum(O):
    """With V = 1 every output is the weight sum, exp(LSE)/(exp(sink)+exp(LSE)) < 1.

    rslog.cc section 4.2 (weights sum below one) and section 6 table (sum is
    exactly one without the sink).
    """
    q, k, v, s = _inputs(1, 30, 2, 1, seed=14)
    ones = np.ones_like(v)
    W = 7
    got = O.swa_sink_prefill(q, k, ones, s, window=W)
    got0 = O.swa_sink_prefill(q, k, ones, None, window=W)
    a = np.einsum("nhd,mhd->hnm", q[0], np.repeat(k[0], 2, axis=1)) / math.sqrt(192)
    for i in range(30):
        lo = max(0, i - W + 1)
        lse = logsumexp(a[:, i, lo:i + 1], axis=1)
        expect = expit(lse - s)       # = 1 / (1 + exp(sink - LSE))
        assert np.abs(got[0, i, :, :] - expect[:, None]).max() < 1e-13
        assert (got[0, i] < 1.0).all()
    assert np.abs(got0 - 1.0).max() < 1e-13


def pin_p5_unit_window(O):
    """W = 1: o_i = sigmoid(a_ii - sink) v_i, the logistic closed form."""
    q, k, v, s = _inputs(1, 12, 2, 2, seed=15)
    got = O.swa_sink_prefill(q, k, v, s, window=1)
    a = np.einsum("nhd,nhd->nh", q[0], k[0]) / math.sqrt(192)
    expect = expit(a - s[None, :])[:, :, None] * v[0]
    assert np.abs(got[0] - expect).max() < 1e-13


def pin_p6_zero_query(O):
    """q = 0: all scores vanish, o_i = sum_J v_j / (exp(sink) + |J_i|)."""
    _, k, v, s = _inputs(1, 20, 4, 2, seed=16)
    q = np.zeros((1, 20, 4, 192))
    for W in (4, 9):
        got = O.swa_sink_prefill(q, k, v, s, window=W, rope_theta=1e4, rotary_fraction=0.334)
        for i in range(20):
            lo = max(0, i - W + 1)
            cnt = i + 1 - lo
            for h in range(4):
                expect = v[0, lo:i + 1, h // 2].sum(axis=0) / (math.exp(s[h]) + cnt)
                assert np.abs(got[0, i, h] - expect).max() < 1e-13


def pin_p7_brute_force(O):
    """Every W <= n, G in {1, 2}, sinks {-inf, -1, 0, 2}, with and without RoPE."""
    rng = np.random.default_rng(17)
    n, d, dv = 6, 8, 4
    for G in (1, 2):
        q = rng.standard_normal((1, n, 2 * G, d)) * 1.5
        k = rng.standard_normal((1, n, 2, d)) * 1.5
        v = rng.standard_normal((1, n, 2, dv))
        for sv in (NEG_INF, -1.0, 0.0, 2.0):
            sink = None if sv == NEG_INF else np.full(2 * G, sv) + np.arange(2 * G) * 0.25
            for W in list(range(1, n + 1)) + [None]:
                for frac, theta in ((0.0, 1.0e4), (0.5, 3.0)):
                    got = (O.ga_prefill(q, k, v, rope_theta=theta, rotary_fraction=frac)
                           if (W is None and sink is None) else
                           O.swa_sink_prefill(q, k, v, sink, window=0 if W is None else W,
                                              rope_theta=theta, rotary_fraction=frac))
                    ref = _brute_prefill(q, k, v, sink, W, theta, frac)
                    assert np.abs(got - ref).max() < 1e-12, (G, sv, W, frac)


def pin_p8_rope(O):
    """RoPE reading: closed form on basis vectors, relative-position property,
    norm preservation, identity at fraction 0, R = 64 at 192 dims and 0.334."""
    assert O.rotary_dims(GOLD["d_qk"]["value"], GOLD["partial_rotary_factor"]["value"]) == \
        GOLD["rotated_dims_at_192"]["value"]
    d, frac, theta = 192, 0.334, 1.0e4
    R = 64
    half = R // 2
    pos = np.array([0, 1, 7, 1000, 262143])
    for r in (0, 1, 13, half - 1):
        e = np.zeros((len(pos), 1, d))
        e[:, 0, r] = 1.0
        out = O.rope(e, pos, theta, frac)
        ang = pos * theta ** (-2.0 * r / R)
        # the angle is pos * inv_freq; two pow() routines may differ by an ulp
        tol = 1e-12 + pos * 4e-16
        assert (np.abs(out[:, 0, r] - np.cos(ang)) < tol).all()
        assert (np.abs(out[:, 0, r + half] - np.sin(ang)) < tol).all()
        e2 = np.zeros((len(pos), 1, d))
        e2[:, 0, r + half] = 1.0
        out2 = O.rope(e2, pos, theta, frac)
        assert (np.abs(out2[:, 0, r] + np.sin(ang)) < tol).all()
        assert (np.abs(out2[:, 0, r + half] - np.cos(ang)) < tol).all()
        mask = np.ones(d, bool)
        mask[[r, r + half]] = False
        assert np.abs(out[:, 0, mask]).max() == 0.0
    rng = np.random.default_rng(18)
    x = rng.standard_normal((5, 3, d))
    y = rng.standard_normal((5, 3, d))
    p = np.array([3, 10, 50, 99, 4000])
    for delta in (1, 17, 100000):
        s0 = np.einsum("nhd,nhd->nh", O.rope(x, p, theta, frac), O.rope(y, p[::-1], theta, frac))
        s1 = np.einsum("nhd,nhd->nh", O.rope(x, p + delta, theta, frac),
                       O.rope(y, p[::-1] + delta, theta, frac))
        assert np.abs(s0 - s1).max() < 1e-9
    xr = O.rope(x, p, theta, frac)
    assert np.abs(np.linalg.norm(xr, axis=-1) - np.linalg.norm(x, axis=-1)).max() < 1e-12
    assert np.array_equal(xr[..., R:], x[..., R:])
    assert np.array_equal(O.rope(x, p, theta, 0.0), x)


def pin_p9_gqa(O):
    """Grouped heads equal multi-head attention with each kv head repeated G times."""
    q, k, v, s = _inputs(1, 20, 8, 2, seed=19)
    got = O.swa_sink_prefill(q, k, v, s, window=6, rope_theta=1e4, rotary_fraction=0.334)
    ref = O.swa_sink_prefill(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), s, window=6,
                             rope_theta=1e4, rotary_fraction=0.334)
    assert np.abs(got - ref).max() < 1e-13
    # and the grouping is contiguous: head h reads kv head h // G
    got1 = O.swa_sink_prefill(q[:, :, :4], k[:, :, :1], v[:, :, :1], s[:4], window=6,
                              rope_theta=1e4, rotary_fraction=0.334)
    assert np.abs(got[:, :, :4] - got1).max() < 1e-13


def pin_p10_decode_equals_prefill_row(O):
    """Decode at p over a cache filled from a sequence equals prefill row p.

    Ring cache: token t sits in slot t mod W (youngju.dev dual-pool cache);
    contiguous cache: rows 0..p.  Keys in the cache carry RoPE already.
    """
    rng = np.random.default_rng(20)
    W, hq, hkv, d, dv = 16, 4, 2, 192, 128
    theta, frac = 1.0e4, 0.334
    sink = rng.uniform(-2, 2, hq)
    for L in (40, 9):                                   # 9 < W - 1: ring warm-up
        q = rng.standard_normal((1, L, hq, d))
        k = rng.standard_normal((1, L, hkv, d))
        v = rng.standard_normal((1, L, hkv, dv))
        p = L - 1
        swa = O.swa_sink_prefill(q, k, v, sink, window=W, rope_theta=theta, rotary_fraction=frac)
        ga = O.ga_prefill(q, k, v, rope_theta=theta, rotary_fraction=frac)
        kr = O.rope(k[0], np.arange(L), theta, frac)
        ring_k = rng.standard_normal((1, W, hkv, d)) * 50.0     # stale junk in unwritten slots
        ring_v = rng.standard_normal((1, W, hkv, dv)) * 50.0
        for t in range(max(0, p - W + 1), p + 1):
            ring_k[0, t % W] = kr[t]
            ring_v[0, t % W] = v[0, t]
        got = O.swa_sink_decode_ring(q[:, p], ring_k, ring_v, np.array([p]), sink,
                                     rope_theta=theta, rotary_fraction=frac)
        assert np.abs(got[0] - swa[0, p]).max() < 1e-12
        offs = np.array([0, L + 3])
        kc = np.concatenate([kr, rng.standard_normal((3, hkv, d))])
        vc = np.concatenate([v[0], rng.standard_normal((3, hkv, dv))])
        got_ga = O.swa_sink_decode_contiguous(q[:, p], kc, vc, offs, np.array([p]), None, None,
                                              rope_theta=theta, rotary_fraction=frac)
        assert np.abs(got_ga[0] - ga[0, p]).max() < 1e-12
        got_sw = O.swa_sink_decode_contiguous(q[:, p], kc, vc, offs, np.array([p]), sink, W,
                                              rope_theta=theta, rotary_fraction=frac)
        assert np.abs(got_sw[0] - swa[0, p]).max() < 1e-12
        got_ld = O.swa_sink_decode_contiguous(q[:, p], None, None, offs, np.array([p]), None,
                                              None, rope_theta=theta, rotary_fraction=frac,
                                              kv_loader=lambda b: (kc, vc))
        assert np.abs(got_ld - got_ga).max() == 0.0


def _brute_sparse(q, k, v, sel_idx, sel_count, rows, sink, recent, theta, frac, off):
    """Scalar loops for token-level sparse attention: the key set of query i
    is the recent window plus its listed tokens, each vector rotated by
    _brute_rope at its own position off + index, sums with math.fsum."""
    B, n, hq, d = q.shape
    hkv = k.shape[2]
    G = hq // hkv
    R = 2 * int(math.floor(frac * d / 2))
    out = np.zeros((B, len(rows), hq, v.shape[-1]))
    for b in range(B):
        for t, i in enumerate(rows):
            i = int(i)
            for g in range(hkv):
                keys = set(range(max(0, i - recent + 1), i + 1))
                keys |= {int(j) for j in sel_idx[b, i, g, :sel_count[b, i, g]]}
                keys = sorted(keys)
                kr = {j: _brute_rope(list(k[b, j, g]), off + j, theta, R) for j in keys}
                for h in range(g * G, (g + 1) * G):
                    qi = _brute_rope(list(q[b, i, h]), off + i, theta, R)
                    a = {j: math.fsum(qi[c] * kr[j][c] for c in range(d)) / math.sqrt(d)
                         for j in keys}
                    sh = NEG_INF if sink is None else float(sink[h])
                    m = max(max(a.values()), sh)
                    terms = [math.exp(a[j] - m) for j in keys]
                    den = math.fsum(terms + ([math.exp(sh - m)] if sh != NEG_INF else []))
                    for c in range(v.shape[-1]):
                        out[b, t, h, c] = math.fsum(terms[u] * v[b, j, g, c]
                                                    for u, j in enumerate(keys)) / den
    return out


def pin_p11_sparse(O):
    """Sparse attention reductions (aideepthink.cn section 4).

    No selection: SWA with W = recent.  Complete selection: causal over
    [0, i] without i - recent.  General lists: SDPA with the lists as a mask.
    """
    recent, n, hq, hkv = 8, 40, 4, 2
    q, k, v, s = _inputs(1, n, hq, hkv, seed=21)
    idx, cnt = synthetic.sparse_selection(1, n, hkv, recent, 1024, 21)
    idx, cnt = idx.numpy(), cnt.numpy()
    got = O.sparse_sink_attn(q, k, v, idx, cnt, s, recent=recent)
    swa = O.swa_sink_prefill(q, k, v, s, window=recent)
    assert np.abs(got[:, :recent + 1] - swa[:, :recent + 1]).max() < 1e-12
    allowed = np.tril(np.ones((n, n), bool))
    for i in range(recent, n):
        allowed[i, i - recent] = False
    ref = _sdpa(q, k, v, allowed[None], s, 1 / math.sqrt(192))
    assert np.abs(got - ref).max() < 1e-12
    # sampled lists (max_sel < available)
    idx2, cnt2 = synthetic.sparse_selection(1, n, hkv, recent, 5, 22)
    idx2, cnt2 = idx2.numpy(), cnt2.numpy()
    got2 = O.sparse_sink_attn(q, k, v, idx2, cnt2, s, recent=recent)
    for g in range(hkv):
        al = np.zeros((n, n), bool)
        for i in range(n):
            al[i, max(0, i - recent + 1):i + 1] = True
            al[i, idx2[0, i, g, :cnt2[0, i, g]]] = True
        ref2 = _sdpa(q[:, :, g * 2:(g + 1) * 2], k[:, :, g:g + 1], v[:, :, g:g + 1], al[None],
                     s[g * 2:(g + 1) * 2], 1 / math.sqrt(192))
        assert np.abs(got2[:, :, g * 2:(g + 1) * 2] - ref2).max() < 1e-12
    # RoPE on, positions shifted by pos_offset, a subset of rows: against scalar
    # loops with the real-arithmetic rotation (every key at its own position)
    rng = np.random.default_rng(24)
    n, hq, hkv, d, dv, recent, off = 16, 4, 2, 8, 4, 3, 11
    q = rng.standard_normal((2, n, hq, d)) * 1.5
    k = rng.standard_normal((2, n, hkv, d)) * 1.5
    v = rng.standard_normal((2, n, hkv, dv))
    sink = np.array([-1.0, 0.5, 0.0, 2.0])
    idx3, cnt3 = synthetic.sparse_selection(2, n, hkv, recent, 4, 25)
    idx3, cnt3 = idx3.numpy(), cnt3.numpy()
    rows = np.array([0, 2, 5, 9, 15])
    for frac, theta in ((0.5, 3.0), (1.0, 7.0)):
        got3 = O.sparse_rows(q, k, v, idx3, cnt3, rows, sink, recent=recent, rope_theta=theta,
                             rotary_fraction=frac, pos_offset=off)
        ref3 = _brute_sparse(q, k, v, idx3, cnt3, rows, sink, recent, theta, frac, off)
        assert np.abs(got3 - ref3).max() < 1e-12, frac
        # the same rows handed over alone (restricted) give the same outputs
        got4 = O.sparse_rows(q[:, rows], k, v, idx3[:, rows], cnt3[:, rows], rows, sink,
                             recent=recent, rope_theta=theta, rotary_fraction=frac,
                             pos_offset=off, restricted=True)
        assert np.abs(got4 - ref3).max() < 1e-12, frac


def pin_p12_large_sink_is_stable(O):
    """The max includes the sink (rslog.cc 4.4): huge sinks give finite, tiny outputs."""
    q, k, v, _ = _inputs(1, 10, 2, 1, seed=23)
    s = np.array([800.0, -800.0])
    got = O.swa_sink_prefill(q, k, v, s, window=4)
    assert np.isfinite(got).all()
    assert np.abs(got[0, :, 0]).max() < 1e-300
    ref = O.swa_sink_prefill(q, k, v, None, window=4)
    assert np.abs(got[0, :, 1] - ref[0, :, 1]).max() < 1e-12


def pin_p13_chunk(O):
    """A chunk behind a cached prefix (youngju.dev, KV-cache restructuring and
    scheduling: fixed-size prefill chunks) gives the last rows of the whole
    prefill: against the scalar brute force (RoPE, sinks, G = 2) and torch SDPA
    with a rectangular window mask."""
    rng = np.random.default_rng(29)
    n, d, dv = 9, 8, 4
    q = rng.standard_normal((1, n, 4, d)) * 1.5
    k = rng.standard_normal((1, n, 2, d)) * 1.5
    v = rng.standard_normal((1, n, 2, dv))
    sink = np.array([-1.0, 0.0, 0.5, 2.0])
    for W in (1, 3, None):
        ref = _brute_prefill(q, k, v, sink, W, 3.0, 0.5)
        for ql in (1, 4, n):
            got = O.swa_sink_prefill_chunk(q[:, n - ql:], k, v, sink, window=0 if W is None else W,
                                           rope_theta=3.0, rotary_fraction=0.5)
            assert got.shape == (1, ql, 4, dv)
            assert np.abs(got - ref[:, n - ql:]).max() < 1e-12, (W, ql)
    # the same chunk over a cache holding the keys already rotated (fp64 here)
    kc = O.rope(k, np.arange(n), 3.0, 0.5)
    for W in (1, 3, None):
        ref = _brute_prefill(q, k, v, sink, W, 3.0, 0.5)
        got = O.swa_sink_prefill_chunk_cached(q[:, n - 4:], kc, v, sink, window=0 if W is None else W,
                                              rope_theta=3.0, rotary_fraction=0.5)
        assert np.abs(got - ref[:, n - 4:]).max() < 1e-12, W
    q, k, v, s = _inputs(2, 40, 8, 2, seed=31)
    ql = 13
    i = np.arange(40 - ql, 40)[:, None]
    j = np.arange(40)[None, :]
    for W in (5, 16):
        allowed = ((j <= i) & (j >= i - W + 1))[None]
        ref = _sdpa(q[:, 40 - ql:], k, v, allowed, s, 1 / math.sqrt(192))
        got = O.swa_sink_prefill_chunk(q[:, 40 - ql:], k, v, s, window=W)
        assert np.abs(got - ref).max() < 1e-12, W


def pin_p14_fp8_cache(O):
    """FP8 KV cache: the E4M3 value of every code against torch's
    float8_e4m3fn (a library routine), the format's landmark values, and
    the FP8 decodes against the plain decodes on caches torch dequantised."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    # largest finite, smallest subnormal, smallest normal, one, NaN, negative zero
    lm = O.e4m3_value(np.array([0x7E, 0x01, 0x08, 0x38, 0x7F, 0xFF, 0x80, 0xFE], dtype=np.uint8))
    assert list(lm[[0, 1, 2, 3, 7]]) == [448.0, 2.0 ** -9, 2.0 ** -6, 1.0, -448.0]
    assert np.isnan(lm[4]) and np.isnan(lm[5]) and lm[6] == 0.0 and np.signbit(lm[6])

    def tdeq(c, s):
        return (torch.from_numpy(c).view(torch.float8_e4m3fn).double()
                * torch.from_numpy(s).double()[:, None]).numpy()
    rng = np.random.default_rng(41)
    B, W, hq, hkv, d, dv = 2, 8, 4, 2, 16, 8
    kc = rng.integers(0, 126, (B, W, hkv, d), dtype=np.uint8) | rng.choice([0, 128], (B, W, hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 126, (B, W, hkv, dv), dtype=np.uint8)
    ks, vs = np.array([0.5, 0.03]), np.array([0.25, 2.0])
    q = rng.standard_normal((B, hq, d))
    pos = np.array([3, 40])
    sink = np.array([0.0, -1.0, 1.0, 2.0])
    got = O.swa_sink_decode_ring_fp8(q, kc, vc, ks, vs, pos, sink, rope_theta=3.0, rotary_fraction=0.5)
    ref = O.swa_sink_decode_ring(q, tdeq(kc, ks), tdeq(vc, vs), pos, sink, rope_theta=3.0,
                                 rotary_fraction=0.5)
    assert np.abs(got - ref).max() < 1e-12
    offs = np.array([0, 5, 17])
    kc2 = rng.integers(0, 126, (17, hkv, d), dtype=np.uint8)
    vc2 = rng.integers(128, 254, (17, hkv, dv), dtype=np.uint8)
    pos2 = np.array([4, 9])
    got = O.swa_sink_decode_contiguous_fp8(q, kc2, vc2, ks, vs, offs, pos2, window=None)
    ref = O.swa_sink_decode_contiguous(q, tdeq(kc2, ks), tdeq(vc2, vs), offs, pos2, window=None)
    assert np.abs(got - ref).max() < 1e-12
    # sparse attention over E4M3 K/V, RoPE rotating the key values
    n, mx = 24, 5
    kc3 = rng.integers(0, 126, (1, n, hkv, d), dtype=np.uint8)
    vc3 = rng.integers(0, 254, (1, n, hkv, dv), dtype=np.uint8) & 0xF7   # no NaN codes
    q3 = rng.standard_normal((1, n, hq, d))
    idx = np.full((1, n, hkv, mx), -1, dtype=np.int64)
    cnt = np.zeros((1, n, hkv), dtype=np.int64)
    for i in range(n):
        for g in range(hkv):
            avail = max(0, i - 3)
            pick = np.sort(rng.choice(avail, size=min(mx, avail), replace=False)) if avail else []
            idx[0, i, g, :len(pick)] = pick
            cnt[0, i, g] = len(pick)
    rows = np.arange(n)
    got_s = O.sparse_rows_fp8(q3, kc3, vc3, ks, vs, idx, cnt, rows, sink, recent=4,
                              rope_theta=3.0, rotary_fraction=0.5)
    ref_s = O.sparse_rows(q3, tdeq(kc3, ks), tdeq(vc3, vs), idx, cnt, rows, sink, recent=4,
                          rope_theta=3.0, rotary_fraction=0.5)
    assert np.abs(got_s - ref_s).max() < 1e-12
    # the same through the per-sequence loader (codes of one sequence at a time)
    got = O.swa_sink_decode_contiguous_fp8(
        q, None, None, ks, vs, offs, pos2, window=None,
        kv_loader=lambda b: (kc2[offs[b]:offs[b + 1]], vc2[offs[b]:offs[b + 1]]))
    assert np.abs(got - ref).max() < 1e-12


def pin_p15_multi_token_decode(O):
    """MTP verification step (syt-nju.github.io MTP section): T queries at
    p .. p + T - 1 over a ring of S >= W + T - 1 slots or a contiguous cache
    equal those rows of the scalar brute-force prefill of the sequence (RoPE,
    sinks, G = 2, causal among the drafts); a ring of W slots is refused."""
    rng = np.random.default_rng(43)
    L, d, dv, hq, hkv = 11, 8, 4, 4, 2
    q = rng.standard_normal((1, L, hq, d)) * 1.5
    k = rng.standard_normal((1, L, hkv, d)) * 1.5
    v = rng.standard_normal((1, L, hkv, dv))
    sink = np.array([-1.0, 0.0, 0.5, 2.0])
    for W in (1, 3, 5):
        ref = _brute_prefill(q, k, v, sink, W, 3.0, 0.5)
        for T in (1, 2, 4):
            p = L - T                      # first query position
            S = W + T - 1 + 1              # one slot to spare
            kr = np.zeros((1, S, hkv, d))
            vr = np.zeros((1, S, hkv, dv))
            # the ring after writing tokens 0 .. L-1 (the raw keys: the cache
            # holds them as written; rotation happens in the reference too)
            for j in range(L):
                kr[0, j % S], vr[0, j % S] = O.rope(k[:, j:j + 1], np.array([j]), 3.0, 0.5)[0, 0], v[0, j]
            got = O.decode_multi_ring(q[:, p:], kr, vr, np.array([p]), sink, W, rope_theta=3.0,
                                      rotary_fraction=0.5)
            assert np.abs(got - ref[:, p:]).max() < 1e-12, (W, T)
            kc = O.rope(k[0], np.arange(L), 3.0, 0.5)
            got = O.decode_multi_contiguous(q[:, p:], kc, v[0], np.array([0, L]), np.array([p]), sink,
                                            W, rope_theta=3.0, rotary_fraction=0.5)
            assert np.abs(got - ref[:, p:]).max() < 1e-12, (W, T)
            if T > 1:
                small = np.zeros((1, W, hkv, d))
                with pytest.raises(ValueError):
                    O.decode_multi_ring(q[:, p:], small, small[..., :dv], np.array([p]), sink, W)
    # GA (no window, no sink) against SDPA over the whole sequence
    ref = _sdpa(q, k, v, _window_mask(L, None), None, 1 / math.sqrt(d))
    got = O.decode_multi_contiguous(q[:, L - 4:], k[0], v[0], np.array([0, L]), np.array([L - 4]))
    assert np.abs(got - ref[:, L - 4:]).max() < 1e-12


def pin_p16_kv_append(O):
    """Cache append: the E4M3 encoder against torch's float8_e4m3fn cast
    (round to nearest even) on every exact tie and random values in range,
    saturation at 448; the float32-step RoPE against the float64 one; the
    ring slot of each position; and decode over a ring filled by appends
    equal to the scalar brute-force prefill row."""
    rng = np.random.default_rng(47)
    finite = O.e4m3_value(np.arange(127, dtype=np.uint8))
    mids = (finite[:-1] + finite[1:]) / 2                    # every tie between neighbours
    xs = np.concatenate([finite, mids, rng.uniform(-440, 440, 4000),
                         rng.standard_normal(4000) * 0.01, -mids]).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(xs)
    assert np.array_equal(got, ref)
    assert list(O.e4m3_encode(np.array([448.0, 500.0, 1e30, -1e9], dtype=np.float32))) == [0x7E, 0x7E, 0x7E, 0xFE]
    x = rng.standard_normal((5, 3, 16)).astype(np.float32)
    p = np.array([0, 1, 7, 1000, 262143])
    f32 = O.rope_f32_steps(x, p, 1.0e4, 0.5)
    f64 = O.rope(x.astype(np.float64), p, 1.0e4, 0.5)
    assert np.abs(f32 - f64).max() < 2e-6 * np.abs(x).max()
    # appends into a ring of S slots; then decode at the last position
    L, S, W, hq, hkv, d, dv = 9, 6, 4, 4, 2, 8, 4
    q = rng.standard_normal((1, L, hq, d))
    k = rng.standard_normal((1, L, hkv, d)).astype(np.float32)
    v = rng.standard_normal((1, L, hkv, dv)).astype(np.float32)
    kc = np.zeros((1, S, hkv, d), dtype=np.float32)
    vc = np.zeros((1, S, hkv, dv), dtype=np.float32)
    for j0, T in ((0, 3), (3, 1), (4, 5)):
        kc2, vc2 = O.kv_append(kc, vc, k[:, j0:j0 + T], v[:, j0:j0 + T], np.array([j0]), 3.0, 0.5,
                               ring_slots=S, store="f32")
        changed = sorted(set(np.nonzero((kc2 != kc).any(axis=(0, 2, 3)))[0]))
        assert set(changed) <= {j % S for j in range(j0, j0 + T)}
        assert np.array_equal(vc2[0, [j % S for j in range(j0, j0 + T)]], v[0, j0:j0 + T])
        kc, vc = kc2, vc2
    sink = np.array([0.5, -1.0, 0.0, 1.0])
    ref = _brute_prefill(q, k.astype(np.float64), v.astype(np.float64), sink, W, 3.0, 0.5)
    got = O.swa_sink_decode_ring(q[:, L - 1], kc[:, :, :, :], vc, np.array([L - 1]), sink,
                                 rope_theta=3.0, rotary_fraction=0.5)
    # the ring has S = 6 > W = 4 slots: the decode reads the W newest ones
    got_w = O.decode_multi_ring(q[:, L - 1:], kc, vc, np.array([L - 1]), sink, W, rope_theta=3.0,
                                rotary_fraction=0.5)
    assert np.abs(got_w[:, 0] - ref[:, L - 1]).max() < 1e-5
    assert got.shape == (1, hq, dv)
    # contiguous pool, E4M3 store: codes decode back to the scaled, rounded values
    offs = np.array([0, 4])
    ks, vs = np.array([0.02, 0.05], dtype=np.float32), np.array([0.03, 0.01], dtype=np.float32)
    kq, vq = O.kv_append(np.zeros((4, hkv, d), np.uint8), np.zeros((4, hkv, dv), np.uint8),
                         k[:, :4], v[:, :4], np.array([0]), 3.0, 0.5, seq_offsets=offs,
                         k_scale=ks, v_scale=vs, store="e4m3")
    back = O.dequantise_kv(vq, vs)
    assert np.abs(back - v[0, :4]).max() <= np.abs(v[0, :4]).max() * 2 ** -3


def _brute_selection(q, k, b, i, g, recent, K, theta=1.0e7, frac=0.0, off=0):
    """Scalar loops: softmax probabilities with math.fsum, then sorted().
    With frac > 0 every q and k vector is first rotated by _brute_rope at its
    own position off + index."""
    hq, d = q.shape[2], q.shape[3]
    G = hq // k.shape[2]
    R = 2 * int(math.floor(frac * d / 2))
    last = i - recent
    if last < 0:
        return []
    kr = [_brute_rope(list(k[b, j, g]), off + j, theta, R) for j in range(i + 1)]
    imp = [0.0] * (last + 1)
    for h in range(g * G, (g + 1) * G):
        qi = _brute_rope(list(q[b, i, h]), off + i, theta, R)
        a = [math.fsum(qi[t] * kr[j][t] for t in range(d)) / math.sqrt(d)
             for j in range(i + 1)]
        m = max(a)
        z = math.fsum(math.exp(x - m) for x in a)
        for j in range(last + 1):
            imp[j] += math.exp(a[j] - m) / z
    order = sorted(range(last + 1), key=lambda j: (-imp[j], j))
    return sorted(order[:min(K, last + 1)])


def pin_p17_token_selection(O):
    """Token selection (aideepthink.cn section 4, reading of the importance):
    against scalar brute force; all candidates when they fit; with one head
    per group the ranking is the logits' (torch topk); exact ties go to the
    lower position; and sparse attention over all candidates is full causal
    attention."""
    rng = np.random.default_rng(53)
    n, hq, hkv, d = 14, 4, 2, 8
    q = rng.standard_normal((1, n, hq, d)) * 2
    k = rng.standard_normal((1, n, hkv, d)) * 2
    rows = np.arange(n)
    for recent, K in ((1, 3), (3, 4), (2, 100)):
        idx, cnt = O.select_tokens(q, k, rows, recent, K)
        for i in rows:
            for g in range(hkv):
                want = _brute_selection(q, k, 0, int(i), g, recent, K)
                assert cnt[0, i, g] == len(want)
                assert list(idx[0, i, g, :len(want)]) == want, (recent, K, i, g)
                assert (idx[0, i, g, len(want):] == -1).all()
    # RoPE on with a position offset, on a subset of rows of two sequences
    q2 = rng.standard_normal((2, n, hq, d)) * 2
    k2 = rng.standard_normal((2, n, hkv, d)) * 2
    rows2 = np.array([3, 8, 13])
    for frac, theta, off in ((0.5, 3.0, 9), (1.0, 5.0, 2)):
        idx, cnt = O.select_tokens(q2, k2, rows2, 2, 4, rope_theta=theta, rotary_fraction=frac,
                                   pos_offset=off)
        for b in range(2):
            for t, i in enumerate(rows2):
                for g in range(hkv):
                    want = _brute_selection(q2, k2, b, int(i), g, 2, 4, theta, frac, off)
                    assert cnt[b, t, g] == len(want)
                    assert list(idx[b, t, g, :len(want)]) == want, (frac, b, i, g)
                    imp = O.selection_importance(q2, k2, b, int(i), g, 2, rope_theta=theta,
                                                 rotary_fraction=frac, pos_offset=off)
                    # probabilities of one head sum to 1 over 0 .. i; the
                    # candidates carry at most G of that
                    assert imp.min() > 0 and imp.sum() < hq // hkv
    # one head per group: the top-K of the probabilities is the top-K of the logits
    q1 = rng.standard_normal((1, 40, 3, 16))
    k1 = rng.standard_normal((1, 40, 3, 16))
    idx, cnt = O.select_tokens(q1, k1, [39], 4, 7)
    for g in range(3):
        logits = torch.from_numpy(k1[0, :36, g] @ q1[0, 39, g])
        want = np.sort(torch.topk(logits, 7).indices.numpy())
        assert list(idx[0, 0, g, :7]) == list(want)
    # exact ties: identical keys at positions 0, 2, 5 tie; the lower ones win
    kt = rng.standard_normal((1, 12, 1, 8))
    kt[0, [0, 2, 5]] = kt[0, 7]
    qt = rng.standard_normal((1, 12, 2, 8))
    qt[0, 11, :] = kt[0, 7, 0] * 3                  # those keys dominate
    idx, cnt = O.select_tokens(qt, kt, [11], 3, 3)
    assert list(idx[0, 0, 0, :3]) == [0, 2, 5]
    # selecting every candidate makes sparse attention the full causal attention
    v = rng.standard_normal((1, n, hkv, 4))
    idx, cnt = O.select_tokens(q, k, rows, 2, n)
    full = O.sparse_sink_attn(q, k, v, idx, cnt, None, recent=2)
    ga = O.ga_prefill(q, k, v)
    assert np.abs(full - ga).max() < 1e-12


PINS = [pin_p1_no_sink_is_masked_softmax, pin_p2_wide_window_is_causal, pin_p3_sink_as_extra_key,
        pin_p4_weights_sum, pin_p5_unit_window, pin_p6_zero_query, pin_p7_brute_force,
        pin_p8_rope, pin_p9_gqa, pin_p10_decode_equals_prefill_row, pin_p11_sparse,
        pin_p12_large_sink_is_stable, pin_p13_chunk, pin_p14_fp8_cache,
        pin_p15_multi_token_decode, pin_p16_kv_append, pin_p17_token_selection]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin_holds(pin):
    pin(OA)


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin.
# ---------------------------------------------------------------------------

MUTANTS = {
    "drop_sink_from_denominator": ("den = math.exp(sink[g] - m[g]) if sink[g] != NEG_INF else 0.0",
                                   "den = 0.0"),
    "window_one_too_wide": ("max(0, i - window + 1)", "max(0, i - window)"),
    "window_one_too_narrow": ("max(0, i - window + 1)", "max(0, i - window + 2)"),
    "rope_wrong_sign": ("np.exp(1j * angle)", "np.exp(-1j * angle)"),
    "rope_freq_over_d": ("-(2.0 * r) / rot)", "-(2.0 * r) / d)"),
    "rope_adjacent_pairs": ("z = (x[..., :half] + 1j * x[..., half:rot]) * turn",
                            "z = (x[..., 0:rot:2] + 1j * x[..., 1:rot:2]) * turn"),
    "gqa_interleaved_heads": ("hs = slice(g * G, (g + 1) * G)", "hs = slice(g, None, hkv)"),
    "scale_by_dv": ("scale = 1.0 / math.sqrt(d)\n    s_all = _sink_vector(sink, hq)\n    qr",
                    "scale = 1.0 / math.sqrt(v.shape[-1])\n    s_all = _sink_vector(sink, hq)\n    qr"),
    "values_misaligned": ("out[g] = (e @ vj) / den", "out[g] = (e @ vj[::-1]) / den"),
    "max_ignores_sink": ("m = np.maximum(a.max(axis=1), sink)", "m = a.max(axis=1)"),
    "ring_slot_reversed": ("return p - np.mod(p - s, window)", "return p - np.mod(s - p, window)"),
    "sparse_drops_selection": ("return np.union1d(sel, rec)", "return rec"),
    "sparse_recent_too_wide": ("lo = max(0, i - recent + 1)", "lo = max(0, i - recent)"),
    "sink_in_numerator": ("out[g] = (e @ vj) / den", "out[g] = (e @ vj + math.exp(min(sink[g] - m[g], 0.0))) / den"),
    "chunk_rows_from_zero": ("rows = n - q_len + np.arange(q_len)", "rows = np.arange(q_len)", ),
    "cached_chunk_query_unrotated": ("qr = rope(q, pos_offset + rows, rope_theta, rotary_fraction)\n    out",
                                     "qr = np.asarray(q, dtype=np.float64)\n    out"),
    "multi_ring_slot_by_window": ("slots = np.mod(J, S)", "slots = np.mod(J, window)"),
    "multi_query_not_causal_among_drafts": ("            p = int(pos[b]) + t\n            J = window_keys(p, window)\n            qt",
                                            "            p = int(pos[b]) + t\n            J = window_keys(int(pos[b]) + T - 1, window)\n            qt"),
    "e4m3_encode_ties_up": ("np.where(hi % 2 == 0, hi, lo)", "hi"),
    "append_slot_by_window": ("rows = (b, np.mod(ps, ring_slots))", "rows = (b, np.mod(ps, ring_slots - 1))"),
    "selection_ties_to_higher": ("order = np.lexsort((np.arange(imp.size), -imp))",
                                 "order = np.lexsort((-np.arange(imp.size), -imp))"),
    "selection_window_inclusive": ("    last = i - recent\n    if last < 0:\n        return np.zeros(0)",
                                   "    last = i - recent + 1\n    if last < 0:\n        return np.zeros(0)"),
    "selection_lse_over_candidates": ("lse = m + math.log(np.exp(a - m).sum())",
                                      "lse = m + math.log(np.exp(a[:last + 1] - m).sum())"),
    "e4m3_bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "e4m3_subnormal_as_normal": ("np.where(e == 0, m * 2.0 ** -9,", "np.where(e < 0, m * 2.0 ** -9,"),
    "fp8_v_scale_dropped": ("dequantise_kv(v_codes, v_scale), pos, sink, scale=scale,",
                            "e4m3_value(v_codes), pos, sink, scale=scale,"),
    "sparse_fp8_k_scale_dropped": ("return sparse_rows(q, dequantise_kv(k_codes, k_scale),",
                                   "return sparse_rows(q, e4m3_value(k_codes),"),
    "fp8_scales_swapped": ("return dequantise_kv(kb, k_scale), dequantise_kv(vb, v_scale)",
                           "return dequantise_kv(kb, v_scale), dequantise_kv(vb, k_scale)"),
    "sparse_query_rotated_at_list_index": ("qr = rope(q_sel, pos_offset + rows, rope_theta, rotary_fraction)",
                                           "qr = rope(q_sel, pos_offset + np.arange(len(rows)), rope_theta, rotary_fraction)",
                                           "sparse_rows"),
    "sparse_keys_rotated_without_offset": ("kr = rope(k, pos_offset + np.arange(n), rope_theta, rotary_fraction)",
                                           "kr = rope(k, np.arange(n), rope_theta, rotary_fraction)",
                                           "sparse_rows"),
    "selection_query_rotated_without_offset": ("qi = rope(q[b, i][None], np.array([pos_offset + i]), rope_theta,",
                                               "qi = rope(q[b, i][None], np.array([i]), rope_theta,"),
    "selection_keys_rotated_one_late": ("kr = rope(k[b, :i + 1], pos_offset + np.arange(i + 1), rope_theta,",
                                        "kr = rope(k[b, :i + 1], pos_offset + np.arange(1, i + 2), rope_theta,"),
    "decode_query_not_rotated": ("qb = rope(q[b][None], np.array([p]), rope_theta, rotary_fraction)[0]\n        slots",
                                 "qb = np.asarray(q[b], dtype=np.float64)\n        slots"),
}


def _mutant(name):
    """A copy of the oracle module with one planted mistake.  An entry of
    MUTANTS is (old, new) or (old, new, function): with a function name only
    that function's text is changed (the same line may appear elsewhere)."""
    old, new, *where = MUTANTS[name]
    src = inspect.getsource(OA)
    if where:
        fsrc = inspect.getsource(getattr(OA, where[0]))
        assert src.count(fsrc) == 1 and fsrc.count(old) >= 1, f"mutation site for {name} not found"
        mutated = src.replace(fsrc, fsrc.replace(old, new))
    else:
        assert src.count(old) >= 1, f"mutation site for {name} not found"
        mutated = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(mutated, "<mutant " + name + ">", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin catches the planted mistake {name}"


# ---------------------------------------------------------------------------
# Input generator checks and the page constants
# ---------------------------------------------------------------------------

def test_sparse_selection_lists_are_valid():
    n, hkv, recent, max_sel = 300, 3, 16, 40
    idx, cnt = synthetic.sparse_selection(2, n, hkv, recent, max_sel, 31)
    idx, cnt = idx.numpy(), cnt.numpy()
    for b in range(2):
        for i in range(n):
            avail = max(0, i - recent)
            for g in range(hkv):
                c = cnt[b, i, g]
                assert c == min(max_sel, avail)
                row = idx[b, i, g]
                sel = row[:c]
                assert (row[c:] == -1).all()
                if c:
                    assert (np.diff(sel) > 0).all()
                    assert sel[0] >= 0 and sel[-1] < avail
                if avail <= max_sel:
                    assert np.array_equal(sel, np.arange(avail))
    # different (i, g) rows draw different sets
    assert not np.array_equal(idx[0, n - 1, 0], idx[0, n - 1, 1])


def test_sparse_selection_is_uniform():
    # Floyd's sampling: every candidate equally likely (chi-square style bound).
    n, recent, max_sel = 64, 4, 10
    idx, cnt = synthetic.sparse_selection(1, n, 400, recent, max_sel, 32)
    i = n - 1
    vals = idx[0, i, :, :max_sel].numpy().ravel()
    hist = np.bincount(vals, minlength=i - recent)
    expect = 400 * max_sel / (i - recent)
    assert hist.min() > 0.4 * expect and hist.max() < 1.8 * expect


def test_workloads_use_page_constants():
    wl = synthetic.WORKLOADS
    W = GOLD["window"]["value"]
    assert wl["swa_prefill_n32768"]["window"] == W
    assert (wl["swa_prefill_n32768"]["hq"], wl["swa_prefill_n32768"]["hkv"]) == \
        tuple(GOLD["swa_heads_q_kv"]["value"])
    assert (wl["ga_prefill_n32768"]["hq"], wl["ga_prefill_n32768"]["hkv"]) == \
        tuple(GOLD["ga_heads_q_kv"]["value"])
    for name in ("swa_prefill_n32768", "ga_prefill_n32768", "sparse_prefill_n65536"):
        assert wl[name]["d_qk"] == GOLD["d_qk"]["value"]
        assert wl[name]["d_v"] == GOLD["d_v"]["value"]
    assert wl["swa_prefill_n32768"]["rope_theta"] == GOLD["swa_rope_theta"]["value"]
    assert wl["ga_prefill_n32768"]["rope_theta"] == GOLD["ga_rope_theta"]["value"]
    assert wl["swa_prefill_n32768"]["rotary_fraction"] == GOLD["partial_rotary_factor"]["value"]
    assert wl["sparse_prefill_n65536"]["recent"] == GOLD["sparse_recent"]["value"]
    assert wl["sparse_prefill_n65536"]["max_sel"] == GOLD["sparse_selected"]["value"]
    for name in ("swa_chunk_q16384_prefix1048576", "ga_chunk_q16384_prefix114688"):
        assert wl[name]["q_len"] == GOLD["prefill_chunk_tokens"]["value"]
    swc = wl["swa_chunk_q16384_prefix1048576"]
    assert swc["kv_len"] - swc["q_len"] == GOLD["longest_prefix_tokens"]["value"]
    assert (swc["hq"], swc["hkv"], swc["window"]) == (*GOLD["swa_heads_q_kv"]["value"], W)
    gac = wl["ga_chunk_q16384_prefix114688"]
    assert (gac["hq"], gac["hkv"], gac["window"]) == (*GOLD["ga_heads_q_kv"]["value"], 0)
    dec = wl["hybrid_decode_b64"]
    assert dec["swa"]["window"] == W
    assert (dec["swa"]["hq"], dec["swa"]["hkv"]) == tuple(GOLD["swa_heads_q_kv"]["value"])
    assert (dec["ga"]["hq"], dec["ga"]["hkv"]) == tuple(GOLD["ga_heads_q_kv"]["value"])


def test_generator_is_seeded_and_rne():
    a = synthetic.normal((1000,), 5, "cpu", "bf16")
    b = synthetic.normal((1000,), 5, "cpu", "bf16")
    assert torch.equal(a, b)
    f = synthetic.normal((1000,), 5, "cpu", "f32")
    # bf16 cast is round-to-nearest-even of the same float32 draw
    bits = f.view(torch.int32).to(torch.int64)
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    assert torch.equal(rne.to(torch.int32), a.view(torch.int16).to(torch.int32) & 0xFFFF)
