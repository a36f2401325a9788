"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Tolerances (from the problem statement of the method and the arithmetic):
  * fp32 storage: max |gpu - oracle| <= 1e-5;
  * bf16 storage (fp32 accumulation): max-abs <= 2e-2 and
    rel-L2 = ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3.
The bf16 budget: the only roundings in the kernels are the RoPE-rotated
dims of q~ and k~ to bf16, P to bf16 before the PV product and the final
store; each is a relative 2^-9 step, together ~2e-3 rel-L2.

Small cases span several tiles and a ragged tail and are checked element by
element over the whole output; the full-size workloads (the same launch
configuration the benchmark times) are checked on sampled rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_MAX, BF16_RL2, F32_MAX = 2e-2, 5e-3, 1e-5


def _np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _check(name, got, ref, fp32=False):
    g = _np(got) if isinstance(got, torch.Tensor) else got
    d = g - ref
    mx = float(np.abs(d).max()) if d.size else 0.0
    rl2 = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    print(f"[parity] {name}: max_abs={mx:.3e} rel_l2={rl2:.3e}", flush=True)
    assert np.isfinite(g).all(), f"{name}: non-finite output"
    if fp32:
        assert mx <= F32_MAX, f"{name}: max_abs {mx}"
    else:
        assert mx <= BF16_MAX and rl2 <= BF16_RL2, f"{name}: max_abs {mx} rel_l2 {rl2}"


def _prefill_case(B, n, hq, hkv, dtype, seed, sink_range=(-2.0, 2.0)):
    return synthetic.prefill_inputs(B, n, hq, hkv, 192, 128, dtype, seed, DEV, sink_range)


def _host(x):
    q, k, v = (_np(x[t]) for t in "qkv")
    s = None if x["sink"] is None else _np(x["sink"])
    return q, k, v, s


# ---------------------------------------------------------------------------
# Tiny fp32 SWA+sink (n = 512, 2 q heads over 1 kv head, no RoPE)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window,with_sink", [(128, True), (128, False), (512, True), (512, False)])
def test_tiny_fp32_prefill(gpu_lib, window, with_sink):
    x = _prefill_case(1, 512, 2, 1, "f32", 1, sink_range=(-3.0, 3.0) if with_sink else None)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=window)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=window)
    _check(f"tiny fp32 W={window} sink={with_sink}", o, ref, fp32=True)
    if window == 512 and not with_sink:
        # W >= n without a sink is plain causal softmax attention
        _check("tiny fp32 W=n vs causal", o, oracle.ga_prefill(q, k, v), fp32=True)
        og = gpu_lib.ga_prefill(x["q"], x["k"], x["v"])
        _check("tiny fp32 ga_prefill", og, oracle.ga_prefill(q, k, v), fp32=True)


# ---------------------------------------------------------------------------
# bf16 prefill, whole outputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,n,hq,hkv,window", [
    (1, 1000, 64, 8, 128),     # SWA layer heads, ragged tail (1000 = 62.5 blocks of 16)
    (2, 333, 16, 16, 128),     # MHA (G = 1): 128-token blocks
    (1, 517, 32, 4, 128),      # G = 8 with batch of one
    (1, 130, 64, 1, 128),      # G = 64: 2 tokens per block
    (1, 300, 8, 4, 1),         # window of one token
    (1, 300, 8, 4, 7),         # narrow window
    (1, 90, 16, 2, 128),       # n < W
    (1, 1, 64, 8, 128),        # a single token
])
def test_swa_prefill_bf16(gpu_lib, B, n, hq, hkv, window):
    x = _prefill_case(B, n, hq, hkv, "bf16", 20 + n)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=window,
                                 rope_theta=1.0e4, rotary_fraction=0.334)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=window, rope_theta=1.0e4, rotary_fraction=0.334)
    _check(f"swa bf16 B={B} n={n} {hq}/{hkv} W={window}", o, ref)


@pytest.mark.parametrize("B,n,hq,hkv", [(1, 700, 64, 4), (2, 257, 8, 8), (1, 1030, 16, 1)])
def test_ga_prefill_bf16(gpu_lib, B, n, hq, hkv):
    x = _prefill_case(B, n, hq, hkv, "bf16", 40 + n, sink_range=None)
    o = gpu_lib.ga_prefill(x["q"], x["k"], x["v"], rope_theta=1.0e7, rotary_fraction=0.334)
    q, k, v, _ = _host(x)
    ref = oracle.ga_prefill(q, k, v, rope_theta=1.0e7, rotary_fraction=0.334)
    _check(f"ga bf16 B={B} n={n} {hq}/{hkv}", o, ref)


@pytest.mark.parametrize("B,n,hq,hkv,window,frac,sink", [
    (2, 611, 64, 8, 128, 0.334, True),    # items of two sequences in one stream
    (1, 403, 64, 2, 33, 0.334, True),     # G = 32, window not a multiple of the tile
    (1, 77, 128, 1, 128, 0.17, True),     # G = 128 (one token per block), R = 32
    (1, 500, 64, 8, 128, 0.0, False),     # no RoPE, no sink
    (3, 129, 32, 4, 1, 0.334, True),      # one-token window
    (1, 960, 16, 2, 300, 0.17, False),    # window wider than the 32-key tile stream start
])
def test_matrix_core_prefill_shapes(gpu_lib, B, n, hq, hkv, window, frac, sink):
    """Shapes routed to the matrix-core prefill kernels (G >= 8, R in {0, 32, 64}):
    the resident-ring kernel for windows up to its limit, the two-tile-step
    kernel for wider ones (W = 300 here)."""
    x = _prefill_case(B, n, hq, hkv, "bf16", 90 + n, sink_range=(-2.0, 2.0) if sink else None)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=window,
                                 rope_theta=1.0e4, rotary_fraction=frac, pos_offset=17)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=window, rope_theta=1.0e4,
                                  rotary_fraction=frac, pos_offset=17)
    _check(f"matrix-core B={B} n={n} {hq}/{hkv} W={window} R/2={int(frac * 96)}", o, ref)


def _windowed_runs(B, n, hq, hkv):
    """Item runs of the windowed ring kernel on this device: an item is one kv
    head and T = 256 / G query tokens, items are ordered (sequence, kv head,
    block), and each workgroup takes ceil(items / CUs) consecutive items.
    Returns T, blocks per head, and the items j whose successor j + 1 lies
    in the same run but belongs to another (sequence, kv head): the point
    where a run restarts its K/V tile ring."""
    G = hq // hkv
    T = 256 // G
    nblk = -(-n // T)
    items = B * hkv * nblk
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    run = -(-items // cus)
    cross = [j for j in range(items - 1) if (j + 1) % run != 0 and j // nblk != (j + 1) // nblk]
    return T, nblk, cross


@pytest.mark.parametrize("B,n,hq,hkv", [(1, 1100, 64, 8), (3, 700, 64, 8), (2, 1000, 64, 4)])
def test_windowed_run_crosses_heads_and_sequences(gpu_lib, B, n, hq, hkv):
    """Runs of the windowed kernel that move on to another kv head or sequence
    (the causal window of rslog.cc section 2.1 over a batch), compared with
    the oracle over the whole output."""
    T, nblk, cross = _windowed_runs(B, n, hq, hkv)
    print(f"[parity] windowed runs: T={T} blocks/head={nblk} crossings after items {cross}",
          flush=True)
    assert cross, "the shape no longer makes a run cross a head on this device"
    x = _prefill_case(B, n, hq, hkv, "bf16", 400 + n)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=128, rope_theta=1.0e4,
                                 rotary_fraction=0.334, pos_offset=5)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=128, rope_theta=1.0e4, rotary_fraction=0.334,
                                  pos_offset=5)
    _check(f"windowed runs B={B} n={n} {hq}/{hkv}", o, ref)


def test_windowed_run_crossings_long_sequences(gpu_lib):
    """Two sequences of 30000 tokens (runs of 59 items on 256 CUs, 938 blocks
    per kv head): every row of the two items on either side of each crossing
    against the oracle, element by element."""
    B, n, hq, hkv = 2, 30000, 64, 8
    T, nblk, cross = _windowed_runs(B, n, hq, hkv)
    print(f"[parity] long windowed runs: {len(cross)} crossings", flush=True)
    assert len(cross) >= 4
    x = _prefill_case(B, n, hq, hkv, "bf16", 410)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=128, rope_theta=1.0e4,
                                 rotary_fraction=0.334)
    toks = set()
    for j in cross:
        for it in (j, j + 1):
            blk = it % nblk
            toks.update(range(blk * T, min(n, blk * T + T)))
    rows = np.array(sorted(toks))
    ridx = torch.from_numpy(rows).to(DEV)
    ref = oracle.prefill_rows(None, _np(x["k"]), _np(x["v"]), rows, sink=_np(x["sink"]),
                              window=128, rope_theta=1.0e4, rotary_fraction=0.334,
                              q_rows=_np(x["q"][:, ridx]))
    _check(f"long windowed runs ({len(rows)} rows at crossings)", o[:, ridx], ref)


@pytest.mark.parametrize("B,n,hq,hkv", [(3, 250, 64, 8), (1, 515, 128, 4)])
def test_matrix_core_ga_shapes(gpu_lib, B, n, hq, hkv):
    x = _prefill_case(B, n, hq, hkv, "bf16", 95 + n, sink_range=None)
    o = gpu_lib.ga_prefill(x["q"], x["k"], x["v"], rope_theta=1.0e7, rotary_fraction=0.334)
    q, k, v, _ = _host(x)
    ref = oracle.ga_prefill(q, k, v, rope_theta=1.0e7, rotary_fraction=0.334)
    _check(f"matrix-core ga B={B} n={n} {hq}/{hkv}", o, ref)


@pytest.mark.parametrize("frac", [0.0, 2.0 / 3.0, 1.0])
def test_prefill_rotary_widths(gpu_lib, frac):
    """R = 0, 128 and 192 rotated dims (the MFMA path pairs r with r + R/2 in lane)."""
    x = _prefill_case(1, 200, 16, 2, "bf16", 61)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=64, rope_theta=500.0,
                                 rotary_fraction=frac, pos_offset=1000)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=64, rope_theta=500.0, rotary_fraction=frac,
                                  pos_offset=1000)
    _check(f"rotary fraction {frac:.3f}", o, ref)


@pytest.mark.parametrize("hq,hkv,frac", [(64, 8, 0.334), (32, 2, 0.17)])
def test_windowed_prefill_far_positions(gpu_lib, hq, hkv, frac):
    """The windowed kernel turns q in registers and K in LDS at the tokens'
    positions: behind a position offset of 2^20 + 123 the angles reach
    ~1e6 rad, where only an fp64 angle keeps them right; 700 tokens leave a
    ragged last block (rows past the end dropped by the range-checked
    stores)."""
    x = _prefill_case(1, 700, hq, hkv, "bf16", 77 + hq)
    off = (1 << 20) + 123
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=128, rope_theta=1.0e4,
                                 rotary_fraction=frac, pos_offset=off)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=128, rope_theta=1.0e4, rotary_fraction=frac,
                                  pos_offset=off)
    _check(f"windowed prefill at positions {off}.. {hq}/{hkv} frac {frac}", o, ref)


@pytest.mark.parametrize("qmul", [2.0, 4.0])
def test_sink_sensitive_case(gpu_lib, qmul):
    """Large sinks U(2, 6) (the sink absorbs a large share of each row) and a
    sharpened q: a kernel that dropped or mis-scaled the sink term fails here
    even where the plain workload cannot tell.

    At q x 4 the rows collapse onto single keys with |o| up to ~5, and
    rounding the rotated q~ and k~ dims to bf16 (the matrix-core operands)
    plus the bf16 store already costs 2.9e-2 to 3.2e-2 max-abs against the
    exact result: the floor measured on the CPU by
    tests/test_tolerance_floor.py on inputs of this recipe.  The max-abs
    bar there is 5e-2 (>= 1.4 x that floor), rel-L2 stays <= 5e-3; at
    q x 2 the floor is 1.4e-2 and the standard bar applies."""
    x = _prefill_case(1, 600, 64, 8, "bf16", 62, sink_range=(2.0, 6.0))
    x["q"] = (x["q"].float() * qmul).to(torch.bfloat16)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=128, rope_theta=1.0e4,
                                 rotary_fraction=0.334)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=128, rope_theta=1.0e4, rotary_fraction=0.334)
    if qmul <= 2.0:
        _check(f"sink-sensitive q x {qmul}", o, ref)
    else:
        g = _np(o)
        d = np.abs(g - ref)
        rl2 = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
        print(f"[parity] sink-sensitive q x {qmul}: max_abs={d.max():.3e} rel_l2={rl2:.3e} "
              f"max|o|={np.abs(ref).max():.2f}", flush=True)
        assert rl2 <= BF16_RL2
        assert d.max() <= 5e-2
    no_sink = oracle.swa_sink_prefill(q, k, v, None, window=128, rope_theta=1.0e4,
                                      rotary_fraction=0.334)
    assert np.abs(_np(o) - no_sink).max() > 0.1          # the sink visibly matters here


def test_weight_sum_closed_form_on_gpu(gpu_lib):
    """V = 1: every output equals the attention weight sum, which is < 1 with a
    sink and exactly 1 without one (the invariant of the pages' comparison table)."""
    x = _prefill_case(1, 400, 16, 2, "bf16", 63)
    ones = torch.ones_like(x["v"])
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], ones, x["sink"], window=128)
    o0 = gpu_lib.swa_sink_prefill(x["q"], x["k"], ones, None, window=128)
    q, k, _, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, np.ones_like(_np(ones)), s, window=128)
    _check("V=1 weight sum", o, ref)
    assert (ref < 1.0).all()            # the sink takes a share of every row
    assert (_np(o) <= 1.0).all()        # bf16 output: sums just below 1 may round to 1
    assert np.abs(_np(o0) - 1.0).max() <= 2e-2


def test_prefill_deterministic(gpu_lib):
    x = _prefill_case(1, 700, 64, 8, "bf16", 64)
    a = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=128, rope_theta=1.0e4,
                                 rotary_fraction=0.334)
    b = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=128, rope_theta=1.0e4,
                                 rotary_fraction=0.334)
    assert torch.equal(a, b)


def test_prefill_generic_shapes(gpu_lib):
    """Head dims the matrix-core kernel does not take run on the generic kernel."""
    x = synthetic.prefill_inputs(1, 150, 6, 3, 64, 96, "bf16", 65, DEV)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=32, rope_theta=1.0e4,
                                 rotary_fraction=0.25)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill(q, k, v, s, window=32, rope_theta=1.0e4, rotary_fraction=0.25)
    _check("generic bf16 d=64/96", o, ref)
    xf = synthetic.prefill_inputs(1, 150, 6, 3, 64, 96, "f32", 66, DEV)
    of = gpu_lib.ga_prefill(xf["q"], xf["k"], xf["v"], rope_theta=1.0e4, rotary_fraction=0.25)
    q, k, v, _ = _host(xf)
    _check("generic f32 GA d=64/96", of, oracle.ga_prefill(q, k, v, rope_theta=1.0e4,
                                                           rotary_fraction=0.25), fp32=True)


def test_empty_inputs(gpu_lib):
    x = _prefill_case(1, 0, 8, 2, "bf16", 67)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=128)
    assert o.shape == (1, 0, 8, 128)


# ---------------------------------------------------------------------------
# Full-size prefill workloads, sampled rows
# ---------------------------------------------------------------------------

def _sample_rows(n, seed, k=96):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(64, n - 64), size=k, replace=False)
    return np.unique(np.concatenate([np.arange(64), mid, np.arange(n - 64, n)]))


def test_swa_prefill_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["swa_prefill_n32768"]
    x = _prefill_case(1, wl["n"], wl["hq"], wl["hkv"], "bf16", wl["seed"], wl["sink_range"])
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=wl["window"],
                                 rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"])
    rows = _sample_rows(wl["n"], 71)
    ridx = torch.from_numpy(rows).to(DEV)
    ref = oracle.prefill_rows(None, _np(x["k"]), _np(x["v"]), rows, sink=_np(x["sink"]),
                              window=wl["window"], rope_theta=wl["rope_theta"],
                              rotary_fraction=wl["rotary_fraction"], q_rows=_np(x["q"][:, ridx]))
    _check("swa full size (sampled rows)", o[:, ridx], ref)


def test_ga_prefill_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["ga_prefill_n32768"]
    x = _prefill_case(1, wl["n"], wl["hq"], wl["hkv"], "bf16", wl["seed"], None)
    o = gpu_lib.ga_prefill(x["q"], x["k"], x["v"], rope_theta=wl["rope_theta"],
                           rotary_fraction=wl["rotary_fraction"])
    rng = np.random.default_rng(72)
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(wl["n"], 40, replace=False),
                                     np.arange(wl["n"] - 8, wl["n"])]))
    ridx = torch.from_numpy(rows).to(DEV)
    ref = oracle.prefill_rows(None, _np(x["k"]), _np(x["v"]), rows, sink=None, window=None,
                              rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"],
                              q_rows=_np(x["q"][:, ridx]))
    _check("ga full size (sampled rows)", o[:, ridx], ref)


# ---------------------------------------------------------------------------
# Chunked prefill: the last q_len positions behind a cached prefix
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,q_len,kv_len,hq,hkv,window,dtype,frac", [
    (2, 300, 1000, 64, 8, 128, "bf16", 0.334),   # ring kernel, ragged chunk and prefix
    (1, 1, 777, 64, 8, 128, "bf16", 0.334),      # a single query behind the prefix
    (1, 100, 150, 64, 8, 128, "bf16", 0.334),    # window reaches back to position 0
    (1, 250, 900, 64, 4, 0, "bf16", 0.334),      # GA chunk (G = 16)
    (1, 33, 400, 128, 1, 33, "bf16", 0.17),      # G = 128, R = 32, odd window
    (1, 200, 700, 16, 8, 128, "bf16", 0.334),    # G = 2: generic kernel
    (1, 130, 600, 4, 2, 64, "f32", 0.334),       # fp32: generic kernel
    (1, 90, 90, 64, 8, 128, "bf16", 0.334),      # the whole sequence is the chunk
])
def test_prefill_chunk(gpu_lib, B, q_len, kv_len, hq, hkv, window, dtype, frac):
    sink = (-2.0, 2.0) if window > 0 else None
    x = synthetic.chunk_inputs(B, q_len, kv_len, hq, hkv, 192, 128, dtype, 300 + q_len, DEV, sink)
    o = gpu_lib.swa_sink_prefill_chunk(x["q"], x["k"], x["v"], x["sink"], window=window,
                                       rope_theta=1.0e4, rotary_fraction=frac, pos_offset=5)
    assert o.shape == (B, q_len, hq, 128)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill_chunk(q, k, v, s, window=window, rope_theta=1.0e4,
                                        rotary_fraction=frac, pos_offset=5)
    _check(f"chunk {dtype} B={B} q={q_len} kv={kv_len} {hq}/{hkv} W={window}", o, ref,
           fp32=(dtype == "f32"))


@pytest.mark.parametrize("hq,hkv,window", [(64, 8, 128), (64, 4, 0), (16, 8, 128)])
def test_prefill_chunk_is_rows_of_whole_prefill(gpu_lib, hq, hkv, window):
    """A chunk starting on a query-block boundary (a multiple of 128 positions)
    walks the same tiles in the same order as the whole prefill does for those
    rows, so its output is bit-for-bit those rows; other starts agree within
    rounding."""
    x = _prefill_case(1, 1100, hq, hkv, "bf16", 310, (-2.0, 2.0) if window else None)
    kw = dict(window=window, rope_theta=1.0e4, rotary_fraction=0.334, pos_offset=3)
    whole = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], **kw)
    for start in (512, 768, 1023, 333):
        part = gpu_lib.swa_sink_prefill_chunk(x["q"][:, start:].contiguous(), x["k"], x["v"],
                                              x["sink"], **kw)
        if start % 128 == 0 and hq // hkv >= 8:
            assert torch.equal(part, whole[:, start:]), start
        else:
            _check(f"chunk at {start} vs whole prefill {hq}/{hkv}", part, _np(whole[:, start:]))


@pytest.mark.parametrize("B,q_len,kv_len,hq,hkv,window,dtype,frac", [
    (2, 300, 1000, 64, 8, 128, "bf16", 0.334),   # ring kernel, keys read as stored
    (1, 250, 900, 64, 4, 0, "bf16", 0.334),      # GA chunk
    (1, 1, 500, 64, 8, 128, "bf16", 0.334),      # a single query
    (1, 200, 700, 16, 8, 128, "bf16", 0.334),    # G = 2: generic kernel
    (1, 130, 600, 4, 2, 64, "f32", 0.334),       # fp32: generic kernel
])
def test_prefill_chunk_cached(gpu_lib, B, q_len, kv_len, hq, hkv, window, dtype, frac):
    """Keys taken as already rotated: any rows serve as the cache."""
    sink = (-2.0, 2.0) if window > 0 else None
    x = synthetic.chunk_inputs(B, q_len, kv_len, hq, hkv, 192, 128, dtype, 330 + q_len, DEV, sink)
    o = gpu_lib.swa_sink_prefill_chunk_cached(x["q"], x["k"], x["v"], x["sink"], window=window,
                                              rope_theta=1.0e4, rotary_fraction=frac,
                                              pos_offset=7)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill_chunk_cached(q, k, v, s, window=window, rope_theta=1.0e4,
                                               rotary_fraction=frac, pos_offset=7)
    _check(f"cached chunk {dtype} B={B} q={q_len} kv={kv_len} {hq}/{hkv} W={window}", o, ref,
           fp32=(dtype == "f32"))


@pytest.mark.parametrize("window", [128, 0])
def test_prefill_chunk_cached_after_append(gpu_lib, window):
    """The serving flow: every token's key and value appended to a contiguous
    cache (keys rotated there), then the chunk attends over the cache.  The
    result is the chunk over the unrotated keys."""
    B, q_len, kv_len, hq, hkv = 2, 260, 800, 64, 8
    sink = (-2.0, 2.0) if window else None
    x = synthetic.chunk_inputs(B, q_len, kv_len, hq, hkv, 192, 128, "bf16", 345, DEV, sink)
    kc = torch.zeros_like(x["k"])
    vc = torch.zeros_like(x["v"])
    offs = torch.arange(0, (B + 1) * kv_len, kv_len, dtype=torch.int64, device=DEV)
    gpu_lib.kv_cache_append(x["k"], x["v"], kc.view(B * kv_len, hkv, 192),
                            vc.view(B * kv_len, hkv, 128), torch.zeros(B, dtype=torch.int64,
                                                                       device=DEV),
                            kv_len - 1, layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=offs,
                            rope_theta=1.0e4, rotary_fraction=0.334)
    o = gpu_lib.swa_sink_prefill_chunk_cached(x["q"], kc, vc, x["sink"], window=window,
                                              rope_theta=1.0e4, rotary_fraction=0.334)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill_chunk(q, k, v, s, window=window, rope_theta=1.0e4,
                                        rotary_fraction=0.334)
    _check(f"chunk over an appended cache W={window}", o, ref)


@pytest.mark.parametrize("q_len,kv_len,hq,hkv,window", [
    (1000, 2003, 64, 8, 129),   # widest window of the K/V ring at G = 8, query start off the tile grid
    (1000, 2003, 64, 8, 130),   # one wider: the two-tile-step kernel
    (700, 1701, 64, 4, 161),    # widest at G = 16
    (260, 260, 64, 8, 100),     # whole sequence, window off the tile grid
])
def test_prefill_window_ring_limits(gpu_lib, q_len, kv_len, hq, hkv, window):
    """The windowed kernel keeps two consecutive query blocks' key tiles in a
    7-tile ring; these shapes sit at (and just past) the widest windows it
    takes, with query blocks not aligned to the 32-key tiles."""
    x = synthetic.chunk_inputs(2, q_len, kv_len, hq, hkv, 192, 128, "bf16", 360 + window, DEV,
                               (-2.0, 2.0))
    o = gpu_lib.swa_sink_prefill_chunk(x["q"], x["k"], x["v"], x["sink"], window=window,
                                       rope_theta=1.0e4, rotary_fraction=0.334, pos_offset=9)
    q, k, v, s = _host(x)
    ref = oracle.swa_sink_prefill_chunk(q, k, v, s, window=window, rope_theta=1.0e4,
                                        rotary_fraction=0.334, pos_offset=9)
    _check(f"ring limits q={q_len} kv={kv_len} {hq}/{hkv} W={window}", o, ref)


def test_prefill_chunk_empty(gpu_lib):
    x = synthetic.chunk_inputs(1, 0, 64, 64, 8, 192, 128, "bf16", 320, DEV)
    o = gpu_lib.swa_sink_prefill_chunk(x["q"], x["k"], x["v"], x["sink"], window=128)
    assert o.shape == (1, 0, 64, 128)


def test_swa_chunk_full_size(gpu_lib):
    """16K-token chunk behind a 2^20-token prefix, sampled rows.  The oracle
    sees only the keys from the first one any query of the chunk reads
    (position kv_len - q_len - W + 1) on, with the RoPE offset moved by the
    same amount: the window makes the output invariant to that shift."""
    wl = synthetic.WORKLOADS["swa_chunk_q16384_prefix1048576"]
    x = synthetic.chunk_inputs(1, wl["q_len"], wl["kv_len"], wl["hq"], wl["hkv"], 192, 128,
                               "bf16", wl["seed"], DEV, wl["sink_range"])
    o = gpu_lib.swa_sink_prefill_chunk(x["q"], x["k"], x["v"], x["sink"], window=wl["window"],
                                       rope_theta=wl["rope_theta"],
                                       rotary_fraction=wl["rotary_fraction"])
    first = wl["kv_len"] - wl["q_len"] - wl["window"] + 1
    rows = _sample_rows(wl["q_len"], 73)
    ridx = torch.from_numpy(rows).to(DEV)
    ref = oracle.prefill_rows(None, _np(x["k"][:, first:]), _np(x["v"][:, first:]),
                              rows + wl["window"] - 1, sink=_np(x["sink"]), window=wl["window"],
                              rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"],
                              pos_offset=first, q_rows=_np(x["q"][:, ridx]))
    _check("swa chunk 16K after 1M (sampled rows)", o[:, ridx], ref)


def test_ga_chunk_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["ga_chunk_q16384_prefix114688"]
    x = synthetic.chunk_inputs(1, wl["q_len"], wl["kv_len"], wl["hq"], wl["hkv"], 192, 128,
                               "bf16", wl["seed"], DEV, None)
    o = gpu_lib.swa_sink_prefill_chunk(x["q"], x["k"], x["v"], None, window=0,
                                       rope_theta=wl["rope_theta"],
                                       rotary_fraction=wl["rotary_fraction"])
    rng = np.random.default_rng(74)
    rows = np.unique(np.concatenate([np.arange(4), rng.choice(wl["q_len"], 24, replace=False),
                                     np.arange(wl["q_len"] - 4, wl["q_len"])]))
    ridx = torch.from_numpy(rows).to(DEV)
    ref = oracle.prefill_rows(None, _np(x["k"]), _np(x["v"]),
                              rows + wl["kv_len"] - wl["q_len"], sink=None, window=None,
                              rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"],
                              q_rows=_np(x["q"][:, ridx]))
    _check("ga chunk 16K after 112K (sampled rows)", o[:, ridx], ref)


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def _ring_case(pos, hq=64, hkv=8, W=128, seed=80, dtype="bf16", sink=(-2.0, 2.0)):
    pos = torch.as_tensor(pos, dtype=torch.int64)
    return synthetic.ring_decode_inputs(len(pos), hq, hkv, W, 192, 128, dtype, seed, pos, DEV, sink)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_decode(gpu_lib, dtype):
    pos = [0, 1, 5, 126, 127, 128, 1000, 131072, 262143, 77777]
    d = _ring_case(pos, dtype=dtype)
    o = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], max(pos), layout=gpu_lib.KV_RING,
                                sink=d["sink"], window=128)
    ref = oracle.swa_sink_decode_ring(_np(d["q"]), _np(d["k"]), _np(d["v"]), np.array(pos),
                                      _np(d["sink"]))
    _check(f"ring decode {dtype}", o, ref, fp32=(dtype == "f32"))


def test_ring_decode_rope_large_positions(gpu_lib):
    """q rotated in the call at p up to 2.6e5 (angles in fp64): base 1e4."""
    pos = [3, 200, 131072, 200001, 262143]
    d = _ring_case(pos, seed=81)
    o = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], 262143, layout=gpu_lib.KV_RING,
                                sink=d["sink"], window=128, rope_theta=1.0e4, rotary_fraction=0.334)
    ref = oracle.swa_sink_decode_ring(_np(d["q"]), _np(d["k"]), _np(d["v"]), np.array(pos),
                                      _np(d["sink"]), rope_theta=1.0e4, rotary_fraction=0.334)
    _check("ring decode rope", o, ref)


@pytest.mark.parametrize("hq,hkv,W", [(64, 4, 64), (16, 4, 100), (32, 8, 33), (8, 8, 128)])
def test_ring_decode_other_windows_and_groups(gpu_lib, hq, hkv, W):
    """The one-launch ring kernels (bf16 and E4M3 caches) at windows below 128,
    where whole wavefronts of slots are empty, and at GQA groups 16, 4 and 1
    (padded MFMA columns), warm-up positions included (rslog.cc section 2.1:
    the window holds the last W tokens, fewer before the W-th)."""
    pos = [0, 3, W - 2, W - 1, W, 5000, 131071]
    d = _ring_case(pos, hq=hq, hkv=hkv, W=W, seed=95)
    o = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], max(pos), layout=gpu_lib.KV_RING,
                                sink=d["sink"], window=W)
    ref = oracle.swa_sink_decode_ring(_np(d["q"]), _np(d["k"]), _np(d["v"]), np.array(pos),
                                      _np(d["sink"]))
    _check(f"ring decode hq {hq} hkv {hkv} W {W}", o, ref)
    f = synthetic.ring_decode_inputs_fp8(len(pos), hq, hkv, W, 192, 128, 96, torch.tensor(pos), DEV)
    o8 = gpu_lib.swa_sink_decode_fp8(f["q"], f["k"], f["v"], f["k_scale"], f["v_scale"], f["pos"],
                                     max(pos), layout=gpu_lib.KV_RING, sink=f["sink"], window=W)
    ref8 = oracle.swa_sink_decode_ring_fp8(_np(f["q"]), f["k"].cpu().numpy(), f["v"].cpu().numpy(),
                                           _np(f["k_scale"]), _np(f["v_scale"]), np.array(pos),
                                           _np(f["sink"]))
    _check(f"ring decode fp8 hq {hq} hkv {hkv} W {W}", o8, ref8)


def _contig_case(pos, hq=64, hkv=4, seed=90, dtype="bf16", sink=None, extra=0):
    pos = torch.as_tensor(pos, dtype=torch.int64)
    return synthetic.contiguous_decode_inputs(len(pos), hq, hkv, 192, 128, dtype, seed, pos, DEV,
                                              sink, extra_rows=extra)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_contiguous_decode(gpu_lib, dtype):
    pos = [0, 31, 32, 1000, 5000, 20000, 777]
    d = _contig_case(pos, dtype=dtype, extra=3)
    o = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], 20000,
                                layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=d["seq_offsets"],
                                window=0, rope_theta=1.0e7, rotary_fraction=0.334)
    ref = oracle.swa_sink_decode_contiguous(_np(d["q"]), _np(d["k"]), _np(d["v"]),
                                            d["seq_offsets"].cpu().numpy(), np.array(pos), None,
                                            None, rope_theta=1.0e7, rotary_fraction=0.334)
    _check(f"contiguous GA decode {dtype}", o, ref, fp32=(dtype == "f32"))


def test_contiguous_windowed_decode(gpu_lib):
    pos = [0, 100, 127, 128, 4000]
    d = _contig_case(pos, hq=64, hkv=8, seed=91, sink=(-2.0, 2.0))
    o = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], 4000,
                                layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=d["seq_offsets"],
                                sink=d["sink"], window=128)
    ref = oracle.swa_sink_decode_contiguous(_np(d["q"]), _np(d["k"]), _np(d["v"]),
                                            d["seq_offsets"].cpu().numpy(), np.array(pos),
                                            _np(d["sink"]), 128)
    _check("contiguous SWA decode", o, ref)


def test_decode_contract_violations_give_nan(gpu_lib):
    pos = [10, 500]
    d = _contig_case(pos, seed=92)
    bad = torch.tensor([10, 600], dtype=torch.int64, device=DEV)   # 600 >= rows of sequence 1
    o = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], bad, 600, layout=gpu_lib.KV_CONTIGUOUS,
                                seq_offsets=d["seq_offsets"], window=0)
    on = _np(o)
    assert np.isfinite(on[0]).all() and np.isnan(on[1]).all()
    r = _ring_case([5, 50], hq=16, hkv=2, seed=93)
    o2 = gpu_lib.swa_sink_decode(r["q"], r["k"], r["v"], r["pos"], 20, layout=gpu_lib.KV_RING,
                                 sink=r["sink"], window=128)          # 50 > max_pos
    on2 = _np(o2)
    assert np.isfinite(on2[0]).all() and np.isnan(on2[1]).all()


def test_decode_matches_prefill_row(gpu_lib):
    """Decode at p over a ring filled from a sequence equals prefill row p (both on GPU)."""
    L, W = 300, 128
    x = _prefill_case(1, L, 64, 8, "bf16", 94)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=W)
    p = L - 1
    ring_k = torch.zeros(1, W, 8, 192, dtype=torch.bfloat16, device=DEV)
    ring_v = torch.zeros(1, W, 8, 128, dtype=torch.bfloat16, device=DEV)
    for t in range(p - W + 1, p + 1):
        ring_k[0, t % W] = x["k"][0, t]
        ring_v[0, t % W] = x["v"][0, t]
    od = gpu_lib.swa_sink_decode(x["q"][:, p].contiguous(), ring_k, ring_v,
                                 torch.tensor([p], device=DEV), p, layout=gpu_lib.KV_RING,
                                 sink=x["sink"], window=W)
    assert (od.float() - o[:, p].float()).abs().max().item() <= 2e-2


def test_hybrid_decode_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["hybrid_decode_b64"]
    pos = synthetic.decode_positions(wl["B"], *wl["pos_range"], wl["seed"])
    sw = wl["swa"]
    d = synthetic.ring_decode_inputs(wl["B"], sw["hq"], sw["hkv"], sw["window"], 192, 128, "bf16",
                                     wl["seed"], pos, DEV, sw["sink_range"])
    o = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], wl["pos_range"][1],
                                layout=gpu_lib.KV_RING, sink=d["sink"], window=sw["window"])
    ref = oracle.swa_sink_decode_ring(_np(d["q"]), _np(d["k"]), _np(d["v"]), pos.numpy(),
                                      _np(d["sink"]))
    _check("hybrid decode SWA ring (all 64 sequences)", o, ref)
    del d
    ga = wl["ga"]
    c = synthetic.contiguous_decode_inputs(wl["B"], ga["hq"], ga["hkv"], 192, 128, "bf16",
                                           wl["seed"], pos, DEV, None)
    og = gpu_lib.swa_sink_decode(c["q"], c["k"], c["v"], c["pos"], wl["pos_range"][1],
                                 layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"],
                                 window=0)
    # bitwise repeatable: every tile is read only after its loads have landed
    og2 = gpu_lib.swa_sink_decode(c["q"], c["k"], c["v"], c["pos"], wl["pos_range"][1],
                                  layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"],
                                  window=0)
    assert torch.equal(og, og2)
    offs = c["seq_offsets"].cpu().numpy()
    seqs = np.array([int(pos.argmin()), int(pos.argmax()), 17])

    def loader(b):
        lo, hi = int(offs[b]), int(offs[b + 1])
        return _np(c["k"][lo:hi]), _np(c["v"][lo:hi])

    refg = oracle.swa_sink_decode_contiguous(_np(c["q"]), None, None, offs, pos.numpy(), None,
                                             None, seqs=seqs, kv_loader=loader)
    _check("hybrid decode GA contiguous (sampled sequences)", og[torch.from_numpy(seqs)], refg)


# ---------------------------------------------------------------------------
# Multi-token (MTP verification) decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,slots,hq,hkv,frac", [
    (4, 131, 64, 8, 0.334),    # the workload's shape: 32 columns, one-launch ring kernel
    (2, 140, 64, 8, 0.0),      # spare slots, 16 columns (one-launch)
    (4, 131, 32, 16, 0.334),   # G = 2: 8 columns (one-launch)
    (3, 130, 128, 8, 0.0),     # G = 16, T = 3: 48 columns: split kernel, two wavefronts per kv head
    (2, 170, 64, 8, 0.0),      # more than 160 slots: split kernel
])
def test_multi_decode_ring(gpu_lib, T, slots, hq, hkv, frac):
    pos = [0, 1, 5, 124, 125, 126, 127, 300, 131072, 262140]
    d = synthetic.multi_ring_inputs(len(pos), T, hq, hkv, slots, 192, 128, "bf16", 200 + T,
                                    torch.tensor(pos), DEV)
    o = gpu_lib.swa_sink_decode_multi(d["q"], d["k"], d["v"], d["pos"], max(pos) + T - 1,
                                      layout=gpu_lib.KV_RING, ring_slots=slots, sink=d["sink"],
                                      window=128, rope_theta=1.0e4, rotary_fraction=frac)
    ref = oracle.decode_multi_ring(_np(d["q"]), _np(d["k"]), _np(d["v"]), np.array(pos),
                                   _np(d["sink"]), 128, rope_theta=1.0e4, rotary_fraction=frac)
    _check(f"multi decode ring T={T} S={slots} {hq}/{hkv}", o, ref)


@pytest.mark.parametrize("T,hq,hkv,window,sink,dtype", [
    (4, 64, 4, 0, None, "bf16"),            # GA layer: 64 columns, two wavefronts per kv head
    (2, 64, 4, 0, None, "bf16"),            # 32 columns
    (1, 64, 4, 0, None, "bf16"),            # one query: 16 columns
    (4, 64, 8, 128, (-2.0, 2.0), "bf16"),   # windowed over the contiguous pool
    (4, 24, 3, 0, None, "bf16"),            # hkv not a multiple of 4: generic kernel
    (4, 16, 4, 64, (-1.0, 1.0), "f32"),     # fp32: generic kernel
])
def test_multi_decode_contiguous(gpu_lib, T, hq, hkv, window, sink, dtype):
    pos = [0, 29, 31, 1000, 5000, 777]
    d = synthetic.multi_contiguous_inputs(len(pos), T, hq, hkv, 192, 128, dtype, 210 + T + hkv,
                                          torch.tensor(pos), DEV, sink, extra_rows=2)
    o = gpu_lib.swa_sink_decode_multi(d["q"], d["k"], d["v"], d["pos"], max(pos) + T - 1,
                                      layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=d["seq_offsets"],
                                      sink=d["sink"], window=window, rope_theta=1.0e7,
                                      rotary_fraction=0.334)
    ref = oracle.decode_multi_contiguous(_np(d["q"]), _np(d["k"]), _np(d["v"]),
                                         d["seq_offsets"].cpu().numpy(), np.array(pos),
                                         None if sink is None else _np(d["sink"]), window or None,
                                         rope_theta=1.0e7, rotary_fraction=0.334)
    _check(f"multi decode contiguous T={T} {hq}/{hkv} W={window} {dtype}", o, ref,
           fp32=(dtype == "f32"))


def test_multi_decode_wide_falls_back(gpu_lib):
    """8 queries x 16 heads = 128 columns per kv head: past the matrix-core
    kernel's 64, the generic kernel serves the step (ring and contiguous)."""
    T, S, W = 8, 140, 128
    pos = [0, 3, 130, 5000]
    d = synthetic.multi_ring_inputs(len(pos), T, 64, 4, S, 192, 128, "bf16", 225,
                                    torch.tensor(pos), DEV)
    o = gpu_lib.swa_sink_decode_multi(d["q"], d["k"], d["v"], d["pos"], max(pos) + T - 1,
                                      layout=gpu_lib.KV_RING, ring_slots=S, sink=d["sink"],
                                      window=W, rope_theta=1.0e4, rotary_fraction=0.334)
    ref = oracle.decode_multi_ring(_np(d["q"]), _np(d["k"]), _np(d["v"]), np.array(pos),
                                   _np(d["sink"]), W, rope_theta=1.0e4, rotary_fraction=0.334)
    _check("multi decode ring T=8 G=16 (generic)", o, ref)
    c = synthetic.multi_contiguous_inputs(len(pos), T, 64, 4, 192, 128, "bf16", 226,
                                          torch.tensor(pos), DEV)
    oc = gpu_lib.swa_sink_decode_multi(c["q"], c["k"], c["v"], c["pos"], max(pos) + T - 1,
                                       layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"],
                                       window=0)
    refc = oracle.decode_multi_contiguous(_np(c["q"]), _np(c["k"]), _np(c["v"]),
                                          c["seq_offsets"].cpu().numpy(), np.array(pos))
    _check("multi decode contiguous T=8 G=16 (generic)", oc, refc)


def test_multi_decode_one_query_is_decode(gpu_lib):
    """q_len = 1 over a ring of W slots is the single-token decode."""
    pos = [0, 5, 127, 128, 1000, 262143]
    d = _ring_case(pos, seed=220)
    o1 = gpu_lib.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], max(pos),
                                 layout=gpu_lib.KV_RING, sink=d["sink"], window=128)
    om = gpu_lib.swa_sink_decode_multi(d["q"][:, None].contiguous(), d["k"], d["v"], d["pos"],
                                       max(pos), layout=gpu_lib.KV_RING, ring_slots=128,
                                       sink=d["sink"], window=128)
    _check("multi decode T=1 vs decode", om[:, 0], _np(o1))


def test_multi_decode_matches_prefill_rows(gpu_lib):
    """The verification step over a ring filled from a sequence equals the
    prefill rows of its last T tokens (both on the GPU)."""
    L, W, T, S = 300, 128, 4, 131
    x = _prefill_case(1, L, 64, 8, "bf16", 221)
    o = gpu_lib.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=W)
    p0 = L - T
    ring_k = torch.zeros(1, S, 8, 192, dtype=torch.bfloat16, device=DEV)
    ring_v = torch.zeros(1, S, 8, 128, dtype=torch.bfloat16, device=DEV)
    for j in range(p0 - W + 1, L):
        ring_k[0, j % S] = x["k"][0, j]
        ring_v[0, j % S] = x["v"][0, j]
    om = gpu_lib.swa_sink_decode_multi(x["q"][:, p0:].contiguous(), ring_k, ring_v,
                                       torch.tensor([p0], device=DEV), L - 1,
                                       layout=gpu_lib.KV_RING, ring_slots=S, sink=x["sink"],
                                       window=W)
    assert (om.float() - o[:, p0:].float()).abs().max().item() <= 2e-2


def test_multi_decode_ring_contract_violation_gives_nan(gpu_lib):
    """A sequence whose last draft position passes max_pos: NaN rows from the
    one-launch ring kernel, the other sequence untouched."""
    pos = [10, 500]
    d = synthetic.multi_ring_inputs(2, 4, 64, 8, 131, 192, 128, "bf16", 223, torch.tensor(pos), DEV)
    bad = torch.tensor([10, 501], dtype=torch.int64, device=DEV)   # 501 + 3 > max_pos
    o = gpu_lib.swa_sink_decode_multi(d["q"], d["k"], d["v"], bad, 503, layout=gpu_lib.KV_RING,
                                      ring_slots=131, sink=d["sink"], window=128)
    on = _np(o)
    assert np.isfinite(on[0]).all() and np.isnan(on[1]).all()


def test_multi_decode_contract_violations_give_nan(gpu_lib):
    pos = [10, 500]
    d = synthetic.multi_contiguous_inputs(2, 4, 64, 4, 192, 128, "bf16", 222, torch.tensor(pos), DEV)
    bad = torch.tensor([10, 501], dtype=torch.int64, device=DEV)   # 501 + 3 >= rows of sequence 1
    o = gpu_lib.swa_sink_decode_multi(d["q"], d["k"], d["v"], bad, 504,
                                      layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=d["seq_offsets"],
                                      window=0)
    on = _np(o)
    assert np.isfinite(on[0]).all() and np.isnan(on[1]).all()


@pytest.mark.parametrize("T,hq,hkv", [(2, 32, 4), (4, 32, 4)])
def test_multi_decode_long_splits(gpu_lib, T, hq, hkv):
    """Splits of at least 32 tiles run the four-stage kernels: 16 and 32
    query columns per kv head (the 64-column one is the full-size case)."""
    pos = torch.tensor([33001, 40006])
    c = synthetic.multi_contiguous_inputs(2, T, hq, hkv, 192, 128, "bf16", 231, pos, DEV, None)
    maxp = int(pos.max()) + T - 1
    o = gpu_lib.swa_sink_decode_multi(c["q"], c["k"], c["v"], c["pos"], maxp,
                                      layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"],
                                      window=0)
    offs = c["seq_offsets"].cpu().numpy()
    for b in range(2):
        lo, hi = int(offs[b]), int(offs[b + 1])
        refb = oracle.decode_multi_contiguous(_np(c["q"][b:b + 1]), _np(c["k"][lo:hi]),
                                              _np(c["v"][lo:hi]), np.array([0, hi - lo]),
                                              pos.numpy()[b:b + 1])
        _check(f"multi decode long splits T={T} hq={hq} (sequence {b})", o[b:b + 1], refb)


def test_mtp_decode_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["mtp_decode_b64_t4"]
    T = wl["T"]
    pos = synthetic.decode_positions(wl["B"], *wl["pos_range"], wl["seed"])
    maxp = wl["pos_range"][1] + T - 1
    sw, ga = wl["swa"], wl["ga"]
    d = synthetic.multi_ring_inputs(wl["B"], T, sw["hq"], sw["hkv"], sw["slots"], 192, 128, "bf16",
                                    wl["seed"], pos, DEV, sw["sink_range"])
    o = gpu_lib.swa_sink_decode_multi(d["q"], d["k"], d["v"], d["pos"], maxp,
                                      layout=gpu_lib.KV_RING, ring_slots=sw["slots"],
                                      sink=d["sink"], window=sw["window"])
    ref = oracle.decode_multi_ring(_np(d["q"]), _np(d["k"]), _np(d["v"]), pos.numpy(),
                                   _np(d["sink"]), sw["window"])
    _check("MTP decode SWA ring (all 64 sequences)", o, ref)
    del d
    c = synthetic.multi_contiguous_inputs(wl["B"], T, ga["hq"], ga["hkv"], 192, 128, "bf16",
                                          wl["seed"], pos, DEV, None)
    og = gpu_lib.swa_sink_decode_multi(c["q"], c["k"], c["v"], c["pos"], maxp,
                                       layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"],
                                       window=0)
    offs = c["seq_offsets"].cpu().numpy()
    seqs = [int(pos.argmin()), int(pos.argmax()), 17]
    for b in seqs:
        lo, hi = int(offs[b]), int(offs[b + 1])
        refb = oracle.decode_multi_contiguous(_np(c["q"][b:b + 1]), _np(c["k"][lo:hi]),
                                              _np(c["v"][lo:hi]), np.array([0, hi - lo]),
                                              pos.numpy()[b:b + 1])
        _check(f"MTP decode GA contiguous (sequence {b})", og[b:b + 1], refb)


# ---------------------------------------------------------------------------
# Decode over FP8 (E4M3) caches with per-kv-head scales
# ---------------------------------------------------------------------------

def _codes(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("qdtype", ["bf16", "f32"])
def test_ring_decode_fp8(gpu_lib, qdtype):
    """bf16 q: matrix-core kernel; fp32 q: generic kernel."""
    pos = [0, 1, 5, 126, 127, 128, 1000, 131072, 262143, 77777]
    d = synthetic.ring_decode_inputs_fp8(len(pos), 64, 8, 128, 192, 128, 180,
                                         torch.tensor(pos), DEV, qdtype=qdtype)
    o = gpu_lib.swa_sink_decode_fp8(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], d["pos"],
                                    max(pos), layout=gpu_lib.KV_RING, sink=d["sink"], window=128,
                                    rope_theta=1.0e4, rotary_fraction=0.334)
    ref = oracle.swa_sink_decode_ring_fp8(_np(d["q"]), _codes(d["k"]), _codes(d["v"]),
                                          _np(d["k_scale"]), _np(d["v_scale"]), np.array(pos),
                                          _np(d["sink"]), rope_theta=1.0e4, rotary_fraction=0.334)
    _check(f"ring decode fp8 cache, q {qdtype}", o, ref, fp32=(qdtype == "f32"))


@pytest.mark.parametrize("hq,hkv,window,sink,qdtype", [
    (64, 4, 0, None, "bf16"),            # GA layer: matrix-core kernel
    (64, 8, 128, (-2.0, 2.0), "bf16"),   # windowed SWA layer over the contiguous pool
    (24, 3, 0, None, "bf16"),            # hkv not a multiple of 4: generic kernel
    (64, 2, 0, None, "bf16"),            # G = 32: generic kernel
    (16, 4, 64, (-1.0, 1.0), "f32"),     # fp32 q / o: generic kernel
])
def test_contiguous_decode_fp8(gpu_lib, hq, hkv, window, sink, qdtype):
    pos = [0, 31, 32, 1000, 5000, 777]
    d = synthetic.contiguous_decode_inputs_fp8(len(pos), hq, hkv, 192, 128, 190 + hq + hkv,
                                               torch.tensor(pos), DEV, sink, extra_rows=2,
                                               qdtype=qdtype)
    o = gpu_lib.swa_sink_decode_fp8(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], d["pos"],
                                    5000, layout=gpu_lib.KV_CONTIGUOUS,
                                    seq_offsets=d["seq_offsets"], sink=d["sink"], window=window,
                                    rope_theta=1.0e7, rotary_fraction=0.334)
    ref = oracle.swa_sink_decode_contiguous_fp8(
        _np(d["q"]), _codes(d["k"]), _codes(d["v"]), _np(d["k_scale"]), _np(d["v_scale"]),
        d["seq_offsets"].cpu().numpy(), np.array(pos), None if sink is None else _np(d["sink"]),
        window or None, rope_theta=1.0e7, rotary_fraction=0.334)
    _check(f"contiguous decode fp8 {hq}/{hkv} W={window} q {qdtype}", o, ref,
           fp32=(qdtype == "f32"))


def test_decode_fp8_contract_violations_give_nan(gpu_lib):
    pos = [10, 500]
    d = synthetic.contiguous_decode_inputs_fp8(2, 64, 4, 192, 128, 195, torch.tensor(pos), DEV)
    bad = torch.tensor([10, 600], dtype=torch.int64, device=DEV)
    o = gpu_lib.swa_sink_decode_fp8(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], bad, 600,
                                    layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=d["seq_offsets"],
                                    window=0)
    on = _np(o)
    assert np.isfinite(on[0]).all() and np.isnan(on[1]).all()


def test_hybrid_decode_fp8_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["hybrid_decode_fp8_b64"]
    pos = synthetic.decode_positions(wl["B"], *wl["pos_range"], wl["seed"])
    sw, ga = wl["swa"], wl["ga"]
    d = synthetic.ring_decode_inputs_fp8(wl["B"], sw["hq"], sw["hkv"], sw["window"], 192, 128,
                                         wl["seed"], pos, DEV, sw["sink_range"], wl["scale_range"])
    o = gpu_lib.swa_sink_decode_fp8(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], d["pos"],
                                    wl["pos_range"][1], layout=gpu_lib.KV_RING, sink=d["sink"],
                                    window=sw["window"])
    ref = oracle.swa_sink_decode_ring_fp8(_np(d["q"]), _codes(d["k"]), _codes(d["v"]),
                                          _np(d["k_scale"]), _np(d["v_scale"]), pos.numpy(),
                                          _np(d["sink"]))
    _check("hybrid decode fp8 SWA ring (all 64 sequences)", o, ref)
    del d
    c = synthetic.contiguous_decode_inputs_fp8(wl["B"], ga["hq"], ga["hkv"], 192, 128, wl["seed"],
                                               pos, DEV, None, scale_range=wl["scale_range"])
    args = (c["q"], c["k"], c["v"], c["k_scale"], c["v_scale"], c["pos"], wl["pos_range"][1])
    og = gpu_lib.swa_sink_decode_fp8(*args, layout=gpu_lib.KV_CONTIGUOUS,
                                     seq_offsets=c["seq_offsets"], window=0)
    og2 = gpu_lib.swa_sink_decode_fp8(*args, layout=gpu_lib.KV_CONTIGUOUS,
                                      seq_offsets=c["seq_offsets"], window=0)
    assert torch.equal(og, og2)
    offs = c["seq_offsets"].cpu().numpy()
    seqs = np.array([int(pos.argmin()), int(pos.argmax()), 17])

    def loader(b):
        lo, hi = int(offs[b]), int(offs[b + 1])
        return _codes(c["k"][lo:hi]), _codes(c["v"][lo:hi])

    refg = oracle.swa_sink_decode_contiguous_fp8(_np(c["q"]), None, None, _np(c["k_scale"]),
                                                 _np(c["v_scale"]), offs, pos.numpy(), None, None,
                                                 seqs=seqs, kv_loader=loader)
    _check("hybrid decode fp8 GA contiguous (sampled sequences)", og[torch.from_numpy(seqs)], refg)


# ---------------------------------------------------------------------------
# Sparse
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,hq,hkv,recent,max_sel,frac", [
    (1500, 64, 4, 128, 1024, 0.0),    # the workload's shape at a size the oracle covers
    (400, 16, 2, 32, 64, 0.334),      # sampling at small n, RoPE on
    (300, 8, 8, 16, 20, 0.0),         # G = 1
])
def test_sparse_bf16(gpu_lib, n, hq, hkv, recent, max_sel, frac):
    x = synthetic.sparse_inputs(1, n, hq, hkv, 192, 128, "bf16", 100 + n, recent, max_sel, DEV)
    o = gpu_lib.sparse_sink_attn(x["q"], x["k"], x["v"], x["sel_idx"], x["sel_count"], x["sink"],
                                 recent_window=recent, rope_theta=1.0e4, rotary_fraction=frac)
    q, k, v, s = _host(x)
    ref = oracle.sparse_sink_attn(q, k, v, x["sel_idx"].cpu().numpy(), x["sel_count"].cpu().numpy(),
                                  s, recent=recent, rope_theta=1.0e4, rotary_fraction=frac)
    _check(f"sparse bf16 n={n} {hq}/{hkv} recent={recent} sel={max_sel}", o, ref)


def test_sparse_fp32_and_invalid_entries(gpu_lib):
    n, recent = 200, 16
    x = synthetic.sparse_inputs(1, n, 4, 2, 192, 128, "f32", 110, recent, 24, DEV)
    idx = x["sel_idx"].clone()
    idx[0, 150, 0, 0] = 10_000        # out of range: skipped by contract
    idx[0, 151, 1, 3] = 151           # inside the recent window: skipped
    o = gpu_lib.sparse_sink_attn(x["q"], x["k"], x["v"], idx, x["sel_count"], x["sink"],
                                 recent_window=recent)
    q, k, v, s = _host(x)
    clean = x["sel_idx"].cpu().numpy().copy()
    cnt = x["sel_count"].cpu().numpy().copy()
    for (i, g, j) in ((150, 0, 0), (151, 1, 3)):
        row = [t for t in clean[0, i, g, :cnt[0, i, g]] if t != clean[0, i, g, j]]
        clean[0, i, g, :len(row)] = row
        cnt[0, i, g] = len(row)
    ref = oracle.sparse_sink_attn(q, k, v, clean, cnt, s, recent=recent)
    _check("sparse fp32 with skipped entries", o, ref, fp32=True)
    # same through the bf16 matrix-core kernel
    xb = {t: (x[t].to(torch.bfloat16) if t in "qkv" else x[t]) for t in x}
    ob = gpu_lib.sparse_sink_attn(xb["q"], xb["k"], xb["v"], idx, x["sel_count"], x["sink"],
                                  recent_window=recent)
    refb = oracle.sparse_sink_attn(*(_np(xb[t]) for t in "qkv"), clean, cnt, s, recent=recent)
    _check("sparse bf16 with skipped entries", ob, refb)


def test_sparse_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["sparse_prefill_n65536"]
    x = synthetic.sparse_inputs(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, "bf16", wl["seed"],
                                wl["recent"], wl["max_sel"], DEV, wl["sink_range"])
    o = gpu_lib.sparse_sink_attn(x["q"], x["k"], x["v"], x["sel_idx"], x["sel_count"], x["sink"],
                                 recent_window=wl["recent"])
    rows = _sample_rows(wl["n"], 120)
    ridx = torch.from_numpy(rows).to(DEV)
    ref = oracle.sparse_rows(_np(x["q"][:, ridx]), _np(x["k"]), _np(x["v"]),
                             x["sel_idx"][:, ridx].cpu().numpy(), x["sel_count"][:, ridx].cpu().numpy(),
                             rows, _np(x["sink"]), recent=wl["recent"], restricted=True)
    _check("sparse full size (sampled rows)", o[:, ridx], ref)


# ---------------------------------------------------------------------------
# Sparse attention over FP8 (E4M3) K/V
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,hq,hkv,recent,max_sel,frac,qdtype", [
    (1500, 64, 4, 128, 1024, 0.0, "bf16"),   # the workload's shape: matrix-core kernel
    (400, 16, 2, 32, 64, 0.334, "bf16"),     # RoPE on the key values (rotated copy from codes)
    (300, 64, 2, 16, 20, 0.0, "bf16"),       # G = 32: generic kernel
    (200, 8, 2, 16, 24, 0.334, "f32"),       # fp32 q / o: generic kernel with RoPE
])
def test_sparse_fp8(gpu_lib, n, hq, hkv, recent, max_sel, frac, qdtype):
    x = synthetic.sparse_inputs_fp8(1, n, hq, hkv, 192, 128, 130 + n, recent, max_sel, DEV,
                                    qdtype=qdtype)
    o = gpu_lib.sparse_sink_attn_fp8(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"],
                                     x["sel_idx"], x["sel_count"], x["sink"], recent_window=recent,
                                     rope_theta=1.0e4, rotary_fraction=frac, pos_offset=9)
    ref = oracle.sparse_rows_fp8(_np(x["q"]), _codes(x["k"]), _codes(x["v"]), _np(x["k_scale"]),
                                 _np(x["v_scale"]), x["sel_idx"].cpu().numpy(),
                                 x["sel_count"].cpu().numpy(), np.arange(n), _np(x["sink"]),
                                 recent=recent, rope_theta=1.0e4, rotary_fraction=frac,
                                 pos_offset=9)
    _check(f"sparse fp8 n={n} {hq}/{hkv} recent={recent} sel={max_sel} q {qdtype}", o, ref,
           fp32=(qdtype == "f32"))


def test_sparse_fp8_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["sparse_prefill_n65536"]
    x = synthetic.sparse_inputs_fp8(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, wl["seed"],
                                    wl["recent"], wl["max_sel"], DEV, wl["sink_range"])
    o = gpu_lib.sparse_sink_attn_fp8(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"],
                                     x["sel_idx"], x["sel_count"], x["sink"],
                                     recent_window=wl["recent"])
    rows = _sample_rows(wl["n"], 121)
    ridx = torch.from_numpy(rows).to(DEV)
    ref = oracle.sparse_rows_fp8(_np(x["q"][:, ridx]), _codes(x["k"]), _codes(x["v"]),
                                 _np(x["k_scale"]), _np(x["v_scale"]),
                                 x["sel_idx"][:, ridx].cpu().numpy(),
                                 x["sel_count"][:, ridx].cpu().numpy(), rows, _np(x["sink"]),
                                 recent=wl["recent"], restricted=True)
    _check("sparse fp8 full size (sampled rows)", o[:, ridx], ref)


# ---------------------------------------------------------------------------
# Appending new tokens to a decode cache
# ---------------------------------------------------------------------------

def _append_case(B, T, hkv, rows, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kn = torch.randn(B, T, hkv, 192, generator=g).to(tdt).to(DEV)
    vn = torch.randn(B, T, hkv, 128, generator=g).to(tdt).to(DEV)
    kc = torch.randn(rows, hkv, 192, generator=g).to(tdt).to(DEV)
    vc = torch.randn(rows, hkv, 128, generator=g).to(tdt).to(DEV)
    return kn, vn, kc, vc


@pytest.mark.parametrize("dtype,frac", [("bf16", 0.334), ("f32", 0.334), ("bf16", 0.0)])
def test_append_ring_exact(gpu_lib, dtype, frac):
    """Every byte of the ring after the append equals the oracle's."""
    B, T, hkv, S = 5, 4, 8, 131
    pos = [0, 2, 127, 130, 262140]
    kn, vn, kc, vc = _append_case(B, T, hkv, B * S, dtype, 230)
    kc, vc = kc.view(B, S, hkv, 192), vc.view(B, S, hkv, 128)
    kref, vref = oracle.kv_append(_np(kc), _np(vc), _np(kn), _np(vn), np.array(pos), 1.0e4, frac,
                                  ring_slots=S, store=dtype)
    gpu_lib.kv_cache_append(kn, vn, kc, vc, torch.tensor(pos, device=DEV), max(pos) + T - 1,
                            layout=gpu_lib.KV_RING, ring_slots=S, rope_theta=1.0e4,
                            rotary_fraction=frac)
    assert np.array_equal(_np(kc), kref) and np.array_equal(_np(vc), vref)


@pytest.mark.parametrize("layout", ["ring", "contiguous"])
def test_append_e4m3_exact(gpu_lib, layout):
    """E4M3 codes written by the append are the oracle's codes, bit for bit."""
    B, T, hkv = 4, 3, 4
    pos = [0, 9, 500, 131071]
    kn, vn, _, _ = _append_case(B, T, hkv, 1, "bf16", 231)
    ks, vs = synthetic.kv_scales(hkv, 0.02, 0.04, 232, DEV)
    if layout == "ring":
        S = 130
        kc = torch.zeros(B, S, hkv, 192, dtype=torch.uint8, device=DEV)
        vc = torch.zeros(B, S, hkv, 128, dtype=torch.uint8, device=DEV)
        kw = dict(layout=gpu_lib.KV_RING, ring_slots=S)
        okw = dict(ring_slots=S)
    else:
        lens = torch.tensor(pos) + T + 1
        offs = torch.zeros(B + 1, dtype=torch.int64)
        offs[1:] = torch.cumsum(lens, 0)
        kc = torch.zeros(int(offs[-1]), hkv, 192, dtype=torch.uint8, device=DEV)
        vc = torch.zeros(int(offs[-1]), hkv, 128, dtype=torch.uint8, device=DEV)
        kw = dict(layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=offs.to(DEV))
        okw = dict(seq_offsets=offs.numpy())
    kref, vref = oracle.kv_append(_codes(kc), _codes(vc), _np(kn), _np(vn), np.array(pos), 1.0e4,
                                  0.334, k_scale=_np(ks), v_scale=_np(vs), store="e4m3", **okw)
    gpu_lib.kv_cache_append(kn, vn, kc, vc, torch.tensor(pos, device=DEV), max(pos) + T - 1,
                            rope_theta=1.0e4, rotary_fraction=0.334, k_scale=ks, v_scale=vs, **kw)
    assert np.array_equal(_codes(kc), kref) and np.array_equal(_codes(vc), vref)


def test_append_contract_violations_write_nothing(gpu_lib):
    B, T, hkv = 2, 2, 4
    lens = torch.tensor([10, 10])
    offs = torch.tensor([0, 10, 20], dtype=torch.int64)
    kn, vn, kc, vc = _append_case(B, T, hkv, 20, "bf16", 233)
    k0, v0 = kc.clone(), vc.clone()
    bad = torch.tensor([9, -1], device=DEV)          # 9 + 1 >= 10 rows; -1 negative
    gpu_lib.kv_cache_append(kn, vn, kc, vc, bad, 10, layout=gpu_lib.KV_CONTIGUOUS,
                            seq_offsets=offs.to(DEV), rope_theta=1.0e7, rotary_fraction=0.334)
    # sequence 0: position 9 is written, position 10 is not; sequence 1:
    # position -1 is not, position 0 (row 10) is
    changed = (kc != k0).any(dim=(1, 2)).cpu().numpy()
    vchanged = (vc != v0).any(dim=(1, 2)).cpu().numpy()
    assert list(np.nonzero(changed)[0]) == [9, 10] and list(np.nonzero(vchanged)[0]) == [9, 10]
    assert int(lens.sum()) == 20


def test_append_then_multi_decode(gpu_lib):
    """A verification step end to end on the GPU: append the 4 new tokens, then
    decode them; the oracle appends and decodes the same way."""
    B, T, hkv, hq, S, W = 3, 4, 8, 64, 131, 128
    pos = [5, 126, 70000]
    kn, vn, kc, vc = _append_case(B, T, hkv, B * S, "bf16", 234)
    kc, vc = kc.view(B, S, hkv, 192), vc.view(B, S, hkv, 128)
    q = synthetic.normal((B, T, hq, 192), 235, DEV, "bf16")
    sink = synthetic.uniform((hq,), -2.0, 2.0, 236, DEV)
    kref, vref = oracle.kv_append(_np(kc), _np(vc), _np(kn), _np(vn), np.array(pos), 1.0e4, 0.334,
                                  ring_slots=S, store="bf16")
    pt = torch.tensor(pos, device=DEV)
    gpu_lib.kv_cache_append(kn, vn, kc, vc, pt, max(pos) + T - 1, layout=gpu_lib.KV_RING,
                            ring_slots=S, rope_theta=1.0e4, rotary_fraction=0.334)
    o = gpu_lib.swa_sink_decode_multi(q, kc, vc, pt, max(pos) + T - 1, layout=gpu_lib.KV_RING,
                                      ring_slots=S, sink=sink, window=W, rope_theta=1.0e4,
                                      rotary_fraction=0.334)
    ref = oracle.decode_multi_ring(_np(q), kref, vref, np.array(pos), _np(sink), W,
                                   rope_theta=1.0e4, rotary_fraction=0.334)
    _check("append + multi-token decode", o, ref)


# ---------------------------------------------------------------------------
# Token selection for the sparse layers
# ---------------------------------------------------------------------------

def _check_selection(name, idx, cnt, q, k, rows, recent, K, frac=0.0, theta=1.0e7, tol=1e-3):
    """Counts exact; lists ascending, distinct, in range, -1 padded; the selected
    set valid against the oracle's float64 importances (no unselected candidate
    above a selected one by more than `tol` relative) and equal to the oracle's
    selection except where importances tie within `tol`."""
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    B, hkv = idx.shape[0], idx.shape[2]
    worst, differ, total = 0.0, 0, 0
    for b in range(B):
        for t, i in enumerate(rows):
            for g in range(hkv):
                ncand = max(0, int(i) - recent + 1)
                want = min(K, ncand)
                assert cnt[b, t, g] == want, (name, b, i, g, cnt[b, t, g], want)
                sel = idx[b, t, g, :want]
                assert (idx[b, t, g, want:] == -1).all()
                assert (np.diff(sel) > 0).all() and (sel >= 0).all() and (sel < max(ncand, 1)).all()
                if want == ncand or want == 0:
                    continue
                imp = oracle.selection_importance(q, k, b, int(i), g, recent, rope_theta=theta,
                                                  rotary_fraction=frac)
                mask = np.zeros(ncand, bool)
                mask[sel] = True
                lo, hi = imp[mask].min(), imp[~mask].max()
                worst = max(worst, (hi - lo) / max(lo, 1e-300))
                ref = np.sort(np.lexsort((np.arange(ncand), -imp))[:want])
                differ += len(np.setdiff1d(sel, ref))
                total += want
    print(f"[parity] {name}: worst inversion {worst:.2e}, {differ}/{total} picks differ", flush=True)
    assert worst <= tol, (name, worst)
    if total:
        assert differ <= max(2, 0.01 * total), (name, differ, total)


@pytest.mark.parametrize("B,n,hkv,recent,K,frac", [
    (1, 300, 4, 16, 40, 0.0),       # the workload's heads at a size the oracle covers
    (2, 211, 2, 32, 64, 0.334),     # ragged rows, RoPE (base 1e7) on both q and k
    (1, 150, 1, 8, 500, 0.0),       # every candidate fits: no ranking
    (1, 64, 2, 100, 8, 0.0),        # window wider than most rows: few or no candidates
])
def test_select_tokens(gpu_lib, B, n, hkv, recent, K, frac):
    hq = 16 * hkv
    x = synthetic.prefill_inputs(B, n, hq, hkv, 192, 128, "bf16", 240 + n, DEV, None)
    idx, cnt = gpu_lib.sparse_select_tokens(x["q"], x["k"], max_sel=K, recent_window=recent,
                                            rope_theta=1.0e7, rotary_fraction=frac)
    # with RoPE the rotated dims enter the products as bf16: the floor that
    # alone causes (tests/test_tolerance_floor.py) sets the bar
    _check_selection(f"select B={B} n={n} hkv={hkv} recent={recent} K={K}", idx, cnt, _np(x["q"]),
                     _np(x["k"]), np.arange(n), recent, K, frac, tol=3e-3 if frac > 0 else 1e-3)


def test_select_tokens_ties_and_empty(gpu_lib):
    """Keys equal to each other tie exactly: the lower positions win; max_sel 0
    keeps nothing."""
    n, hkv, hq = 48, 1, 16
    x = synthetic.prefill_inputs(1, n, hq, hkv, 192, 128, "bf16", 250, DEV, None)
    k = x["k"].clone()
    for j in (3, 9, 10, 20, 30):
        k[0, j] = k[0, 40]
    q = x["q"].clone()
    q[0, 47] = (k[0, 40] * 2).to(torch.bfloat16).expand(hq, 192)
    idx, cnt = gpu_lib.sparse_select_tokens(q, k, max_sel=3, recent_window=4)
    assert cnt[0, 47, 0].item() == 3
    assert idx[0, 47, 0].tolist() == [3, 9, 10]
    idx0, cnt0 = gpu_lib.sparse_select_tokens(q, k, max_sel=0, recent_window=4)
    assert (cnt0 == 0).all() and idx0.numel() == 0


def test_select_tokens_all_tied(gpu_lib):
    """q = 0 gives every key of a row the same importance, so every row keeps
    its lowest candidates: the tie ranks run across lanes and 256-key chunks,
    and max_sel = 701 cuts the ties inside one lane's group of four.  Rows
    with up to 4096 candidates rank a compact list; longer rows (all tied in
    one bin) take the two-read path."""
    B, n, hkv, K, recent = 1, 6000, 2, 701, 16
    x = synthetic.prefill_inputs(B, n, 16 * hkv, hkv, 192, 128, "bf16", 251, DEV, None)
    q = torch.zeros_like(x["q"])
    idx, cnt = gpu_lib.sparse_select_tokens(q, x["k"], max_sel=K, recent_window=recent)
    i = np.arange(n)
    want_cnt = np.minimum(K, np.maximum(0, i - recent + 1))
    got_cnt = cnt[0].cpu().numpy()
    assert (got_cnt == want_cnt[:, None]).all()
    got = idx[0].cpu().numpy()
    want = np.where(np.arange(K)[None, :] < want_cnt[:, None], np.arange(K)[None, :], -1)
    assert (got == want[:, None, :]).all()


def test_select_then_sparse(gpu_lib):
    """The lists feed sparse attention directly (the reuse of section 4)."""
    n, hkv, hq, recent, K = 400, 2, 32, 32, 48
    x = synthetic.prefill_inputs(1, n, hq, hkv, 192, 128, "bf16", 251, DEV)
    idx, cnt = gpu_lib.sparse_select_tokens(x["q"], x["k"], max_sel=K, recent_window=recent)
    o = gpu_lib.sparse_sink_attn(x["q"], x["k"], x["v"], idx, cnt, x["sink"], recent_window=recent)
    q, k, v, s = _host(x)
    ref = oracle.sparse_sink_attn(q, k, v, idx.cpu().numpy(), cnt.cpu().numpy(), s, recent=recent)
    _check("sparse attention over selected tokens", o, ref)


def test_select_tokens_full_size(gpu_lib):
    wl = synthetic.WORKLOADS["sparse_prefill_n65536"]
    x = synthetic.prefill_inputs(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, "bf16", wl["seed"], DEV,
                                 None)
    idx, cnt = gpu_lib.sparse_select_tokens(x["q"], x["k"], max_sel=wl["max_sel"],
                                            recent_window=wl["recent"])
    rows = np.array([0, 127, 128, 1151, 1152, 1153, 5000, 33333, 65535])
    ridx = torch.from_numpy(rows).to(DEV)
    _check_selection("select full size (sampled rows)", idx[:, ridx], cnt[:, ridx], _np(x["q"]),
                     _np(x["k"]), rows, wl["recent"], wl["max_sel"])
