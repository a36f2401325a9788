"""Workload shapes and seeded generators.

Recipe (the same for every workload):
  * every tensor draws from its own torch.Generator seeded with
    tensor_seed(base, tensor_id[, part]) so that any tensor can be rebuilt
    alone;
  * q, k, v ~ N(0, 1) drawn in float32 and, for bf16 workloads, cast to
    bfloat16 with round-to-nearest-even;
  * per-head sinks ~ U(lo, hi) in float32;
  * decode positions ~ U{lo .. hi} drawn on the host;
  * FP8 caches: per-kv-head scales ~ U(lo, hi) in float32, K and V drawn
    as above in float32, divided by their head's scale and cast to E4M3
    codes by torch (round-to-nearest-even; magnitudes stay below 448);
  * sparse selections: for query i and kv head g, `avail = max(0, i - recent)`
    candidates [0, avail); all of them when avail <= max_sel, otherwise
    max_sel distinct ones drawn uniformly (Floyd's sampling), sorted
    ascending and padded with -1.

Shapes follow the pages: window 128, 64 query heads with 8 (SWA) or 4 (GA)
kv heads, head dims 192 / 128, RoPE bases 1e4 (SWA) / 1e7 (GA) on the first
64 dims ("39 SWA + 9 GA layers: MiMo-V2.6-Flash hybrid SWA", pwwt.cn,
sections 3-5), 128 recent + 1024 selected tokens ("MiMo-V3 HySparse2",
aideepthink.cn, section 4).
"""

import torch

# Tensor ids inside one workload seed space.
TID_Q, TID_K, TID_V, TID_SINK, TID_POS, TID_SEL = 1, 2, 3, 4, 5, 6
TID_K_GA, TID_V_GA, TID_Q_GA = 12, 13, 11
TID_KSCALE, TID_VSCALE = 21, 22

WORKLOADS = {
    # Tiny fp32 SWA+sink prefill, no RoPE; also run with sink = -inf and W = 512.
    "tiny_fp32_swa_n512": dict(kind="prefill", seed=1, B=1, n=512, hq=2, hkv=1, d_qk=192,
                               d_v=128, window=128, dtype="f32", sink_range=(-3.0, 3.0),
                               rope_theta=10000.0, rotary_fraction=0.0),
    # SWA layer prefill: n = 32768, 64 q / 8 kv heads, W = 128, RoPE 1e4 on 64 dims, sink.
    "swa_prefill_n32768": dict(kind="prefill", seed=2, B=1, n=32768, hq=64, hkv=8, d_qk=192,
                               d_v=128, window=128, dtype="bf16", sink_range=(-2.0, 2.0),
                               rope_theta=1.0e4, rotary_fraction=0.334),
    # GA layer prefill: n = 32768, 64 q / 4 kv heads, full causal, no sink, RoPE 1e7.
    "ga_prefill_n32768": dict(kind="prefill", seed=3, B=1, n=32768, hq=64, hkv=4, d_qk=192,
                              d_v=128, window=0, dtype="bf16", sink_range=None,
                              rope_theta=1.0e7, rotary_fraction=0.334),
    # Chunked prefill ("MiMo v2.5 inference optimisation", youngju.dev, KV-cache
    # restructuring and scheduling: fixed 16K-token chunks, prefixes up to 1M
    # tokens): one 16384-token chunk behind a 2^20-token cached prefix (SWA
    # layer) and behind a 114688-token prefix (GA layer, kv_len 131072).
    "swa_chunk_q16384_prefix1048576": dict(kind="chunk", seed=6, B=1, q_len=16384,
                                           kv_len=16384 + 1048576, hq=64, hkv=8, d_qk=192,
                                           d_v=128, window=128, dtype="bf16",
                                           sink_range=(-2.0, 2.0), rope_theta=1.0e4,
                                           rotary_fraction=0.334),
    "ga_chunk_q16384_prefix114688": dict(kind="chunk", seed=7, B=1, q_len=16384,
                                         kv_len=131072, hq=64, hkv=4, d_qk=192, d_v=128,
                                         window=0, dtype="bf16", sink_range=None,
                                         rope_theta=1.0e7, rotary_fraction=0.334),
    # Hybrid decode step: 64 sequences, one token each at p in [131072, 262143].
    "hybrid_decode_b64": dict(kind="decode", seed=4, B=64, pos_range=(131072, 262143),
                              d_qk=192, d_v=128, dtype="bf16",
                              swa=dict(hq=64, hkv=8, window=128, sink_range=(-2.0, 2.0)),
                              ga=dict(hq=64, hkv=4, window=0, sink_range=None)),
    # Multi-token (MTP verification) decode step: 64 sequences, the last accepted
    # token plus 3 drafts each ("visual reading: MiMo MTP/SWA, not MLA",
    # syt-nju.github.io: 3 MTP blocks), first position in [131072, 262140];
    # the SWA ring holds W + 3 = 131 slots.
    "mtp_decode_b64_t4": dict(kind="decode_multi", seed=9, B=64, T=4, pos_range=(131072, 262140),
                              d_qk=192, d_v=128, dtype="bf16",
                              swa=dict(hq=64, hkv=8, window=128, slots=131,
                                       sink_range=(-2.0, 2.0)),
                              ga=dict(hq=64, hkv=4, window=0, sink_range=None)),
    # The same decode step over FP8 (E4M3) caches with per-kv-head scales.
    "hybrid_decode_fp8_b64": dict(kind="decode_fp8", seed=8, B=64, pos_range=(131072, 262143),
                                  d_qk=192, d_v=128, dtype="bf16", scale_range=(0.02, 0.04),
                                  swa=dict(hq=64, hkv=8, window=128, sink_range=(-2.0, 2.0)),
                                  ga=dict(hq=64, hkv=4, window=0, sink_range=None)),
    # Token-level sparse prefill: n = 65536, 64 q / 4 kv heads, 128 recent + <= 1024 selected.
    "sparse_prefill_n65536": dict(kind="sparse", seed=5, B=1, n=65536, hq=64, hkv=4, d_qk=192,
                                  d_v=128, recent=128, max_sel=1024, dtype="bf16",
                                  sink_range=(-2.0, 2.0), rope_theta=1.0e4, rotary_fraction=0.0),
}


def tensor_seed(base, tensor_id, part=0):
    """Seed of one tensor (or one part of it, e.g. one sequence of a cache)."""
    return (int(base) * 1000 + int(tensor_id)) * 100003 + int(part)


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _torch_dtype(dtype):
    if dtype in ("f32", torch.float32):
        return torch.float32
    if dtype in ("bf16", torch.bfloat16):
        return torch.bfloat16
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(shape, seed, device="cpu", dtype="f32", out=None):
    """N(0,1) drawn in float32, then cast (round-to-nearest-even) to `dtype`."""
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if out is not None:
        out.copy_(x)
        return out
    return x.to(_torch_dtype(dtype))


def uniform(shape, lo, hi, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def prefill_inputs(B, n, hq, hkv, d_qk, d_v, dtype, seed, device="cpu", sink_range=(-2.0, 2.0)):
    """q [B,n,Hq,d_qk], k [B,n,Hkv,d_qk], v [B,n,Hkv,d_v] and sink [Hq] (or None)."""
    q = normal((B, n, hq, d_qk), tensor_seed(seed, TID_Q), device, dtype)
    k = normal((B, n, hkv, d_qk), tensor_seed(seed, TID_K), device, dtype)
    v = normal((B, n, hkv, d_v), tensor_seed(seed, TID_V), device, dtype)
    sink = None
    if sink_range is not None:
        sink = uniform((hq,), sink_range[0], sink_range[1], tensor_seed(seed, TID_SINK), device)
    return dict(q=q, k=k, v=v, sink=sink)


def chunk_inputs(B, q_len, kv_len, hq, hkv, d_qk, d_v, dtype, seed, device="cpu",
                 sink_range=(-2.0, 2.0)):
    """A prefill chunk: q [B,q_len,Hq,d_qk] for the last q_len positions, and
    k [B,kv_len,Hkv,d_qk], v [B,kv_len,Hkv,d_v] for the whole sequence (the
    cached prefix followed by the chunk), sink [Hq] (or None)."""
    q = normal((B, q_len, hq, d_qk), tensor_seed(seed, TID_Q), device, dtype)
    k = normal((B, kv_len, hkv, d_qk), tensor_seed(seed, TID_K), device, dtype)
    v = normal((B, kv_len, hkv, d_v), tensor_seed(seed, TID_V), device, dtype)
    sink = None
    if sink_range is not None:
        sink = uniform((hq,), sink_range[0], sink_range[1], tensor_seed(seed, TID_SINK), device)
    return dict(q=q, k=k, v=v, sink=sink)


def decode_positions(B, lo, hi, seed):
    """Host int64 positions p ~ U{lo .. hi}."""
    g = _gen(tensor_seed(seed, TID_POS), "cpu")
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)


def ring_decode_inputs(B, hq, hkv, window, d_qk, d_v, dtype, seed, pos, device="cpu",
                       sink_range=(-2.0, 2.0)):
    """q [B,Hq,d_qk] and a W-slot ring cache k [B,W,Hkv,d_qk], v [B,W,Hkv,d_v]."""
    q = normal((B, hq, d_qk), tensor_seed(seed, TID_Q), device, dtype)
    k = normal((B, window, hkv, d_qk), tensor_seed(seed, TID_K), device, dtype)
    v = normal((B, window, hkv, d_v), tensor_seed(seed, TID_V), device, dtype)
    sink = None
    if sink_range is not None:
        sink = uniform((hq,), sink_range[0], sink_range[1], tensor_seed(seed, TID_SINK), device)
    return dict(q=q, k=k, v=v, sink=sink, pos=pos.to(device))


def contiguous_decode_inputs(B, hq, hkv, d_qk, d_v, dtype, seed, pos, device="cpu",
                             sink_range=None, extra_rows=0):
    """q [B,Hq,d_qk] and a packed cache: sequence b owns pos[b] + 1 + extra_rows rows.

    k [sum len, Hkv, d_qk], v [sum len, Hkv, d_v], seq_offsets [B+1] int64.
    Each sequence's rows come from their own seeds, so one sequence can be
    drawn again on its own.
    """
    lens = pos.to(torch.int64).cpu() + 1 + int(extra_rows)
    offs = torch.zeros(B + 1, dtype=torch.int64)
    offs[1:] = torch.cumsum(lens, 0)
    total = int(offs[-1])
    tdt = _torch_dtype(dtype)
    q = normal((B, hq, d_qk), tensor_seed(seed, TID_Q_GA), device, dtype)
    k = torch.empty((total, hkv, d_qk), dtype=tdt, device=device)
    v = torch.empty((total, hkv, d_v), dtype=tdt, device=device)
    for b in range(B):
        lo, hi = int(offs[b]), int(offs[b + 1])
        k[lo:hi] = normal((hi - lo, hkv, d_qk), tensor_seed(seed, TID_K_GA, b), device, "f32")
        v[lo:hi] = normal((hi - lo, hkv, d_v), tensor_seed(seed, TID_V_GA, b), device, "f32")
    sink = None
    if sink_range is not None:
        sink = uniform((hq,), sink_range[0], sink_range[1], tensor_seed(seed, TID_SINK), device)
    return dict(q=q, k=k, v=v, sink=sink, pos=pos.to(device), seq_offsets=offs.to(device))


def multi_ring_inputs(B, T, hq, hkv, slots, d_qk, d_v, dtype, seed, pos, device="cpu",
                      sink_range=(-2.0, 2.0)):
    """q [B,T,Hq,d_qk] (T queries per sequence) and a ring k [B,S,Hkv,d_qk],
    v [B,S,Hkv,d_v] of S slots."""
    q = normal((B, T, hq, d_qk), tensor_seed(seed, TID_Q), device, dtype)
    k = normal((B, slots, hkv, d_qk), tensor_seed(seed, TID_K), device, dtype)
    v = normal((B, slots, hkv, d_v), tensor_seed(seed, TID_V), device, dtype)
    sink = None
    if sink_range is not None:
        sink = uniform((hq,), sink_range[0], sink_range[1], tensor_seed(seed, TID_SINK), device)
    return dict(q=q, k=k, v=v, sink=sink, pos=pos.to(device))


def multi_contiguous_inputs(B, T, hq, hkv, d_qk, d_v, dtype, seed, pos, device="cpu",
                            sink_range=None, extra_rows=0):
    """q [B,T,Hq,d_qk] and a packed cache in which sequence b owns
    pos[b] + T + extra_rows rows (layout as contiguous_decode_inputs)."""
    d = contiguous_decode_inputs(B, hq, hkv, d_qk, d_v, dtype, seed, pos, device, sink_range,
                                 extra_rows=extra_rows + T - 1)
    d["q"] = normal((B, T, hq, d_qk), tensor_seed(seed, TID_Q_GA), device, dtype)
    return d


def kv_scales(hkv, lo, hi, seed, device="cpu"):
    """Per-kv-head FP8 scales of K and V, float32 [hkv] each."""
    return (uniform((hkv,), lo, hi, tensor_seed(seed, TID_KSCALE), device),
            uniform((hkv,), lo, hi, tensor_seed(seed, TID_VSCALE), device))


def e4m3_codes(x, scale):
    """E4M3 codes (uint8) of x / scale[head] for x [..., Hkv, d] float32."""
    return (x / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)


def ring_decode_inputs_fp8(B, hq, hkv, window, d_qk, d_v, seed, pos, device="cpu",
                           sink_range=(-2.0, 2.0), scale_range=(0.02, 0.04), qdtype="bf16"):
    """q [B,Hq,d_qk] and an E4M3 ring cache k [B,W,Hkv,d_qk], v [B,W,Hkv,d_v] (uint8)
    with scales k_scale, v_scale [Hkv]."""
    ks, vs = kv_scales(hkv, scale_range[0], scale_range[1], seed, device)
    q = normal((B, hq, d_qk), tensor_seed(seed, TID_Q), device, qdtype)
    k = e4m3_codes(normal((B, window, hkv, d_qk), tensor_seed(seed, TID_K), device, "f32"), ks)
    v = e4m3_codes(normal((B, window, hkv, d_v), tensor_seed(seed, TID_V), device, "f32"), vs)
    sink = None
    if sink_range is not None:
        sink = uniform((hq,), sink_range[0], sink_range[1], tensor_seed(seed, TID_SINK), device)
    return dict(q=q, k=k, v=v, k_scale=ks, v_scale=vs, sink=sink, pos=pos.to(device))


def contiguous_decode_inputs_fp8(B, hq, hkv, d_qk, d_v, seed, pos, device="cpu", sink_range=None,
                                 extra_rows=0, scale_range=(0.02, 0.04), qdtype="bf16"):
    """q [B,Hq,d_qk] and a packed E4M3 cache (layout as contiguous_decode_inputs),
    with scales k_scale, v_scale [Hkv]."""
    ks, vs = kv_scales(hkv, scale_range[0], scale_range[1], seed, device)
    lens = pos.to(torch.int64).cpu() + 1 + int(extra_rows)
    offs = torch.zeros(B + 1, dtype=torch.int64)
    offs[1:] = torch.cumsum(lens, 0)
    total = int(offs[-1])
    q = normal((B, hq, d_qk), tensor_seed(seed, TID_Q_GA), device, qdtype)
    k = torch.empty((total, hkv, d_qk), dtype=torch.uint8, device=device)
    v = torch.empty((total, hkv, d_v), dtype=torch.uint8, device=device)
    for b in range(B):
        lo, hi = int(offs[b]), int(offs[b + 1])
        k[lo:hi] = e4m3_codes(normal((hi - lo, hkv, d_qk), tensor_seed(seed, TID_K_GA, b), device,
                                     "f32"), ks)
        v[lo:hi] = e4m3_codes(normal((hi - lo, hkv, d_v), tensor_seed(seed, TID_V_GA, b), device,
                                     "f32"), vs)
    sink = None
    if sink_range is not None:
        sink = uniform((hq,), sink_range[0], sink_range[1], tensor_seed(seed, TID_SINK), device)
    return dict(q=q, k=k, v=v, k_scale=ks, v_scale=vs, sink=sink, pos=pos.to(device),
                seq_offsets=offs.to(device))


def sparse_selection(B, n, hkv, recent, max_sel, seed, device="cpu", chunk_rows=8192):
    """Selected-token lists idx [B,n,Hkv,max_sel] int32 (-1 padded) and counts [B,n,Hkv].

    Candidates for query i are [0, max(0, i - recent)).  When there are more
    than max_sel, Floyd's algorithm draws max_sel distinct ones uniformly:
    for j = avail - max_sel .. avail - 1 draw t ~ U{0..j}; keep t unless it
    was already taken, in which case keep j.  A per-row bitmap records the
    set, so reading it back in index order gives the sorted list.
    """
    avail = torch.clamp(torch.arange(n, dtype=torch.int64) - recent, min=0)   # [n]
    count = torch.clamp(avail, max=max_sel)
    idx = torch.full((B, n, hkv, max_sel), -1, dtype=torch.int32, device=device)
    cols = torch.arange(max_sel, dtype=torch.int64)
    small = avail <= max_sel
    # Rows with few candidates take all of them.
    small_rows = torch.nonzero(small).flatten()
    if small_rows.numel():
        fill = torch.where(cols[None, :] < avail[small_rows][:, None],
                           cols[None, :], torch.full_like(cols[None, :], -1)).to(torch.int32)
        idx[:, small_rows] = fill[None, :, None, :].to(device)
    big_rows = torch.nonzero(~small).flatten()
    if big_rows.numel():
        g = _gen(tensor_seed(seed, TID_SEL), device)
        # Flatten (b, i, head) over the rows that need sampling.
        A = avail[big_rows].to(device)                                        # [R]
        R = big_rows.numel()
        flatA = A[None, :, None].expand(B, R, hkv).reshape(-1)
        total = flatA.numel()
        out = torch.empty((total, max_sel), dtype=torch.int32, device=device)
        amax = int(avail.max())
        for c0 in range(0, total, chunk_rows):
            c1 = min(total, c0 + chunk_rows)
            Ac = flatA[c0:c1]
            m = c1 - c0
            bitmap = torch.zeros((m, amax), dtype=torch.bool, device=device)
            ar = torch.arange(m, device=device)
            for step in range(max_sel):
                j = Ac - max_sel + step                                        # [m]
                u = torch.rand(m, generator=g, device=device, dtype=torch.float64)
                t = torch.minimum(torch.floor(u * (j + 1).to(torch.float64)).to(torch.int64), j)
                taken = bitmap[ar, t]
                pick = torch.where(taken, j, t)
                bitmap[ar, pick] = True
            nz = torch.nonzero(bitmap)                                         # row-major: sorted
            out[c0:c1] = nz[:, 1].reshape(m, max_sel).to(torch.int32)
        idx[:, big_rows] = out.reshape(B, R, hkv, max_sel)
    cnt = count[None, :, None].expand(B, n, hkv).to(torch.int32).contiguous().to(device)
    return idx, cnt


def sparse_inputs_fp8(B, n, hq, hkv, d_qk, d_v, seed, recent=128, max_sel=1024, device="cpu",
                      sink_range=(-2.0, 2.0), scale_range=(0.02, 0.04), qdtype="bf16"):
    """sparse_inputs with K/V as E4M3 codes (uint8) and scales k_scale, v_scale [Hkv]."""
    d = prefill_inputs(B, n, hq, hkv, d_qk, d_v, "f32", seed, device, sink_range)
    ks, vs = kv_scales(hkv, scale_range[0], scale_range[1], seed, device)
    d.update(q=d["q"].to(_torch_dtype(qdtype)), k=e4m3_codes(d["k"], ks), v=e4m3_codes(d["v"], vs),
             k_scale=ks, v_scale=vs)
    idx, cnt = sparse_selection(B, n, hkv, recent, max_sel, seed, device)
    d.update(sel_idx=idx, sel_count=cnt)
    return d


def sparse_inputs(B, n, hq, hkv, d_qk, d_v, dtype, seed, recent=128, max_sel=1024,
                  device="cpu", sink_range=(-2.0, 2.0)):
    d = prefill_inputs(B, n, hq, hkv, d_qk, d_v, dtype, seed, device, sink_range)
    idx, cnt = sparse_selection(B, n, hkv, recent, max_sel, seed, device)
    d.update(sel_idx=idx, sel_count=cnt)
    return d
