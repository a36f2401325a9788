"""swa_sink_decode_noalloc: the decode for callers that cannot allocate,
through the C ABI, against swa_sink_decode with a caller workspace (the same
kernels: outputs must agree bit for bit) and against the oracle (bf16 bar:
2e-2 max-abs, 5e-3 rel-L2).  Two calls in a row share the static scratch,
the second smaller than the first; a call needing more scratch than the
static maximum is refused before anything runs."""

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _bar(name, got, ref):
    g = _np(got)
    d = g - ref
    mx = float(np.abs(d).max())
    rl2 = float(np.linalg.norm(d) / np.linalg.norm(ref))
    print(f"[no-alloc] {name}: max_abs={mx:.3e} rel_l2={rl2:.3e}", flush=True)
    assert np.isfinite(g).all() and mx <= 2e-2 and rl2 <= 5e-3


def test_noalloc_decode_matches_workspace_decode(gpu_lib):
    # call 1: a GA layer's contiguous caches, 8 sequences up to position 20000
    pos = torch.tensor([0, 31, 4000, 20000, 777, 12345, 19999, 1], dtype=torch.int64)
    c = synthetic.contiguous_decode_inputs(len(pos), 64, 4, 192, 128, "bf16", 501, pos, DEV, None)
    need = gpu_lib.decode_workspace_size(gpu_lib.KV_CONTIGUOUS, 8, 64, 128, 0, 20000)
    assert 0 < need <= gpu_lib.NOALLOC_SCRATCH_BYTES
    kw = dict(layout=gpu_lib.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"], window=0,
              rope_theta=1.0e7, rotary_fraction=0.334)
    want = gpu_lib.swa_sink_decode(c["q"], c["k"], c["v"], c["pos"], 20000, **kw)
    got = gpu_lib.swa_sink_decode_noalloc(c["q"], c["k"], c["v"], c["pos"], 20000, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    ref = oracle.swa_sink_decode_contiguous(_np(c["q"]), _np(c["k"]), _np(c["v"]),
                                            c["seq_offsets"].cpu().numpy(), pos.numpy(), None, None,
                                            rope_theta=1.0e7, rotary_fraction=0.334)
    _bar("GA contiguous, 8 sequences", got, ref)

    # call 2: smaller, an SWA layer's ring of 128 slots, 4 sequences, the
    # output in a caller tensor (nothing allocated by the call)
    pos2 = torch.tensor([5, 127, 4000, 131072], dtype=torch.int64)
    r = synthetic.ring_decode_inputs(4, 64, 8, 128, 192, 128, "bf16", 502, pos2, DEV, (-2.0, 2.0))
    assert gpu_lib.decode_workspace_size(gpu_lib.KV_RING, 4, 64, 128, 128, 131072) < need
    out = torch.empty(4, 64, 128, dtype=torch.bfloat16, device=DEV)
    kw2 = dict(layout=gpu_lib.KV_RING, sink=r["sink"], window=128, rope_theta=1.0e4,
               rotary_fraction=0.334)
    gpu_lib.swa_sink_decode_noalloc(r["q"], r["k"], r["v"], r["pos"], 131072, out=out, **kw2)
    want2 = gpu_lib.swa_sink_decode(r["q"], r["k"], r["v"], r["pos"], 131072, **kw2)
    torch.cuda.synchronize()
    assert torch.equal(out, want2)
    ref2 = oracle.swa_sink_decode_ring(_np(r["q"]), _np(r["k"]), _np(r["v"]), pos2.numpy(),
                                       _np(r["sink"]), rope_theta=1.0e4, rotary_fraction=0.334)
    _bar("SWA ring, 4 sequences", out, ref2)

    # a call above the static maximum is refused, nothing enqueued
    big = gpu_lib.decode_workspace_size(gpu_lib.KV_CONTIGUOUS, 64, 64, 128, 0, 262143)
    assert big > gpu_lib.NOALLOC_SCRATCH_BYTES
    bpos = torch.zeros(64, dtype=torch.int64, device=DEV)
    offs = torch.zeros(65, dtype=torch.int64, device=DEV)
    q = torch.zeros(64, 64, 192, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, 4, 192, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(1, 4, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gpu_lib.HswaError, match="static maximum"):
        gpu_lib.swa_sink_decode_noalloc(q, kc, vc, bpos, 262143, layout=gpu_lib.KV_CONTIGUOUS,
                                        seq_offsets=offs, window=0)
