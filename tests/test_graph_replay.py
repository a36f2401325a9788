"""The one-launch ring decodes captured in a HIP graph (the form in which
the bench times them, and in which a serving loop would replay a decode
step) give on every replay exactly what eager calls give: two calls with
different inputs and outputs per entry point, replayed three times with the
program's own eager work and synchronisations in between."""

import pytest
import torch

import hybrid_sliding_window_amd as hswa
import synthetic

DEV = "cuda"
pytestmark = pytest.mark.gpu


def _ring_calls():
    """(call(out), out shape) pairs: bf16 ring, E4M3 ring and multi-token ring
    decode steps at small batch, two input sets each."""
    pos = torch.tensor([0, 5, 127, 128, 4000, 131071], dtype=torch.int64)
    B, hq, hkv, W = len(pos), 64, 8, 128
    calls = []
    for r in range(2):
        d = synthetic.ring_decode_inputs(B, hq, hkv, W, 192, 128, "bf16", 300 + r, pos, DEV)
        ws = torch.empty(hswa.decode_workspace_size(hswa.KV_RING, B, hq, 128, W, 131071),
                         dtype=torch.uint8, device=DEV)
        calls.append(((B, hq, 128), lambda o, d=d, ws=ws: hswa.swa_sink_decode(
            d["q"], d["k"], d["v"], d["pos"], 131071, layout=hswa.KV_RING, sink=d["sink"],
            window=W, out=o, workspace=ws)))
        f = synthetic.ring_decode_inputs_fp8(B, hq, hkv, W, 192, 128, 310 + r, pos, DEV)
        calls.append(((B, hq, 128), lambda o, f=f, ws=ws: hswa.swa_sink_decode_fp8(
            f["q"], f["k"], f["v"], f["k_scale"], f["v_scale"], f["pos"], 131071,
            layout=hswa.KV_RING, sink=f["sink"], window=W, out=o, workspace=ws)))
        T, S = 4, 131
        m = synthetic.multi_ring_inputs(B, T, hq, hkv, S, 192, 128, "bf16", 320 + r, pos, DEV)
        wsm = torch.empty(hswa.decode_multi_workspace_size(hswa.KV_RING, B, T, hq, 128, W, S,
                                                           131071 + T - 1),
                          dtype=torch.uint8, device=DEV)
        calls.append(((B, T, hq, 128), lambda o, m=m, wsm=wsm: hswa.swa_sink_decode_multi(
            m["q"], m["k"], m["v"], m["pos"], 131071 + T - 1, layout=hswa.KV_RING, ring_slots=S,
            sink=m["sink"], window=W, out=o, workspace=wsm)))
    return calls


def test_ring_decodes_replayed_from_a_graph_match_eager(gpu_lib):
    calls = _ring_calls()
    eager = []
    for shape, call in calls:
        o = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        call(o)
        eager.append(o)
    torch.cuda.synchronize()
    outs = [torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV) for shape, _ in calls]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for (_, call), o in zip(calls, outs):
            call(o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (_, call), o in zip(calls, outs):
            call(o)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))          # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {rep}, call {k}: differs from the eager result"
    del g
