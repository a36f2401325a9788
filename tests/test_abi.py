"""The C ABI on the host: the library loads, exports every symbol the header
declares, sizes workspaces, and rejects bad arguments before enqueuing any
work.  None of these calls reach the GPU, so they run without one."""

import ctypes
import os
import re

import pytest

import hybrid_sliding_window_amd as hswa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hswa.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
FAKE = 0x10000          # 16-byte aligned fake device address, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hswa.lib_path()):
        from hybrid_sliding_window_amd.build import build
        build()
    return hswa.load()


def _declared():
    inc = os.path.dirname(HEADER)
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_and_binding_agree(lib):
    declared = _declared()
    assert set(declared) == set(hswa.EXPORTED_SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} is declared but not exported"


def test_version_string(lib):
    assert hswa.version().startswith("hswa")


def test_workspace_sizes(lib):
    # cos/sin table (seqlen * R/2 * 8 bytes) then rotated K dims (B * n * hkv * R * 2 bytes),
    # each rounded up to 256 bytes; R = 64 at d = 192 and fraction 0.334
    assert hswa.prefill_workspace_size(1, 32768, 8, 192, 0.334) == 32768 * 32 * 8 + 32768 * 8 * 64 * 2
    assert hswa.prefill_workspace_size(2, 1000, 4, 192, 0.0) == 0
    r256 = lambda x: ((x + 255) // 256) * 256  # noqa: E731
    assert hswa.sparse_workspace_size(1, 100, 3, 192, 0.334) == r256(100 * 32 * 8) + r256(100 * 3 * 64 * 2)
    # decode: fp32 partial (O, m, l) per (sequence, head, split), then q rotated
    # to its position (bf16, 192 dims); the ring splits 128 keys in 4, a
    # 262144-key prefix in 64 splits of 4096
    qrot = 64 * 64 * 192 * 2
    ring = hswa.decode_workspace_size(hswa.KV_RING, 64, 64, 128, 128, 262143)
    assert ring == 64 * 64 * 4 * 128 * 4 + r256(64 * 64 * 4 * 2 * 4) + qrot
    contig = hswa.decode_workspace_size(hswa.KV_CONTIGUOUS, 64, 64, 128, 0, 262143)
    assert contig == 64 * 64 * 64 * 128 * 4 + 64 * 64 * 64 * 2 * 4 + qrot
    assert hswa.decode_workspace_size(hswa.KV_RING, 64, 64, 128, 0, 10) == 0


def _prefill(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, sink=None, o=FAKE, batch=1, seqlen=16, hq=4, hkv=2,
                d_qk=192, d_v=128, window=8, scale=0.0, theta=1e4, frac=0.0, pos_offset=0,
                dtype=1, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    return lib.swa_sink_prefill(*args.values())


def test_prefill_validation(lib):
    assert _prefill(lib, q=None) == INVALID
    assert "non-null" in lib.hswa_last_error().decode()
    assert _prefill(lib, hq=5) == INVALID                 # not a multiple of hkv
    assert _prefill(lib, hkv=0) == INVALID
    assert _prefill(lib, d_qk=0) == INVALID
    assert _prefill(lib, window=-1) == INVALID
    assert _prefill(lib, dtype=7) == INVALID
    assert _prefill(lib, scale=-1.0) == INVALID
    assert _prefill(lib, frac=1.5) == INVALID
    assert _prefill(lib, frac=0.334, theta=0.0) == INVALID
    assert _prefill(lib, o=MISALIGNED) == INVALID
    assert _prefill(lib, frac=0.334) == INVALID           # workspace missing
    assert _prefill(lib, frac=0.334, ws=FAKE, ws_bytes=8) == INVALID
    assert _prefill(lib, d_qk=300) == UNSUPPORTED          # generic path caps head dims at 256
    assert _prefill(lib, d_qk=300, dtype=0) == UNSUPPORTED
    # empty work is a successful no-op that never touches the device
    assert _prefill(lib, seqlen=0, q=None) == OK
    assert _prefill(lib, batch=0, q=None) == OK
    assert lib.hswa_last_error().decode() == ""


@pytest.mark.parametrize("entry", ["swa_sink_prefill_chunk", "swa_sink_prefill_chunk_cached"])
def test_prefill_chunk_validation(lib, entry):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sink=None, o=FAKE, batch=1, q_len=16, kv_len=40, hq=4,
                 hkv=2, d_qk=192, d_v=128, window=8, scale=0.0, theta=1e4, frac=0.0,
                 pos_offset=0, dtype=1, ws=None, ws_bytes=0, stream=None)
        a.update(kw)
        return getattr(lib, entry)(*a.values())
    assert call(q_len=41) == INVALID                       # longer than its sequence
    assert "q_len" in lib.hswa_last_error().decode()
    assert call(q_len=-1) == INVALID
    assert call(kv_len=-1, q_len=0) == INVALID
    assert call(k=None) == INVALID
    assert call(frac=0.334) == INVALID                     # workspace missing (sized by kv_len)
    assert call(frac=0.334, ws=FAKE, ws_bytes=(16 * 32 * 8 + 255) // 256 * 256) == INVALID
    assert call(d_qk=300) == UNSUPPORTED
    assert call(q_len=0, q=None) == OK                     # empty chunk: nothing to do
    assert call(batch=0, q=None) == OK


def test_decode_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, layout=0, offs=None, pos=FAKE, sink=None, o=FAKE, batch=2,
                 hq=8, hkv=4, d_qk=192, d_v=128, window=128, max_pos=1000, scale=0.0, theta=1e4,
                 frac=0.0, dtype=1, ws=None, ws_bytes=0, stream=None)
        a.update(kw)
        return lib.swa_sink_decode(*a.values())
    assert call(layout=5) == INVALID
    assert call(window=0) == INVALID                       # ring needs its slot count
    assert call(offs=FAKE) == INVALID                      # ring takes no offsets
    assert call(layout=1) == INVALID                       # contiguous needs offsets
    assert call(pos=None) == INVALID
    assert call(max_pos=-1) == INVALID
    assert call() == INVALID                               # workspace missing
    assert call(batch=0) == OK


def test_decode_multi_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, layout=0, slots=131, offs=None, pos=FAKE, sink=None,
                 o=FAKE, batch=2, q_len=4, hq=8, hkv=4, d_qk=192, d_v=128, window=128,
                 max_pos=1000, scale=0.0, theta=1e4, frac=0.0, dtype=1, ws=None, ws_bytes=0,
                 stream=None)
        a.update(kw)
        return lib.swa_sink_decode_multi(*a.values())
    assert call(slots=130) == INVALID                      # ring too small for 4 queries
    assert "ring_slots" in lib.hswa_last_error().decode()
    assert call(window=0) == INVALID                       # a ring serves a window
    assert call(offs=FAKE) == INVALID
    assert call(layout=1, slots=0) == INVALID              # contiguous needs offsets
    assert call(layout=1, slots=5, offs=FAKE) == INVALID   # ... and no slot count
    assert call(q_len=-1) == INVALID
    assert call() == INVALID                               # workspace missing
    assert call(q_len=0, q=None) == OK
    r256 = lambda x: ((x + 255) // 256) * 256  # noqa: E731
    # ring of 131 slots: 5 splits of 32 keys per (sequence, token, head)
    assert hswa.decode_multi_workspace_size(hswa.KV_RING, 64, 4, 64, 128, 128, 131, 262143) == \
        64 * 4 * 64 * 5 * 128 * 4 + r256(64 * 4 * 64 * 5 * 2 * 4) + 64 * 4 * 64 * 192 * 2


def test_append_validation(lib):
    def call(fp8=False, **kw):
        a = dict(kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, layout=0, slots=131, offs=None, pos=FAKE,
                 batch=2, q_len=4, hkv=8, d_qk=192, d_v=128, max_pos=1000, theta=1e4, frac=0.334,
                 dtype=1, stream=None)
        a.update(kw)
        if fp8:
            v = list(a.values())
            return lib.kv_cache_append_fp8(*v[:4], kw.get("ks", FAKE), kw.get("vs", FAKE), *v[4:])
        return lib.kv_cache_append(*a.values())
    assert call(slots=0) == INVALID                        # a ring needs its slot count
    assert call(offs=FAKE) == INVALID
    assert call(layout=1, slots=0) == INVALID              # contiguous needs offsets
    assert call(frac=0.1) == UNSUPPORTED                   # R/2 = 9: not a multiple of 8
    assert call(d_v=100) == UNSUPPORTED
    assert call(frac=1.0) == UNSUPPORTED                   # R/2 = 96 > 64
    assert call(pos=None) == INVALID
    assert call(kc=MISALIGNED) == INVALID
    assert call(q_len=0, kn=None) == OK
    assert lib.kv_cache_append_fp8(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 131, None, FAKE, 2, 4, 8,
                                   192, 128, 1000, 1e4, 0.334, 1, None) == INVALID   # k_scale missing


def test_select_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, idx=FAKE, cnt=FAKE, max_sel=64, recent=16, batch=1, seqlen=100,
                 hq=64, hkv=4, d_qk=192, scale=0.0, theta=1e7, frac=0.0, pos_offset=0, dtype=1,
                 ws=None, ws_bytes=0, stream=None)
        a.update(kw)
        return lib.sparse_select_tokens(*a.values())
    assert call(hq=32) == UNSUPPORTED                      # 16 query heads per kv head only
    assert call(dtype=0) == UNSUPPORTED                    # bf16 only
    assert call(d_qk=128) == UNSUPPORTED
    assert call(max_sel=-1) == INVALID
    assert call(recent=0) == INVALID
    assert call(cnt=None) == INVALID
    assert call(frac=0.334) == INVALID                     # workspace missing
    assert call() == INVALID                               # importance scratch missing
    assert call(seqlen=0, q=None) == OK
    # log-sum-exp rows (fp32, rounded up to 256 bytes), then 256 slots of 32
    # rows: round64(100) words and a 4096-entry list of 8 bytes per row
    lse = (100 * 64 * 4 + 255) // 256 * 256
    scratch = lse + 256 * 32 * (128 * 4 + 4096 * 8)
    size = hswa._binding.load().hswa_select_workspace_size
    assert size(1, 100, 64, 4, 192, 0.334) == 100 * 64 * 192 * 2 + 100 * 4 * 192 * 2 + scratch
    assert size(1, 100, 64, 4, 192, 0.0) == scratch
    assert call(ws=FAKE, ws_bytes=scratch - 1) == INVALID


def test_decode_fp8_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, layout=0, offs=None, pos=FAKE, sink=None,
                 o=FAKE, batch=2, hq=8, hkv=4, d_qk=192, d_v=128, window=128, max_pos=1000,
                 scale=0.0, theta=1e4, frac=0.0, dtype=1, ws=None, ws_bytes=0, stream=None)
        a.update(kw)
        return lib.swa_sink_decode_fp8(*a.values())
    assert call(ks=None) == INVALID
    assert "k_scale" in lib.hswa_last_error().decode()
    assert call(vs=None) == INVALID
    assert call(layout=1) == INVALID                       # contiguous needs offsets
    assert call(window=0) == INVALID                       # ring needs its slot count
    assert call(k=MISALIGNED) == INVALID
    assert call() == INVALID                               # workspace missing
    assert call(batch=0, ks=None) == OK


def test_sparse_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE, max_sel=16, recent=8, sink=None,
                 o=FAKE, batch=1, seqlen=32, hq=4, hkv=2, d_qk=192, d_v=128, scale=0.0, theta=1e4,
                 frac=0.0, pos_offset=0, dtype=1, ws=None, ws_bytes=0, stream=None)
        a.update(kw)
        return lib.sparse_sink_attn(*a.values())
    assert call(recent=0) == INVALID
    assert call(max_sel=-1) == INVALID
    assert call(cnt=None) == INVALID
    assert call(idx=None) == INVALID
    assert call(frac=0.334) == INVALID                     # workspace missing
    assert call(seqlen=0) == OK


def test_sparse_fp8_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, idx=FAKE, cnt=FAKE, max_sel=16, recent=8,
                 sink=None, o=FAKE, batch=1, seqlen=32, hq=4, hkv=2, d_qk=192, d_v=128, scale=0.0,
                 theta=1e4, frac=0.0, pos_offset=0, dtype=1, ws=None, ws_bytes=0, stream=None)
        a.update(kw)
        return lib.sparse_sink_attn_fp8(*a.values())
    assert call(ks=None) == INVALID
    assert "k_scale" in lib.hswa_last_error().decode()
    assert call(vs=None) == INVALID
    assert call(recent=0) == INVALID
    assert call(frac=0.334) == INVALID                     # workspace missing
    assert call(seqlen=0, ks=None) == OK


def test_binding_rejects_bad_tensors(lib):
    import torch
    q = torch.zeros(1, 4, 2, 192, dtype=torch.float16)
    with pytest.raises(TypeError):
        hswa._binding._dtype_code(q)
    with pytest.raises(TypeError):
        hswa._binding._sink(torch.zeros(2, dtype=torch.float64), q, 2)
    with pytest.raises(TypeError, match="q has dtype"):
        hswa.swa_sink_prefill(q, q[:, :, :1], torch.zeros(1, 4, 1, 128, dtype=torch.float16))


def test_product_path_does_not_use_the_oracle():
    """The package never imports the CPU oracle or falls back to the CPU."""
    pkg = os.path.join(ROOT, "hybrid_sliding_window_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("the oracle", ""), f
                assert "scaled_dot_product_attention" not in text, f


# ---------------------------------------------------------------------------
# The Python binding checks shapes and dtypes before any call into the
# library: mismatches raise on host tensors, so no kernel is ever launched.
# ---------------------------------------------------------------------------

import torch  # noqa: E402


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _prefill_set(B=1, n=40, hq=16, hkv=2, dtype=torch.bfloat16):
    return _t(B, n, hq, 192, dtype=dtype), _t(B, n, hkv, 192, dtype=dtype), _t(B, n, hkv, 128, dtype=dtype)


@pytest.mark.parametrize("case,exc,match", [
    ("k_dtype", TypeError, "k has dtype"),
    ("k_len", ValueError, "k has shape"),
    ("k_dim", ValueError, "k has shape"),
    ("v_heads", ValueError, "v has shape"),
    ("v_batch", ValueError, "v has shape"),
    ("out_shape", ValueError, "out has shape"),
    ("out_dtype", TypeError, "out has dtype"),
    ("sink_shape", ValueError, "sink has shape"),
    ("sink_dtype", TypeError, "sink has dtype"),
    ("heads", ValueError, "multiple of hkv"),
    ("q_dims", ValueError, "q must have 4 dims"),
    ("workspace", ValueError, "workspace holds"),
    ("host_tensors", ValueError, "GPU device"),
])
def test_binding_rejects_prefill_mismatch(lib, case, exc, match):
    q, k, v = _prefill_set()
    kw = dict(window=16, rope_theta=1e4, rotary_fraction=0.334)
    sink = torch.zeros(16, dtype=torch.float32)
    if case == "k_dtype":
        q = q.float()
        v = v.float()
    elif case == "k_len":
        k = _t(1, 39, 2, 192)
    elif case == "k_dim":
        k = _t(1, 40, 2, 128)
    elif case == "v_heads":
        v = _t(1, 40, 4, 128)
    elif case == "v_batch":
        v = _t(2, 40, 2, 128)
    elif case == "out_shape":
        kw["out"] = _t(1, 40, 16, 192)
    elif case == "out_dtype":
        kw["out"] = _t(1, 40, 16, 128, dtype=torch.float32)
    elif case == "sink_shape":
        sink = torch.zeros(8, dtype=torch.float32)
    elif case == "sink_dtype":
        sink = torch.zeros(16, dtype=torch.float64)
    elif case == "heads":
        q = _t(1, 40, 15, 192)
        sink = torch.zeros(15, dtype=torch.float32)
    elif case == "q_dims":
        q = _t(40, 16, 192)
    elif case == "workspace":
        kw["workspace"] = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(exc, match=match):
        hswa.swa_sink_prefill(q, k, v, sink, **kw)


def test_binding_rejects_other_prefill_mismatches(lib):
    q, k, v = _prefill_set()
    with pytest.raises(ValueError, match="must not exceed kv_len"):
        hswa.swa_sink_prefill_chunk(_t(1, 41, 16, 192), k, v, None, window=16)
    with pytest.raises(ValueError, match="v has shape"):
        hswa.swa_sink_prefill_chunk(q[:, :10], k, v[:, :30], None, window=16)
    with pytest.raises(TypeError, match="k has dtype"):
        hswa.ga_prefill(q, k.float(), v)
    with pytest.raises(ValueError, match="k has shape"):
        hswa.swa_sink_prefill_chunk_cached(q[:, :10], _t(2, 40, 2, 192), v, None)


def test_binding_rejects_decode_mismatch(lib):
    B, hq, hkv, W = 3, 16, 2, 128
    q = _t(B, hq, 192)
    kr, vr = _t(B, W, hkv, 192), _t(B, W, hkv, 128)
    pos = torch.zeros(B, dtype=torch.int64)
    with pytest.raises(ValueError, match="k_cache has shape"):       # ring shorter than the window
        hswa.swa_sink_decode(q, _t(B, W - 1, hkv, 192), vr, pos, 10, window=W)
    with pytest.raises(ValueError, match="v_cache has shape"):
        hswa.swa_sink_decode(q, kr, _t(B, W, hkv + 1, 128), pos, 10, window=W)
    with pytest.raises(TypeError, match="pos has dtype"):
        hswa.swa_sink_decode(q, kr, vr, pos.int(), 10, window=W)
    with pytest.raises(ValueError, match="pos has shape"):
        hswa.swa_sink_decode(q, kr, vr, pos[:2], 10, window=W)
    with pytest.raises(TypeError, match="k_cache has dtype"):
        hswa.swa_sink_decode(q.float(), kr, vr, pos, 10, window=W)
    with pytest.raises(ValueError, match="seq_offsets must be None"):
        hswa.swa_sink_decode(q, kr, vr, pos, 10, window=W, seq_offsets=torch.zeros(B + 1, dtype=torch.int64))
    kc, vc = _t(100, hkv, 192), _t(100, hkv, 128)
    with pytest.raises(ValueError, match="seq_offsets is required"):
        hswa.swa_sink_decode(q, kc, vc, pos, 10, layout=hswa.KV_CONTIGUOUS, window=0)
    with pytest.raises(ValueError, match="seq_offsets has shape"):
        hswa.swa_sink_decode(q, kc, vc, pos, 10, layout=hswa.KV_CONTIGUOUS, window=0,
                             seq_offsets=torch.zeros(B, dtype=torch.int64))
    with pytest.raises(ValueError, match="out has shape"):
        hswa.swa_sink_decode(q, kc, vc, pos, 10, layout=hswa.KV_CONTIGUOUS, window=0,
                             seq_offsets=torch.zeros(B + 1, dtype=torch.int64), out=_t(B, hq, 192))
    # multi-token: the ring holds ring_slots rows
    qm = _t(B, 4, hq, 192)
    with pytest.raises(ValueError, match="k_cache has shape"):
        hswa.swa_sink_decode_multi(qm, kr, vr, pos, 10, ring_slots=131, window=W)
    # FP8: codes and per-kv-head scales
    ks = torch.ones(hkv, dtype=torch.float32)
    k8, v8 = _t(B, W, hkv, 192, dtype=torch.uint8), _t(B, W, hkv, 128, dtype=torch.uint8)
    with pytest.raises(TypeError, match="k_cache has dtype"):
        hswa.swa_sink_decode_fp8(q, kr, vr, ks, ks, pos, 10, window=W)
    with pytest.raises(ValueError, match="v_scale has shape"):
        hswa.swa_sink_decode_fp8(q, k8, v8, ks, torch.ones(hkv + 1), pos, 10, window=W)


def test_binding_rejects_append_sparse_select_mismatch(lib):
    B, T, hkv = 2, 3, 2
    kn, vn = _t(B, T, hkv, 192), _t(B, T, hkv, 128)
    pos = torch.zeros(B, dtype=torch.int64)
    with pytest.raises(ValueError, match="v_new has shape"):
        hswa.kv_cache_append(kn, _t(B, T + 1, hkv, 128), _t(B, 8, hkv, 192), _t(B, 8, hkv, 128), pos,
                             10, ring_slots=8)
    with pytest.raises(ValueError, match="v_cache has shape"):
        hswa.kv_cache_append(kn, vn, _t(B, 8, hkv + 1, 192), _t(B, 8, hkv, 128), pos, 10, ring_slots=8)
    with pytest.raises(ValueError, match="caches hold 3 kv heads"):
        hswa.kv_cache_append(kn, vn, _t(B, 8, hkv + 1, 192), _t(B, 8, hkv + 1, 128), pos, 10,
                             ring_slots=8)
    with pytest.raises(ValueError, match="k_cache has shape"):
        hswa.kv_cache_append(kn, vn, _t(B, 7, hkv, 192), _t(B, 7, hkv, 128), pos, 10, ring_slots=8)
    with pytest.raises(TypeError, match="type of the new keys"):
        hswa.kv_cache_append(kn, vn, _t(B, 8, hkv, 192, dtype=torch.float32),
                             _t(B, 8, hkv, 128, dtype=torch.float32), pos, 10, ring_slots=8)
    with pytest.raises(ValueError, match="k_scale"):
        hswa.kv_cache_append(kn, vn, _t(B, 8, hkv, 192, dtype=torch.uint8),
                             _t(B, 8, hkv, 128, dtype=torch.uint8), pos, 10, ring_slots=8)
    q, k, v = _prefill_set(n=300, hq=64, hkv=4)
    idx = torch.zeros(1, 300, 4, 16, dtype=torch.int32)
    cnt = torch.zeros(1, 300, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="sel_idx has shape"):
        hswa.sparse_sink_attn(q, k, v, idx[:, :299], cnt)
    with pytest.raises(TypeError, match="sel_count has dtype"):
        hswa.sparse_sink_attn(q, k, v, idx, cnt.long())
    with pytest.raises(ValueError, match="sel_idx has shape"):
        hswa.sparse_select_tokens(q, k, max_sel=8, out=(idx, cnt))
    with pytest.raises(TypeError, match="k has dtype"):
        hswa.sparse_sink_attn_fp8(q, k, v, torch.ones(4), torch.ones(4), idx, cnt)


def test_noalloc_decode_refuses_oversize_on_the_host(lib):
    """The no-allocation decode refuses a call whose scratch would exceed the
    static maximum before any HIP call (so this runs without a GPU)."""
    import ctypes as C
    text = open(HEADER).read()
    assert "#define HSWA_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert hswa.NOALLOC_SCRATCH_BYTES == 64 << 20
    need = hswa.decode_workspace_size(hswa.KV_CONTIGUOUS, 64, 64, 128, 0, 262143)
    assert need > hswa.NOALLOC_SCRATCH_BYTES
    st = lib.swa_sink_decode_noalloc(C.c_void_p(FAKE), C.c_void_p(FAKE), C.c_void_p(FAKE), 1,
                                     C.c_void_p(FAKE), C.c_void_p(FAKE), None, C.c_void_p(FAKE),
                                     64, 64, 4, 192, 128, 0, 262143, 0.0, 1e7, 0.0, 1, None)
    assert st == INVALID
    assert "static maximum" in lib.hswa_last_error().decode()


def test_probes_reject_bad_arguments(lib):
    gp = lambda **kw: lib.hswa_gather_probe(*[kw.get(k_, d) for k_, d in (  # noqa: E731
        ("k", FAKE), ("v", FAKE), ("rows", 10), ("idx", FAKE), ("nwaves", 2), ("tiles", 1),
        ("out", FAKE), ("stream", None))])
    assert gp(k=None) == INVALID
    assert gp(rows=0) == INVALID
    assert gp(v=MISALIGNED) == INVALID
    assert gp(nwaves=1 << 26, tiles=1 << 4) == INVALID      # index list past 2^31 entries
    sp = lambda **kw: lib.hswa_stream_probe(*[kw.get(k_, d) for k_, d in (  # noqa: E731
        ("src", FAKE), ("nr", 4096), ("dst", FAKE), ("nw", 2048), ("blocks", 4), ("out", FAKE),
        ("stream", None))])
    assert sp(out=None) == INVALID
    assert sp(blocks=0) == INVALID
    assert sp(nr=0, nw=0) == INVALID
    assert sp(nr=-1024) == INVALID
    assert sp(nr=1000) == INVALID                            # not a multiple of 1024
    assert sp(src=None) == INVALID
    assert sp(dst=None) == INVALID
    assert sp(dst=MISALIGNED) == INVALID
    assert sp(blocks=1 << 30) == INVALID
