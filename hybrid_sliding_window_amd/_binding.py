"""ctypes binding of libhswa.so.  Argument marshalling only."""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libhswa.so")
_lib = None

HSWA_F32, HSWA_BF16 = 0, 1
KV_RING, KV_CONTIGUOUS = 0, 1
_STATUS = {0: "HSWA_OK", 1: "HSWA_ERR_INVALID_ARGUMENT", 2: "HSWA_ERR_UNSUPPORTED",
           3: "HSWA_ERR_HIP"}

_vp, _i, _ll, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_size_t

# Every symbol include/hswa.h and include/hswa_measure.h declare, with
# (restype, argtypes).
_SIGNATURES = {
    "hswa_prefill_workspace_size": (_sz, [_i, _i, _i, _i, _f]),
    "swa_sink_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _f, _f,
                              _ll, _i, _vp, _sz, _vp]),
    "swa_sink_prefill_chunk": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f,
                                    _f, _f, _ll, _i, _vp, _sz, _vp]),
    "swa_sink_prefill_chunk_cached": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                           _f, _f, _f, _ll, _i, _vp, _sz, _vp]),
    "ga_prefill": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _f, _ll, _i, _vp, _sz,
                        _vp]),
    "hswa_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i, _ll]),
    "swa_sink_decode": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _ll,
                             _f, _f, _f, _i, _vp, _sz, _vp]),
    "swa_sink_decode_noalloc": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                     _ll, _f, _f, _f, _i, _vp]),
    "kv_cache_append": (_i, [_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _i, _ll, _f, _f,
                             _i, _vp]),
    "kv_cache_append_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _i,
                                 _ll, _f, _f, _i, _vp]),
    "hswa_decode_multi_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _ll]),
    "swa_sink_decode_multi": (_i, [_vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                   _i, _i, _ll, _f, _f, _f, _i, _vp, _sz, _vp]),
    "swa_sink_decode_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                 _i, _i, _ll, _f, _f, _f, _i, _vp, _sz, _vp]),
    "hswa_sparse_workspace_size": (_sz, [_i, _i, _i, _i, _f]),
    "sparse_sink_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i, _i, _i, _i,
                              _f, _f, _f, _ll, _i, _vp, _sz, _vp]),
    "sparse_sink_attn_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _i, _i, _i,
                                  _i, _i, _i, _f, _f, _f, _ll, _i, _vp, _sz, _vp]),
    "hswa_select_workspace_size": (_sz, [_i, _i, _i, _i, _i, _f]),
    "sparse_select_tokens": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _f, _f, _ll,
                                  _i, _vp, _sz, _vp]),
    "hswa_gather_probe": (_i, [_vp, _vp, _i, _vp, _i, _i, _vp, _vp]),
    "hswa_stream_probe": (_i, [_vp, _ll, _vp, _ll, _i, _vp, _vp]),
    "hswa_last_error": (ctypes.c_char_p, []),
    "hswa_version": (ctypes.c_char_p, []),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class HswaError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.status_name = _STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


def lib_path():
    return _LIB_PATH


def load():
    """Load libhswa.so (built by hybrid_sliding_window_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m hybrid_sliding_window_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def version():
    return load().hswa_version().decode()


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return HSWA_F32
    if t.dtype == torch.bfloat16:
        return HSWA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check_same(ref, *ts):
    """Every tensor on ref's device (a GPU: the kernels take device pointers)
    and dense.  Called after the shape and dtype checks."""
    if ref.device.type != "cuda":
        raise ValueError("tensors must live on a GPU device (the library takes device pointers)")
    for t in ts:
        if t is None:
            continue
        if t.device != ref.device:
            raise ValueError("all tensors must live on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, name, shape, dtypes=None):
    """t has exactly `shape` (None entries match anything) and one of `dtypes`."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != len(shape) or any(w is not None and w != g for w, g in zip(shape, t.shape)):
        want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")


def _dims(t, name, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {list(t.shape)}")
    return tuple(t.shape)


_FLOAT = (torch.float32, torch.bfloat16)
_E4M3 = (torch.uint8, torch.float8_e4m3fn)


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def _check_workspace(ws, need, ref):
    if ws is None:
        return
    if ws.device != ref.device or not ws.is_contiguous():
        raise ValueError("workspace must be a dense tensor on the query's device")
    if _ws_bytes(ws) < need:
        raise ValueError(f"workspace holds {_ws_bytes(ws)} bytes, the call needs {need}")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _raise(status):
    if status != 0:
        raise HswaError(status, load().hswa_last_error().decode())


def _sink(sink, q, hq):
    if sink is None:
        return None
    _expect(sink, "sink", (hq,), (torch.float32,))
    if sink.device != q.device or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 tensor on the query's device")
    return sink


def _out(out, shape, dtype, device):
    """The caller's output tensor after a shape / dtype check, or a new one."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _expect(out, "out", shape, (dtype,))
    return out


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _positions(pos, B, seq_offsets, contiguous):
    _expect(pos, "pos", (B,), (torch.int64,))
    if contiguous:
        _expect(seq_offsets, "seq_offsets", (B + 1,), (torch.int64,))
    elif seq_offsets is not None:
        raise ValueError("seq_offsets must be None for a ring cache")


def _scales(k_scale, v_scale, hkv):
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _expect(t, name, (hkv,), (torch.float32,))


def prefill_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction):
    return load().hswa_prefill_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction)


def sparse_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction):
    return load().hswa_sparse_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction)


def decode_workspace_size(layout, batch, hq, d_v, window, max_pos):
    return load().hswa_decode_workspace_size(layout, batch, hq, d_v, window, max_pos)


def _prefill_operands(q, k, v, sink, out, q_len_may_differ=False):
    """Shapes of a prefill-type call: q [B,nq,Hq,d_qk], k [B,n,Hkv,d_qk],
    v [B,n,Hkv,d_v] with nq == n unless q_len_may_differ."""
    B, nq, hq, dqk = _dims(q, "q", 4)
    if q.dtype not in _FLOAT:
        raise TypeError(f"q has dtype {q.dtype}, expected float32 or bfloat16")
    _, n, hkv, _ = _dims(k, "k", 4)
    _expect(k, "k", (B, None if q_len_may_differ else nq, hkv, dqk), (q.dtype,))
    _expect(v, "v", (B, n, hkv, None), (q.dtype,))
    dv = v.shape[3]
    if hkv == 0 or hq % hkv != 0:
        raise ValueError(f"hq ({hq}) must be a positive multiple of hkv ({hkv})")
    sink = _sink(sink, q, hq)
    o = _out(out, (B, nq, hq, dv), q.dtype, q.device)
    return B, nq, n, hq, hkv, dqk, dv, sink, o


def swa_sink_prefill(q, k, v, sink=None, window=128, scale=0.0, rope_theta=10000.0,
                     rotary_fraction=0.0, pos_offset=0, out=None, workspace=None):
    """q [B,n,Hq,d_qk], k [B,n,Hkv,d_qk], v [B,n,Hkv,d_v] -> o [B,n,Hq,d_v]."""
    lib = load()
    B, n, _, hq, hkv, dqk, dv, sink, o = _prefill_operands(q, k, v, sink, out)
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    _check_workspace(workspace, need, q)
    _check_same(q, k, v, o)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o), B, n, hq, hkv, dqk,
                              dv, window, scale, rope_theta, rotary_fraction, pos_offset,
                              _dtype_code(q), _ptr(ws), _ws_bytes(ws), _stream(q))
    _raise(st)
    return o


def swa_sink_prefill_chunk(q, k, v, sink=None, window=128, scale=0.0, rope_theta=10000.0,
                           rotary_fraction=0.0, pos_offset=0, out=None, workspace=None):
    """The last q_len positions of sequences of kv_len tokens (a chunk behind a
    cached prefix): q [B,q_len,Hq,d_qk], k [B,kv_len,Hkv,d_qk],
    v [B,kv_len,Hkv,d_v] -> o [B,q_len,Hq,d_v].  window=0 with sink=None is
    the GA layer's chunk."""
    lib = load()
    B, nq, n, hq, hkv, dqk, dv, sink, o = _prefill_operands(q, k, v, sink, out, True)
    if nq > n:
        raise ValueError(f"q_len ({nq}) must not exceed kv_len ({n})")
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    _check_workspace(workspace, need, q)
    _check_same(q, k, v, o)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o), B, nq, n, hq,
                                    hkv, dqk, dv, window, scale, rope_theta, rotary_fraction,
                                    pos_offset, _dtype_code(q), _ptr(ws), _ws_bytes(ws),
                                    _stream(q))
    _raise(st)
    return o


def swa_sink_prefill_chunk_cached(q, k_cache, v_cache, sink=None, window=128, scale=0.0,
                                  rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0, out=None,
                                  workspace=None):
    """swa_sink_prefill_chunk over a cache whose keys are stored already rotated
    (as kv_cache_append writes them): k_cache [B,kv_len,Hkv,d_qk]."""
    lib = load()
    B, nq, n, hq, hkv, dqk, dv, sink, o = _prefill_operands(q, k_cache, v_cache, sink, out, True)
    if nq > n:
        raise ValueError(f"q_len ({nq}) must not exceed kv_len ({n})")
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    _check_workspace(workspace, need, q)
    _check_same(q, k_cache, v_cache, o)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_prefill_chunk_cached(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sink),
                                           _ptr(o), B, nq, n, hq, hkv, dqk, dv, window, scale,
                                           rope_theta, rotary_fraction, pos_offset, _dtype_code(q),
                                           _ptr(ws), _ws_bytes(ws), _stream(q))
    _raise(st)
    return o


def ga_prefill(q, k, v, scale=0.0, rope_theta=1.0e7, rotary_fraction=0.0, pos_offset=0,
               out=None, workspace=None):
    """Full causal attention without a sink (GA layer)."""
    lib = load()
    B, n, _, hq, hkv, dqk, dv, _, o = _prefill_operands(q, k, v, None, out)
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    _check_workspace(workspace, need, q)
    _check_same(q, k, v, o)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.ga_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, n, hq, hkv, dqk, dv, scale,
                        rope_theta, rotary_fraction, pos_offset, _dtype_code(q), _ptr(ws),
                        _ws_bytes(ws), _stream(q))
    _raise(st)
    return o


def _decode_caches(k_cache, v_cache, layout, B, rows, dqk, cache_dtypes):
    """Ring caches [B, rows, Hkv, d]; contiguous caches [total_rows, Hkv, d]."""
    if layout == KV_RING:
        _, _, hkv, _ = _dims(k_cache, "k_cache", 4)
        _expect(k_cache, "k_cache", (B, rows, hkv, dqk), cache_dtypes)
        _expect(v_cache, "v_cache", (B, rows, hkv, None), cache_dtypes)
    elif layout == KV_CONTIGUOUS:
        total, hkv, _ = _dims(k_cache, "k_cache", 3)
        _expect(k_cache, "k_cache", (total, hkv, dqk), cache_dtypes)
        _expect(v_cache, "v_cache", (total, hkv, None), cache_dtypes)
    else:
        raise ValueError("layout must be KV_RING or KV_CONTIGUOUS")
    if v_cache.dtype != k_cache.dtype:
        raise TypeError("k_cache and v_cache must have the same dtype")
    return hkv, v_cache.shape[-1]


def swa_sink_decode(q, k_cache, v_cache, pos, max_pos, layout=KV_RING, seq_offsets=None,
                    sink=None, window=128, scale=0.0, rope_theta=10000.0, rotary_fraction=0.0,
                    out=None, workspace=None):
    """q [B,Hq,d_qk] against a ring [B,W,Hkv,d] or packed [rows,Hkv,d] cache -> o [B,Hq,d_v]."""
    lib = load()
    B, hq, dqk = _dims(q, "q", 3)
    if q.dtype not in _FLOAT:
        raise TypeError(f"q has dtype {q.dtype}, expected float32 or bfloat16")
    hkv, dv = _decode_caches(k_cache, v_cache, layout, B, window, dqk, (q.dtype,))
    _positions(pos, B, seq_offsets, layout == KV_CONTIGUOUS)
    sink = _sink(sink, q, hq)
    o = _out(out, (B, hq, dv), q.dtype, q.device)
    need = lib.hswa_decode_workspace_size(layout, B, hq, dv, window, int(max_pos))
    _check_workspace(workspace, need, q)
    _check_same(q, k_cache, v_cache, o, pos, seq_offsets)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), layout, _ptr(seq_offsets),
                             _ptr(pos), _ptr(sink), _ptr(o), B, hq, hkv, dqk, dv, window,
                             int(max_pos), scale, rope_theta, rotary_fraction, _dtype_code(q),
                             _ptr(ws), _ws_bytes(ws), _stream(q))
    _raise(st)
    return o


# Bytes of the library's static decode scratch (HSWA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def swa_sink_decode_noalloc(q, k_cache, v_cache, pos, max_pos, layout=KV_RING, seq_offsets=None,
                            sink=None, window=128, scale=0.0, rope_theta=10000.0,
                            rotary_fraction=0.0, out=None):
    """swa_sink_decode with its scratch in the library's static device array
    (no workspace is allocated; pass `out` to allocate nothing at all)."""
    lib = load()
    B, hq, dqk = _dims(q, "q", 3)
    if q.dtype not in _FLOAT:
        raise TypeError(f"q has dtype {q.dtype}, expected float32 or bfloat16")
    hkv, dv = _decode_caches(k_cache, v_cache, layout, B, window, dqk, (q.dtype,))
    _positions(pos, B, seq_offsets, layout == KV_CONTIGUOUS)
    sink = _sink(sink, q, hq)
    o = _out(out, (B, hq, dv), q.dtype, q.device)
    _check_same(q, k_cache, v_cache, o, pos, seq_offsets)
    st = lib.swa_sink_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), layout,
                                     _ptr(seq_offsets), _ptr(pos), _ptr(sink), _ptr(o), B, hq, hkv,
                                     dqk, dv, window, int(max_pos), scale, rope_theta,
                                     rotary_fraction, _dtype_code(q), _stream(q))
    _raise(st)
    return o


def decode_multi_workspace_size(layout, batch, q_len, hq, d_v, window, ring_slots, max_pos):
    return load().hswa_decode_multi_workspace_size(layout, batch, q_len, hq, d_v, window,
                                                   ring_slots, max_pos)


def swa_sink_decode_multi(q, k_cache, v_cache, pos, max_pos, layout=KV_RING, ring_slots=0,
                          seq_offsets=None, sink=None, window=128, scale=0.0, rope_theta=10000.0,
                          rotary_fraction=0.0, out=None, workspace=None):
    """q [B,T,Hq,d_qk]: T queries per sequence at pos[b] .. pos[b] + T - 1 against a
    ring [B,S,Hkv,d] (S = ring_slots >= window + T - 1) or packed [rows,Hkv,d] cache
    -> o [B,T,Hq,d_v]."""
    lib = load()
    B, T, hq, dqk = _dims(q, "q", 4)
    if q.dtype not in _FLOAT:
        raise TypeError(f"q has dtype {q.dtype}, expected float32 or bfloat16")
    hkv, dv = _decode_caches(k_cache, v_cache, layout, B, ring_slots, dqk, (q.dtype,))
    _positions(pos, B, seq_offsets, layout == KV_CONTIGUOUS)
    sink = _sink(sink, q, hq)
    o = _out(out, (B, T, hq, dv), q.dtype, q.device)
    need = lib.hswa_decode_multi_workspace_size(layout, B, T, hq, dv, window, ring_slots,
                                                int(max_pos))
    _check_workspace(workspace, need, q)
    _check_same(q, k_cache, v_cache, o, pos, seq_offsets)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_decode_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), layout, ring_slots,
                                   _ptr(seq_offsets), _ptr(pos), _ptr(sink), _ptr(o), B, T, hq,
                                   hkv, dqk, dv, window, int(max_pos), scale, rope_theta,
                                   rotary_fraction, _dtype_code(q), _ptr(ws), _ws_bytes(ws),
                                   _stream(q))
    _raise(st)
    return o


def kv_cache_append(k_new, v_new, k_cache, v_cache, pos, max_pos, layout=KV_RING, ring_slots=0,
                    seq_offsets=None, rope_theta=10000.0, rotary_fraction=0.0, k_scale=None,
                    v_scale=None):
    """Write k_new [B,T,Hkv,d_qk] and v_new [B,T,Hkv,d_v] (token t at pos[b] + t) into
    a ring or contiguous cache, keys rotated.  An E4M3 cache (uint8 or
    float8_e4m3fn) needs k_scale and v_scale.  Modifies the caches in place."""
    lib = load()
    B, T, hkv, dqk = _dims(k_new, "k_new", 4)
    if k_new.dtype not in _FLOAT:
        raise TypeError(f"k_new has dtype {k_new.dtype}, expected float32 or bfloat16")
    _expect(v_new, "v_new", (B, T, hkv, None), (k_new.dtype,))
    dv = v_new.shape[-1]
    fp8 = k_cache.dtype in _E4M3
    cache_dtypes = _E4M3 if fp8 else (k_new.dtype,)
    if not fp8 and k_cache.dtype != k_new.dtype:
        raise TypeError("a bf16 / fp32 cache has the type of the new keys and values")
    chkv, cdv = _decode_caches(k_cache, v_cache, layout, B, ring_slots, dqk, cache_dtypes)
    if chkv != hkv or cdv != dv:
        raise ValueError(f"caches hold {chkv} kv heads of {cdv} value dims; the new tokens "
                         f"{hkv} of {dv}")
    _positions(pos, B, seq_offsets, layout == KV_CONTIGUOUS)
    if fp8:
        _scales(k_scale, v_scale, hkv)
    _check_same(k_new, v_new, k_cache, v_cache, pos, seq_offsets)
    if fp8:
        _check_same(k_new, k_scale, v_scale)
        st = lib.kv_cache_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_scale), _ptr(v_scale), layout, ring_slots,
                                     _ptr(seq_offsets), _ptr(pos), B, T, hkv, dqk, dv,
                                     int(max_pos), rope_theta, rotary_fraction,
                                     _dtype_code(k_new), _stream(k_new))
    else:
        st = lib.kv_cache_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), layout,
                                 ring_slots, _ptr(seq_offsets), _ptr(pos), B, T, hkv, dqk, dv,
                                 int(max_pos), rope_theta, rotary_fraction, _dtype_code(k_new),
                                 _stream(k_new))
    _raise(st)


def swa_sink_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, pos, max_pos, layout=KV_RING,
                        seq_offsets=None, sink=None, window=128, scale=0.0, rope_theta=10000.0,
                        rotary_fraction=0.0, out=None, workspace=None):
    """swa_sink_decode over E4M3 caches: the value of a code is e4m3(code) times
    k_scale[g] (K) or v_scale[g] (V) of its kv head g."""
    lib = load()
    B, hq, dqk = _dims(q, "q", 3)
    if q.dtype not in _FLOAT:
        raise TypeError(f"q has dtype {q.dtype}, expected float32 or bfloat16")
    hkv, dv = _decode_caches(k_cache, v_cache, layout, B, window, dqk, _E4M3)
    _scales(k_scale, v_scale, hkv)
    _positions(pos, B, seq_offsets, layout == KV_CONTIGUOUS)
    sink = _sink(sink, q, hq)
    o = _out(out, (B, hq, dv), q.dtype, q.device)
    need = lib.hswa_decode_workspace_size(layout, B, hq, dv, window, int(max_pos))
    _check_workspace(workspace, need, q)
    _check_same(q, k_cache, v_cache, o, pos, seq_offsets, k_scale, v_scale)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                 _ptr(v_scale), layout, _ptr(seq_offsets), _ptr(pos), _ptr(sink),
                                 _ptr(o), B, hq, hkv, dqk, dv, window, int(max_pos), scale,
                                 rope_theta, rotary_fraction, _dtype_code(q), _ptr(ws),
                                 _ws_bytes(ws), _stream(q))
    _raise(st)
    return o


def _sparse_operands(q, k, v, sel_idx, sel_count, sink, out, kv_dtypes):
    B, n, hq, dqk = _dims(q, "q", 4)
    if q.dtype not in _FLOAT:
        raise TypeError(f"q has dtype {q.dtype}, expected float32 or bfloat16")
    _, _, hkv, _ = _dims(k, "k", 4)
    _expect(k, "k", (B, n, hkv, dqk), kv_dtypes)
    _expect(v, "v", (B, n, hkv, None), kv_dtypes)
    if v.dtype != k.dtype:
        raise TypeError("k and v must have the same dtype")
    if hkv == 0 or hq % hkv != 0:
        raise ValueError(f"hq ({hq}) must be a positive multiple of hkv ({hkv})")
    _expect(sel_idx, "sel_idx", (B, n, hkv, None), (torch.int32,))
    _expect(sel_count, "sel_count", (B, n, hkv), (torch.int32,))
    dv = v.shape[3]
    sink = _sink(sink, q, hq)
    o = _out(out, (B, n, hq, dv), q.dtype, q.device)
    return B, n, hq, hkv, dqk, dv, sel_idx.shape[-1], sink, o


def sparse_sink_attn(q, k, v, sel_idx, sel_count, sink=None, recent_window=128, scale=0.0,
                     rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0, out=None,
                     workspace=None):
    """Recent window plus selected tokens per (query, kv head) -> o [B,n,Hq,d_v]."""
    lib = load()
    B, n, hq, hkv, dqk, dv, max_sel, sink, o = _sparse_operands(q, k, v, sel_idx, sel_count, sink,
                                                                out, (q.dtype,))
    need = lib.hswa_sparse_workspace_size(B, n, hkv, dqk, rotary_fraction)
    _check_workspace(workspace, need, q)
    _check_same(q, k, v, o, sel_idx, sel_count)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.sparse_sink_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(sel_idx), _ptr(sel_count), max_sel,
                              recent_window, _ptr(sink), _ptr(o), B, n, hq, hkv, dqk, dv, scale,
                              rope_theta, rotary_fraction, pos_offset, _dtype_code(q), _ptr(ws),
                              _ws_bytes(ws), _stream(q))
    _raise(st)
    return o


def sparse_sink_attn_fp8(q, k, v, k_scale, v_scale, sel_idx, sel_count, sink=None,
                         recent_window=128, scale=0.0, rope_theta=10000.0, rotary_fraction=0.0,
                         pos_offset=0, out=None, workspace=None):
    """sparse_sink_attn over E4M3 K/V codes with per-kv-head scales."""
    lib = load()
    B, n, hq, hkv, dqk, dv, max_sel, sink, o = _sparse_operands(q, k, v, sel_idx, sel_count, sink,
                                                                out, _E4M3)
    _scales(k_scale, v_scale, hkv)
    need = lib.hswa_sparse_workspace_size(B, n, hkv, dqk, rotary_fraction)
    _check_workspace(workspace, need, q)
    _check_same(q, k, v, o, sel_idx, sel_count, k_scale, v_scale)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.sparse_sink_attn_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
                                  _ptr(sel_idx), _ptr(sel_count), max_sel, recent_window,
                                  _ptr(sink), _ptr(o), B, n, hq, hkv, dqk, dv, scale, rope_theta,
                                  rotary_fraction, pos_offset, _dtype_code(q), _ptr(ws),
                                  _ws_bytes(ws), _stream(q))
    _raise(st)
    return o


def sparse_select_tokens(q, k, max_sel=1024, recent_window=128, scale=0.0, rope_theta=1.0e7,
                         rotary_fraction=0.0, pos_offset=0, out=None, workspace=None):
    """Selected-token lists for the sparse layers from the full-attention
    layer's q [B,n,Hq,192] and k [B,n,Hkv,192] (bf16, Hq = 16 Hkv):
    returns (sel_idx int32 [B,n,Hkv,max_sel], sel_count int32 [B,n,Hkv])."""
    lib = load()
    B, n, hq, dqk = _dims(q, "q", 4)
    if q.dtype not in _FLOAT:
        raise TypeError(f"q has dtype {q.dtype}, expected float32 or bfloat16")
    _, _, hkv, _ = _dims(k, "k", 4)
    _expect(k, "k", (B, n, hkv, dqk), (q.dtype,))
    if out is not None:
        idx, cnt = out
        _expect(idx, "sel_idx", (B, n, hkv, max_sel), (torch.int32,))
        _expect(cnt, "sel_count", (B, n, hkv), (torch.int32,))
    else:
        idx = torch.empty((B, n, hkv, max_sel), dtype=torch.int32, device=q.device)
        cnt = torch.empty((B, n, hkv), dtype=torch.int32, device=q.device)
    need = lib.hswa_select_workspace_size(B, n, hq, hkv, dqk, rotary_fraction)
    _check_workspace(workspace, need, q)
    _check_same(q, k, idx, cnt)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.sparse_select_tokens(_ptr(q), _ptr(k), _ptr(idx), _ptr(cnt), max_sel, recent_window,
                                  B, n, hq, hkv, dqk, scale, rope_theta, rotary_fraction,
                                  pos_offset, _dtype_code(q), _ptr(ws), _ws_bytes(ws), _stream(q))
    _raise(st)
    return idx, cnt


def gather_probe(k, v, idx, tiles_per_wave, out=None):
    """Random-row gather probe (include/hswa_measure.h): k bf16 [rows, 192],
    v bf16 [rows, 128], idx int32 [nwaves * tiles_per_wave * 32] -> one
    uint32 checksum (as int32) per wavefront."""
    lib = load()
    rows = _dims(k, "k", 2)[0]
    _expect(k, "k", (rows, 192), (torch.bfloat16,))
    _expect(v, "v", (rows, 128), (torch.bfloat16,))
    n_idx = _dims(idx, "idx", 1)[0]
    if idx.dtype != torch.int32 or n_idx % (32 * tiles_per_wave) != 0 or n_idx == 0:
        raise ValueError("idx must be int32 with a positive multiple of 32 * tiles_per_wave entries")
    nwaves = n_idx // (32 * tiles_per_wave)
    o = _out(out, (nwaves,), torch.int32, k.device)
    _check_same(k, v, idx, o)
    _raise(lib.hswa_gather_probe(_ptr(k), _ptr(v), rows, _ptr(idx), nwaves, tiles_per_wave, _ptr(o),
                                 _stream(k)))
    return o


def stream_probe(src, dst, blocks, out=None):
    """Streaming probe (include/hswa_measure.h): reads every byte of src,
    overwrites every byte of dst (either may be None), each wavefront of
    blocks * 4 walking its shares of both together -> one uint32 checksum
    (as int32) per wavefront."""
    lib = load()
    ref = src if src is not None else dst
    if ref is None:
        raise ValueError("stream_probe needs a source or a destination")
    nr = 0 if src is None else src.numel() * src.element_size()
    nw = 0 if dst is None else dst.numel() * dst.element_size()
    for t, name in ((src, "src"), (dst, "dst")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if nr % 1024 or nw % 1024:
        raise ValueError("src and dst sizes must be multiples of 1024 bytes")
    if blocks <= 0:
        raise ValueError("blocks must be positive")
    o = _out(out, (4 * blocks,), torch.int32, ref.device)
    _check_same(*[t for t in (src, dst) if t is not None], o)
    _raise(lib.hswa_stream_probe(None if src is None else _ptr(src), nr,
                                 None if dst is None else _ptr(dst), nw, blocks, _ptr(o),
                                 _stream(ref)))
    return o
