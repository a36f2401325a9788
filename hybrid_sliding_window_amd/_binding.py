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

# Every symbol include/hswa.h declares, with (restype, argtypes).
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
    for t in ts:
        if t is None:
            continue
        if t.device != ref.device:
            raise ValueError("all tensors must live on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _raise(status):
    if status != 0:
        raise HswaError(status, load().hswa_last_error().decode())


def _sink(sink, q):
    if sink is None:
        return None
    if sink.dtype != torch.float32 or sink.device != q.device or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 tensor on the query's device")
    return sink


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefill_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction):
    return load().hswa_prefill_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction)


def sparse_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction):
    return load().hswa_sparse_workspace_size(batch, seqlen, hkv, d_qk, rotary_fraction)


def decode_workspace_size(layout, batch, hq, d_v, window, max_pos):
    return load().hswa_decode_workspace_size(layout, batch, hq, d_v, window, max_pos)


def swa_sink_prefill(q, k, v, sink=None, window=128, scale=0.0, rope_theta=10000.0,
                     rotary_fraction=0.0, pos_offset=0, out=None, workspace=None):
    """q [B,n,Hq,d_qk], k [B,n,Hkv,d_qk], v [B,n,Hkv,d_v] -> o [B,n,Hq,d_v]."""
    lib = load()
    B, n, hq, dqk = q.shape
    hkv, dv = k.shape[2], v.shape[3]
    sink = _sink(sink, q)
    o = out if out is not None else torch.empty((B, n, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k, v, o)
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o), B, n, hq, hkv, dqk,
                              dv, window, scale, rope_theta, rotary_fraction, pos_offset,
                              _dtype_code(q), _ptr(ws), 0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def swa_sink_prefill_chunk(q, k, v, sink=None, window=128, scale=0.0, rope_theta=10000.0,
                           rotary_fraction=0.0, pos_offset=0, out=None, workspace=None):
    """The last q_len positions of sequences of kv_len tokens (a chunk behind a
    cached prefix): q [B,q_len,Hq,d_qk], k [B,kv_len,Hkv,d_qk],
    v [B,kv_len,Hkv,d_v] -> o [B,q_len,Hq,d_v].  window=0 with sink=None is
    the GA layer's chunk."""
    lib = load()
    B, nq, hq, dqk = q.shape
    n, hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    sink = _sink(sink, q)
    o = out if out is not None else torch.empty((B, nq, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k, v, o)
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o), B, nq, n, hq,
                                    hkv, dqk, dv, window, scale, rope_theta, rotary_fraction,
                                    pos_offset, _dtype_code(q), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def swa_sink_prefill_chunk_cached(q, k_cache, v_cache, sink=None, window=128, scale=0.0,
                                  rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0, out=None,
                                  workspace=None):
    """swa_sink_prefill_chunk over a cache whose keys are stored already rotated
    (as kv_cache_append writes them): k_cache [B,kv_len,Hkv,d_qk]."""
    lib = load()
    B, nq, hq, dqk = q.shape
    n, hkv, dv = k_cache.shape[1], k_cache.shape[2], v_cache.shape[3]
    sink = _sink(sink, q)
    o = out if out is not None else torch.empty((B, nq, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k_cache, v_cache, o)
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_prefill_chunk_cached(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sink),
                                           _ptr(o), B, nq, n, hq, hkv, dqk, dv, window, scale,
                                           rope_theta, rotary_fraction, pos_offset, _dtype_code(q),
                                           _ptr(ws), 0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def ga_prefill(q, k, v, scale=0.0, rope_theta=1.0e7, rotary_fraction=0.0, pos_offset=0,
               out=None, workspace=None):
    """Full causal attention without a sink (GA layer)."""
    lib = load()
    B, n, hq, dqk = q.shape
    hkv, dv = k.shape[2], v.shape[3]
    o = out if out is not None else torch.empty((B, n, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k, v, o)
    need = lib.hswa_prefill_workspace_size(B, n, hkv, dqk, rotary_fraction)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.ga_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, n, hq, hkv, dqk, dv, scale,
                        rope_theta, rotary_fraction, pos_offset, _dtype_code(q), _ptr(ws),
                        0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def swa_sink_decode(q, k_cache, v_cache, pos, max_pos, layout=KV_RING, seq_offsets=None,
                    sink=None, window=128, scale=0.0, rope_theta=10000.0, rotary_fraction=0.0,
                    out=None, workspace=None):
    """q [B,Hq,d_qk] against a ring [B,W,Hkv,d] or packed [rows,Hkv,d] cache -> o [B,Hq,d_v]."""
    lib = load()
    B, hq, dqk = q.shape
    hkv, dv = k_cache.shape[-2], v_cache.shape[-1]
    sink = _sink(sink, q)
    if pos.dtype != torch.int64:
        raise TypeError("pos must be int64")
    if seq_offsets is not None and seq_offsets.dtype != torch.int64:
        raise TypeError("seq_offsets must be int64")
    o = out if out is not None else torch.empty((B, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k_cache, v_cache, o, pos, seq_offsets)
    need = lib.hswa_decode_workspace_size(layout, B, hq, dv, window, int(max_pos))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), layout, _ptr(seq_offsets),
                             _ptr(pos), _ptr(sink), _ptr(o), B, hq, hkv, dqk, dv, window,
                             int(max_pos), scale, rope_theta, rotary_fraction, _dtype_code(q),
                             _ptr(ws), 0 if ws is None else ws.numel(), _stream(q))
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
    B, T, hq, dqk = q.shape
    hkv, dv = k_cache.shape[-2], v_cache.shape[-1]
    sink = _sink(sink, q)
    if pos.dtype != torch.int64:
        raise TypeError("pos must be int64")
    if seq_offsets is not None and seq_offsets.dtype != torch.int64:
        raise TypeError("seq_offsets must be int64")
    o = out if out is not None else torch.empty((B, T, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k_cache, v_cache, o, pos, seq_offsets)
    need = lib.hswa_decode_multi_workspace_size(layout, B, T, hq, dv, window, ring_slots,
                                                int(max_pos))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_decode_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), layout, ring_slots,
                                   _ptr(seq_offsets), _ptr(pos), _ptr(sink), _ptr(o), B, T, hq,
                                   hkv, dqk, dv, window, int(max_pos), scale, rope_theta,
                                   rotary_fraction, _dtype_code(q), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def kv_cache_append(k_new, v_new, k_cache, v_cache, pos, max_pos, layout=KV_RING, ring_slots=0,
                    seq_offsets=None, rope_theta=10000.0, rotary_fraction=0.0, k_scale=None,
                    v_scale=None):
    """Write k_new [B,T,Hkv,d_qk] and v_new [B,T,Hkv,d_v] (token t at pos[b] + t) into
    a ring or contiguous cache, keys rotated.  An E4M3 cache (uint8 or
    float8_e4m3fn) needs k_scale and v_scale.  Modifies the caches in place."""
    lib = load()
    B, T, hkv, dqk = k_new.shape
    dv = v_new.shape[-1]
    if pos.dtype != torch.int64:
        raise TypeError("pos must be int64")
    if seq_offsets is not None and seq_offsets.dtype != torch.int64:
        raise TypeError("seq_offsets must be int64")
    _check_same(k_new, v_new, k_cache, v_cache, pos, seq_offsets)
    fp8 = k_cache.dtype in (torch.uint8, torch.float8_e4m3fn)
    if fp8:
        for t in (k_scale, v_scale):
            if t is None or t.dtype != torch.float32 or t.numel() != hkv:
                raise ValueError("an E4M3 cache needs float32 k_scale and v_scale, one per kv head")
        _check_same(k_new, k_scale, v_scale)
        st = lib.kv_cache_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_scale), _ptr(v_scale), layout, ring_slots,
                                     _ptr(seq_offsets), _ptr(pos), B, T, hkv, dqk, dv,
                                     int(max_pos), rope_theta, rotary_fraction,
                                     _dtype_code(k_new), _stream(k_new))
    else:
        if k_cache.dtype != k_new.dtype or v_cache.dtype != v_new.dtype:
            raise TypeError("a bf16 / fp32 cache has the type of the new keys and values")
        st = lib.kv_cache_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), layout,
                                 ring_slots, _ptr(seq_offsets), _ptr(pos), B, T, hkv, dqk, dv,
                                 int(max_pos), rope_theta, rotary_fraction, _dtype_code(k_new),
                                 _stream(k_new))
    _raise(st)


def _fp8_cache(t):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("an FP8 cache holds E4M3 codes: uint8 or float8_e4m3fn")
    return t


def swa_sink_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, pos, max_pos, layout=KV_RING,
                        seq_offsets=None, sink=None, window=128, scale=0.0, rope_theta=10000.0,
                        rotary_fraction=0.0, out=None, workspace=None):
    """swa_sink_decode over E4M3 caches: the value of a code is e4m3(code) times
    k_scale[g] (K) or v_scale[g] (V) of its kv head g."""
    lib = load()
    B, hq, dqk = q.shape
    hkv, dv = k_cache.shape[-2], v_cache.shape[-1]
    _fp8_cache(k_cache)
    _fp8_cache(v_cache)
    for t in (k_scale, v_scale):
        if t.dtype != torch.float32 or t.numel() != hkv:
            raise ValueError("k_scale and v_scale must be float32 with one entry per kv head")
    sink = _sink(sink, q)
    if pos.dtype != torch.int64:
        raise TypeError("pos must be int64")
    if seq_offsets is not None and seq_offsets.dtype != torch.int64:
        raise TypeError("seq_offsets must be int64")
    o = out if out is not None else torch.empty((B, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k_cache, v_cache, o, pos, seq_offsets, k_scale, v_scale)
    need = lib.hswa_decode_workspace_size(layout, B, hq, dv, window, int(max_pos))
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.swa_sink_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                 _ptr(v_scale), layout, _ptr(seq_offsets), _ptr(pos), _ptr(sink),
                                 _ptr(o), B, hq, hkv, dqk, dv, window, int(max_pos), scale,
                                 rope_theta, rotary_fraction, _dtype_code(q), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def sparse_sink_attn(q, k, v, sel_idx, sel_count, sink=None, recent_window=128, scale=0.0,
                     rope_theta=10000.0, rotary_fraction=0.0, pos_offset=0, out=None,
                     workspace=None):
    """Recent window plus selected tokens per (query, kv head) -> o [B,n,Hq,d_v]."""
    lib = load()
    B, n, hq, dqk = q.shape
    hkv, dv = k.shape[2], v.shape[3]
    max_sel = sel_idx.shape[-1]
    sink = _sink(sink, q)
    if sel_idx.dtype != torch.int32 or sel_count.dtype != torch.int32:
        raise TypeError("sel_idx and sel_count must be int32")
    o = out if out is not None else torch.empty((B, n, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k, v, o, sel_idx, sel_count)
    need = lib.hswa_sparse_workspace_size(B, n, hkv, dqk, rotary_fraction)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.sparse_sink_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(sel_idx), _ptr(sel_count), max_sel,
                              recent_window, _ptr(sink), _ptr(o), B, n, hq, hkv, dqk, dv, scale,
                              rope_theta, rotary_fraction, pos_offset, _dtype_code(q), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def sparse_sink_attn_fp8(q, k, v, k_scale, v_scale, sel_idx, sel_count, sink=None,
                         recent_window=128, scale=0.0, rope_theta=10000.0, rotary_fraction=0.0,
                         pos_offset=0, out=None, workspace=None):
    """sparse_sink_attn over E4M3 K/V codes with per-kv-head scales."""
    lib = load()
    B, n, hq, dqk = q.shape
    hkv, dv = k.shape[2], v.shape[3]
    max_sel = sel_idx.shape[-1]
    _fp8_cache(k)
    _fp8_cache(v)
    for t in (k_scale, v_scale):
        if t.dtype != torch.float32 or t.numel() != hkv:
            raise ValueError("k_scale and v_scale must be float32 with one entry per kv head")
    sink = _sink(sink, q)
    if sel_idx.dtype != torch.int32 or sel_count.dtype != torch.int32:
        raise TypeError("sel_idx and sel_count must be int32")
    o = out if out is not None else torch.empty((B, n, hq, dv), dtype=q.dtype, device=q.device)
    _check_same(q, k, v, o, sel_idx, sel_count, k_scale, v_scale)
    need = lib.hswa_sparse_workspace_size(B, n, hkv, dqk, rotary_fraction)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.sparse_sink_attn_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
                                  _ptr(sel_idx), _ptr(sel_count), max_sel, recent_window,
                                  _ptr(sink), _ptr(o), B, n, hq, hkv, dqk, dv, scale, rope_theta,
                                  rotary_fraction, pos_offset, _dtype_code(q), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return o


def sparse_select_tokens(q, k, max_sel=1024, recent_window=128, scale=0.0, rope_theta=1.0e7,
                         rotary_fraction=0.0, pos_offset=0, out=None, workspace=None):
    """Selected-token lists for the sparse layers from the full-attention
    layer's q [B,n,Hq,192] and k [B,n,Hkv,192] (bf16, Hq = 16 Hkv):
    returns (sel_idx int32 [B,n,Hkv,max_sel], sel_count int32 [B,n,Hkv])."""
    lib = load()
    B, n, hq, dqk = q.shape
    hkv = k.shape[2]
    if out is not None:
        idx, cnt = out
    else:
        idx = torch.empty((B, n, hkv, max_sel), dtype=torch.int32, device=q.device)
        cnt = torch.empty((B, n, hkv), dtype=torch.int32, device=q.device)
    _check_same(q, k, idx, cnt)
    need = lib.hswa_select_workspace_size(B, n, hq, hkv, dqk, rotary_fraction)
    ws = workspace if workspace is not None else _workspace(need, q.device)
    st = lib.sparse_select_tokens(_ptr(q), _ptr(k), _ptr(idx), _ptr(cnt), max_sel, recent_window,
                                  B, n, hq, hkv, dqk, scale, rope_theta, rotary_fraction,
                                  pos_offset, _dtype_code(q), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(q))
    _raise(st)
    return idx, cnt
