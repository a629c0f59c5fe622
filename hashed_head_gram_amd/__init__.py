"""Python binding of libpagegram.so (the MI355X n-gram memory path).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. The functions carry the C entry points' names and take torch device
tensors (PyTorch supplies device memory and the current stream). There is no
CPU fallback: importing works without the library, but the first call raises
if libpagegram.so has not been built (python -m hashed_head_gram_amd.build).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagegram.so")

PG_OK, PG_EINVAL, PG_EUNSUPPORTED, PG_EHIP, PG_ERANGE = 0, -1, -2, -3, -4
PG_PAGEGRAM, PG_ENGRAM = 0, 1
PG_F32, PG_BF16, PG_NF4 = 0, 1, 2
PG_GATE_SCALAR, PG_GATE_ENGRAM = 0, 1
PG_STAGE_PAGE, PG_STAGE_ROW = 0, 1
PG_MAX_ORDERS, PG_MAX_HEADS = 4, 16

_i32, _i64, _u64, _f32, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                               ctypes.c_float, ctypes.c_void_p)


class PgLayout(ctypes.Structure):
    _fields_ = [("kind", _i32), ("n_min", _i32), ("n_max", _i32), ("K", _i32),
                ("S", _i32), ("r", _i32),
                ("pages", _i64 * PG_MAX_ORDERS),
                ("head_rows", (_i64 * PG_MAX_HEADS) * PG_MAX_ORDERS),
                ("hash_seed", _u64), ("use_signs", _i32), ("pad_id", _i32)]


class PgTable(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("reserved", _i32), ("data", _vp),
                ("scales", _vp), ("n_rows", _i64)]


class PgFuse(ctypes.Structure):
    _fields_ = [("gate", _i32), ("dtype", _i32), ("d", _i32), ("M", _i32),
                ("g", _f32), ("eps", _f32), ("gamma_h", _vp), ("gamma_k", _vp),
                ("gamma_u", _vp), ("conv_w", _vp), ("conv_k", _i32),
                ("conv_dil", _i32), ("increment_only", _i32), ("reserved", _i32)]


class PgCacheStats(ctypes.Structure):
    _fields_ = [("tokens", _i64), ("lookups", _i64), ("distinct", _i64), ("misses", _i64)]


_P = ctypes.POINTER
_SIGS = {
    "pg_index": (_i32, [_P(PgLayout), _vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp,
                        _vp, _vp, _vp, _vp]),
    "pg_gather": (_i32, [_P(PgLayout), _P(PgTable), _vp, _vp, _i64, _i32, _vp, _vp]),
    "pg_index_gather": (_i32, [_P(PgLayout), _P(PgTable), _vp, _i64, _i64, _vp,
                               _i64, _i32, _vp, _vp, _vp]),
    "pg_project_gate": (_i32, [_P(PgFuse), _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                               _vp, _i64, _vp]),
    "pg_forward": (_i32, [_P(PgLayout), _P(PgTable), _P(PgFuse), _vp, _i64, _i64,
                          _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp]),
    "pg_forward_noalloc": (_i32, [_P(PgLayout), _P(PgTable), _P(PgFuse), _vp, _i64, _i64,
                                  _vp, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pg_index_records": (_i32, [_P(PgLayout), _vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "pg_project_gathered": (_i32, [_P(PgLayout), _P(PgTable), _P(PgFuse), _vp, _i64, _i64,
                                   _vp, _vp, _vp, _vp]),
    "pg_stage_geometry": (_i32, [_P(PgLayout), _i32, _i32, _i64, _P(_i64), _P(_i64),
                                 _P(_i64)]),
    "pg_stage_rows": (_i32, [_P(PgLayout), _P(PgTable), _i32, _vp, _i64, _P(PgTable), _vp, _vp,
                             _vp, _vp, _i64, _vp]),
    "pg_gather_staged": (_i32, [_P(PgLayout), _P(PgTable), _vp, _vp, _i64, _i32, _vp, _vp]),
    "pg_quantize_fp8": (_i32, [_vp, _i32, _i64, _i32, _vp, _vp]),
    "pg_index_gather_fp8": (_i32, [_P(PgLayout), _P(PgTable), _vp, _i64, _i64, _vp,
                                   _i64, _i32, _vp, _vp, _vp]),
    "pg_project_gate_fp8": (_i32, [_P(PgFuse), _vp, _i64, _i64, _i64, _vp, _i32, _i32,
                                   _vp, _vp, _vp, _i64, _vp]),
    "pg_forward_fp8": (_i32, [_P(PgLayout), _P(PgTable), _P(PgFuse), _vp, _i64, _i64,
                              _vp, _i64, _vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _vp]),
    "pg_engram_project": (_i32, [_P(PgFuse), _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "pg_engram_project_fp8": (_i32, [_P(PgFuse), _vp, _i64, _i64, _i64, _vp, _i32, _i32, _vp,
                                     _vp, _i64, _vp]),
    "pg_engram_gate": (_i32, [_P(PgFuse), _i64, _i64, _vp, _i64, _vp]),
    "pg_engram_mix": (_i32, [_P(PgFuse), _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "pg_read_probe": (_i32, [_vp, _i64, _vp, _vp]),
    "pg_strerror": (ctypes.c_char_p, [_i32]),
    "pg_hash_version": (ctypes.c_uint32, []),
    "pg_layout_rows": (_i32, [_P(PgLayout), _P(_i64)]),
    "pg_workspace_size": (_i64, [_P(PgLayout), _P(PgFuse), _i64, _i64]),
    "pg_backward_workspace_size": (_i64, [_P(PgLayout), _P(PgFuse), _i64, _i64]),
    "pg_backward_scalar": (_i32, [_P(PgLayout), _P(PgFuse), _vp, _vp, _vp, _vp, _vp, _i64,
                                  _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "pg_row_rms_step": (_i32, [_P(PgLayout), _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _f32,
                               _f32, _f32, _f32, _vp]),
    "pg_row_rms_flush": (_i32, [_P(PgLayout), _vp, _vp, _vp, _i64, _f32, _f32, _f32, _vp]),
    "pg_flash_blocks": (_i32, [_P(PgLayout), _i32, _vp, _i64, _vp]),
    "pg_lru_cache_sim": (_i32, [_vp, _i64, _i32, _i64, _P(PgCacheStats)]),
}

_lib = None


class PagegramError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().pg_strerror(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m hashed_head_gram_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ----------------------------------------------------------------------------
# Struct builders


def make_layout(kind, K, r, S=1, pages=(), head_rows=(), hash_seed=0,
                use_signs=1, n_min=2, n_max=3, pad_id=0):
    """pg_layout from plain values; ``kind`` is "pagegram"/"engram" or 0/1.
    head_rows is flat in (order, head) order."""
    L = PgLayout()
    L.kind = {"pagegram": PG_PAGEGRAM, "engram": PG_ENGRAM}.get(kind, kind)
    L.n_min, L.n_max, L.K, L.S, L.r = n_min, n_max, K, S, r
    for i, p in enumerate(pages):
        L.pages[i] = int(p)
    for q, p in enumerate(head_rows):
        L.head_rows[q // K][q % K] = int(p)
    L.hash_seed = int(hash_seed)
    L.use_signs = int(use_signs)
    L.pad_id = int(pad_id)
    return L


def make_table(dtype, data, n_rows, scales=None):
    t = PgTable()
    t.dtype = dtype
    t.data = _ptr(data)
    t.scales = _ptr(scales)
    t.n_rows = int(n_rows)
    t._keep = (data, scales)
    return t


def make_fuse(gate, dtype, d, g=0.5, M=0, eps=1e-6, gamma_h=None, gamma_k=None,
              gamma_u=None, conv_w=None, conv_k=4, conv_dil=3, increment_only=0):
    f = PgFuse()
    f.gate, f.dtype, f.d, f.M = gate, dtype, int(d), int(M)
    f.g, f.eps = float(g), float(eps)
    f.gamma_h, f.gamma_k = _ptr(gamma_h), _ptr(gamma_k)
    f.gamma_u, f.conv_w = _ptr(gamma_u), _ptr(conv_w)
    f.conv_k, f.conv_dil, f.increment_only = int(conv_k), int(conv_dil), int(increment_only)
    f._keep = (gamma_h, gamma_k, gamma_u, conv_w)
    return f


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn, status):
    if status != PG_OK:
        raise PagegramError(fn, status)


# ----------------------------------------------------------------------------
# Entry points (same names as the C ABI)


def pg_layout_rows(layout):
    n = _i64()
    _check("pg_layout_rows", lib().pg_layout_rows(ctypes.byref(layout), ctypes.byref(n)))
    return n.value


def pg_workspace_size(layout, fuse, B, T):
    v = lib().pg_workspace_size(ctypes.byref(layout) if layout is not None else None,
                                ctypes.byref(fuse), int(B), int(T))
    if v < 0:
        raise PagegramError("pg_workspace_size", v)
    return v


def pg_hash_version():
    return lib().pg_hash_version()


def pg_index(layout, tokens, canon_map, rows_out, signs_out, canon_out=None,
             hash_out=None, pages_out=None, dev_status=None, stream=None):
    """tokens int32 [B, T]; outputs as described in include/pagegram.h."""
    B, T = tokens.shape
    _check("pg_index", lib().pg_index(
        ctypes.byref(layout), _ptr(tokens), B, T, _ptr(canon_map), canon_map.numel(),
        _ptr(canon_out), _ptr(hash_out), _ptr(rows_out), _ptr(pages_out),
        _ptr(signs_out), _ptr(dev_status), _stream(stream)))


def pg_gather(layout, table, rows, signs, e_dtype, e_out, stream=None):
    _check("pg_gather", lib().pg_gather(
        ctypes.byref(layout), ctypes.byref(table), _ptr(rows), _ptr(signs),
        rows.shape[0], e_dtype, _ptr(e_out), _stream(stream)))


def pg_index_gather(layout, table, tokens, canon_map, e_dtype, e_out,
                    dev_status=None, stream=None):
    B, T = tokens.shape
    _check("pg_index_gather", lib().pg_index_gather(
        ctypes.byref(layout), ctypes.byref(table), _ptr(tokens), B, T,
        _ptr(canon_map), canon_map.numel(), e_dtype, _ptr(e_out),
        _ptr(dev_status), _stream(stream)))


def pg_project_gate(fuse, e, B, T, W, resid, out, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pg_project_gate", lib().pg_project_gate(
        ctypes.byref(fuse), _ptr(e), int(B), int(T), e.shape[-1], _ptr(W),
        _ptr(resid), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def pg_forward(layout, table, fuse, tokens, canon_map, W, resid, out, workspace,
               dev_status=None, stream=None):
    B, T = tokens.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pg_forward", lib().pg_forward(
        ctypes.byref(layout), ctypes.byref(table), ctypes.byref(fuse), _ptr(tokens),
        B, T, _ptr(canon_map), canon_map.numel(), _ptr(W), _ptr(resid), _ptr(out),
        _ptr(workspace), ws_bytes, _ptr(dev_status), _stream(stream)))


def pg_forward_noalloc(layout, table, fuse, tokens, canon_map, W, resid, out,
                       dev_status=None, stream=None):
    B, T = tokens.shape
    _check("pg_forward_noalloc", lib().pg_forward_noalloc(
        ctypes.byref(layout), ctypes.byref(table), ctypes.byref(fuse), _ptr(tokens),
        B, T, _ptr(canon_map), canon_map.numel(), _ptr(W), _ptr(resid), _ptr(out),
        _ptr(dev_status), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20


def records_bytes(layout, n_tok):
    """Bytes of pg_index_records' output: 16 per (head slot, token)."""
    return 16 * n_tok * (layout.n_max - layout.n_min + 1) * layout.K


def pg_index_records(layout, tokens, canon_map, rec_out, dev_status=None, stream=None):
    B, T = tokens.shape
    _check("pg_index_records", lib().pg_index_records(
        ctypes.byref(layout), _ptr(tokens), B, T, _ptr(canon_map), canon_map.numel(),
        _ptr(rec_out), _ptr(dev_status), _stream(stream)))


def pg_project_gathered(layout, table, fuse, rec, B, T, W, resid, out, stream=None):
    _check("pg_project_gathered", lib().pg_project_gathered(
        ctypes.byref(layout), ctypes.byref(table), ctypes.byref(fuse), _ptr(rec), int(B),
        int(T), _ptr(W), _ptr(resid), _ptr(out), _stream(stream)))


# ----------------------------------------------------------------------------
# The Engram gate's three stages (pg_project_gate runs them in order)


def _ws_bytes(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def pg_engram_project(fuse, e, B, T, W, h, workspace, stream=None):
    _check("pg_engram_project", lib().pg_engram_project(
        ctypes.byref(fuse), _ptr(e), int(B), int(T), e.shape[-1], _ptr(W), _ptr(h),
        _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def pg_engram_project_fp8(fuse, e8, B, T, W8, e_scale_exp, w_scale_exp, h, workspace,
                          stream=None):
    _check("pg_engram_project_fp8", lib().pg_engram_project_fp8(
        ctypes.byref(fuse), _ptr(e8), int(B), int(T), e8.shape[-1], _ptr(W8),
        int(e_scale_exp), int(w_scale_exp), _ptr(h), _ptr(workspace), _ws_bytes(workspace),
        _stream(stream)))


def pg_engram_gate(fuse, B, T, workspace, stream=None):
    _check("pg_engram_gate", lib().pg_engram_gate(
        ctypes.byref(fuse), int(B), int(T), _ptr(workspace), _ws_bytes(workspace),
        _stream(stream)))


def pg_engram_mix(fuse, B, T, h, out, workspace, stream=None):
    _check("pg_engram_mix", lib().pg_engram_mix(
        ctypes.byref(fuse), int(B), int(T), _ptr(h), _ptr(out), _ptr(workspace),
        _ws_bytes(workspace), _stream(stream)))


def pg_read_probe(src, sink, stream=None):
    """Streaming read of the whole tensor src (measurement utility)."""
    _check("pg_read_probe", lib().pg_read_probe(
        _ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))


# ----------------------------------------------------------------------------
# Staging from a host-resident table


def pg_stage_geometry(layout, table_dtype, n_tok, unit_kind=0):
    """(rows per unit, most units per step, workspace bytes); unit_kind
    PG_STAGE_PAGE (0) or PG_STAGE_ROW (1)."""
    u, m, w = _i64(), _i64(), _i64()
    _check("pg_stage_geometry", lib().pg_stage_geometry(
        ctypes.byref(layout), table_dtype, int(unit_kind), int(n_tok), ctypes.byref(u),
        ctypes.byref(m), ctypes.byref(w)))
    return u.value, m.value, w.value


def pg_stage_rows(layout, src, rows, cache, cache_rows, n_units, workspace, unit_first=None,
                  unit_kind=0, stream=None):
    """rows int64 [N, O, K] (device); src / cache pg_table structures."""
    _check("pg_stage_rows", lib().pg_stage_rows(
        ctypes.byref(layout), ctypes.byref(src), int(unit_kind), _ptr(rows), rows.shape[0],
        ctypes.byref(cache),
        _ptr(cache_rows), _ptr(n_units), _ptr(unit_first), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def pg_gather_staged(layout, cache, cache_rows, signs, e_dtype, e_out, stream=None):
    _check("pg_gather_staged", lib().pg_gather_staged(
        ctypes.byref(layout), ctypes.byref(cache), _ptr(cache_rows), _ptr(signs),
        cache_rows.shape[0], e_dtype, _ptr(e_out), _stream(stream)))


# ----------------------------------------------------------------------------
# FP8 (E4M3) operands


def pg_quantize_fp8(src, src_dtype, scale_exp, dst, stream=None):
    """dst (uint8, same element count) = E4M3(src * 2^scale_exp)."""
    _check("pg_quantize_fp8", lib().pg_quantize_fp8(
        _ptr(src), src_dtype, src.numel(), int(scale_exp), _ptr(dst), _stream(stream)))


def pg_index_gather_fp8(layout, table, tokens, canon_map, e_scale_exp, e_out,
                        dev_status=None, stream=None):
    B, T = tokens.shape
    _check("pg_index_gather_fp8", lib().pg_index_gather_fp8(
        ctypes.byref(layout), ctypes.byref(table), _ptr(tokens), B, T,
        _ptr(canon_map), canon_map.numel(), int(e_scale_exp), _ptr(e_out),
        _ptr(dev_status), _stream(stream)))


def pg_project_gate_fp8(fuse, e8, B, T, W8, e_scale_exp, w_scale_exp, resid, out,
                        workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pg_project_gate_fp8", lib().pg_project_gate_fp8(
        ctypes.byref(fuse), _ptr(e8), int(B), int(T), e8.shape[-1], _ptr(W8),
        int(e_scale_exp), int(w_scale_exp), _ptr(resid), _ptr(out), _ptr(workspace),
        ws_bytes, _stream(stream)))


def pg_forward_fp8(layout, table, fuse, tokens, canon_map, W8, e_scale_exp, w_scale_exp,
                   resid, out, workspace, dev_status=None, stream=None):
    B, T = tokens.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pg_forward_fp8", lib().pg_forward_fp8(
        ctypes.byref(layout), ctypes.byref(table), ctypes.byref(fuse), _ptr(tokens),
        B, T, _ptr(canon_map), canon_map.numel(), _ptr(W8), int(e_scale_exp),
        int(w_scale_exp), _ptr(resid), _ptr(out), _ptr(workspace), ws_bytes,
        _ptr(dev_status), _stream(stream)))


# ----------------------------------------------------------------------------
# Backward pass and table update


def pg_backward_workspace_size(layout, fuse, B, T):
    v = lib().pg_backward_workspace_size(ctypes.byref(layout), ctypes.byref(fuse), int(B),
                                         int(T))
    if v < 0:
        raise PagegramError("pg_backward_workspace_size", v)
    return v


def pg_backward_scalar(layout, fuse, rows, signs, e, dy, W, B, T, dW, de, urows, ugrad,
                       n_unique, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pg_backward_scalar", lib().pg_backward_scalar(
        ctypes.byref(layout), ctypes.byref(fuse), _ptr(rows), _ptr(signs), _ptr(e), _ptr(dy),
        _ptr(W), int(B), int(T), _ptr(dW), _ptr(de), _ptr(urows), _ptr(ugrad),
        _ptr(n_unique), _ptr(workspace), ws_bytes, _stream(stream)))


def pg_row_rms_step(layout, urows, ugrad, n_unique, max_unique, table, vhat, last_step, step,
                    lr, beta2=0.95, weight_decay=0.0, eps=1e-8, stream=None):
    _check("pg_row_rms_step", lib().pg_row_rms_step(
        ctypes.byref(layout), _ptr(urows), _ptr(ugrad), _ptr(n_unique), int(max_unique),
        _ptr(table), _ptr(vhat), _ptr(last_step), int(step), float(lr), float(beta2),
        float(weight_decay), float(eps), _stream(stream)))


def pg_row_rms_flush(layout, table, vhat, last_step, step, lr, beta2=0.95, weight_decay=0.0,
                     stream=None):
    _check("pg_row_rms_flush", lib().pg_row_rms_flush(
        ctypes.byref(layout), _ptr(table), _ptr(vhat), _ptr(last_step), int(step), float(lr),
        float(beta2), float(weight_decay), _stream(stream)))


# ----------------------------------------------------------------------------
# Flash page-cache simulation (host arrays)


def pg_flash_blocks(layout, table_dtype, rows):
    """4 KiB block of each row; rows: host int64 numpy array of any shape."""
    import numpy as np
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty_like(rows)
    _check("pg_flash_blocks", lib().pg_flash_blocks(
        ctypes.byref(layout), int(table_dtype), rows.ctypes.data, rows.size,
        out.ctypes.data))
    return out


def pg_lru_cache_sim(blocks, capacity_blocks):
    """LRU run over blocks [n_tok, per_token] (host int64); returns the counters."""
    import numpy as np
    blocks = np.ascontiguousarray(blocks, dtype=np.int64)
    n_tok = blocks.shape[0]
    per = int(blocks.size // n_tok) if n_tok else 1
    st = PgCacheStats()
    _check("pg_lru_cache_sim", lib().pg_lru_cache_sim(
        blocks.ctypes.data, n_tok, per, int(capacity_blocks), ctypes.byref(st)))
    return dict(tokens=st.tokens, lookups=st.lookups, distinct=st.distinct,
                misses=st.misses)
