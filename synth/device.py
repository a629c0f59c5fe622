"""Device-side fills with the synth module's counter-based generator.

Large inputs (multi-GB tables, weights, residual streams) are generated on
the GPU by synth/libhhg_synth.so (built from synth/fill.hip); the host
recomputes any element from its flat index with the functions in
synth/__init__.py. Input generation only.
"""
import ctypes
import os

import numpy as np

from . import configs, normal_scale, stream_base

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhhg_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_float, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_void_p]
        L.synth_fill_words.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_void_p]
        L.synth_fill_nf4_scales.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_uint64, ctypes.c_void_p]
        for f in (L.synth_fill_normal, L.synth_fill_words, L.synth_fill_nf4_scales):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fill_normal(t, seed, stream, sigma, offset=0):
    """Fill a float32 / bfloat16 CUDA tensor with N(0, sigma)-like values of
    the given stream at flat indices offset .. offset + numel - 1."""
    import torch
    bf16 = {torch.float32: 0, torch.bfloat16: 1}[t.dtype]
    scale = float(normal_scale(sigma))
    assert np.float32(scale) == normal_scale(sigma)
    rc = lib().synth_fill_normal(t.data_ptr(), t.numel(), stream_base(seed, stream),
                                 scale, bf16, int(offset), _stream())
    if rc:
        raise RuntimeError("synth_fill_normal failed")
    return t


def fill_nf4_table(codes, scales, seed):
    """codes uint8 [R, r/2] and scales fp16 [R] of an NF4 table."""
    assert codes.numel() % 8 == 0
    rc = lib().synth_fill_words(codes.data_ptr(), codes.numel() // 8,
                                stream_base(seed, configs.STREAM_TABLE), _stream())
    rc |= lib().synth_fill_nf4_scales(scales.data_ptr(), scales.numel(),
                                      stream_base(seed, configs.STREAM_NF4_SCALE),
                                      _stream())
    if rc:
        raise RuntimeError("synth NF4 fill failed")
    return codes, scales
