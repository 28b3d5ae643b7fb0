"""ctypes binding of libmla (include/mla.h).

Argument marshalling only: every step of MLA runs in the HIP library.  Torch
supplies device memory (``tensor.data_ptr()``) and the HIP stream
(``torch.cuda.current_stream().cuda_stream``).  If the built library is
missing the binding raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int32, c_int64, c_size_t, c_void_p
from typing import Dict, Optional

LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                         "libmla.so")

MLA_FP32, MLA_BF16 = 0, 1
MLA_CACHE_LAYER, MLA_CACHE_FP8_E4M3 = 0, 1
MLA_WEIGHTS_LAYER, MLA_WEIGHTS_FP8_BLOCK = 0, 1
MLA_OP_PREFILL, MLA_OP_DECODE, MLA_OP_COMPRESS = 0, 1, 2
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_WORKSPACE", -5: "MLA_ERR_CACHE", -6: "MLA_ERR_HIP", -7: "MLA_ERR_UNSUPPORTED"}
WEIGHT_NAMES = ("w_dq", "w_uq", "w_qr", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")
# the block scales of the FP8 projections (MLA_WEIGHTS_FP8_BLOCK), by weight
SCALE_NAMES = ("w_dq", "w_dkv", "w_kr", "w_o")


class MlaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({_lib().mla_status_string(code).decode()})")


class mla_config(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("n_heads", c_int32), ("d_nope", c_int32), ("d_rope", c_int32),
                ("d_v", c_int32), ("d_c", c_int32), ("d_cq", c_int32), ("dtype", c_int32),
                ("rope_base", c_double), ("yarn_factor", c_double), ("yarn_beta_slow", c_double),
                ("yarn_beta_fast", c_double), ("yarn_orig_len", c_int32), ("cache_dtype", c_int32),
                ("weight_dtype", c_int32)]


class mla_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in WEIGHT_NAMES] + [("s_" + n[2:], c_void_p) for n in SCALE_NAMES]


class mla_cache(ctypes.Structure):
    _fields_ = [("pool", c_void_p), ("block_size", c_int32), ("n_blocks", c_int32),
                ("block_table", c_void_p), ("max_blocks_per_seq", c_int32), ("max_len", c_int32)]


_LIB = None


def load(path: str) -> ctypes.CDLL:
    """A libmla build at `path` (e.g. lib/libmla_debug.so) with every
    function's argument and result types declared."""
    if not os.path.exists(path):
        raise RuntimeError(f"libmla is not built ({path} missing); run "
                           "`python -m head_latent_attention_18_amd.build`")
    lib = ctypes.CDLL(path)
    P = POINTER
    lib.mla_cache_bytes_per_token.argtypes = [P(mla_config)]
    lib.mla_cache_bytes_per_token.restype = c_size_t
    lib.mla_mha_cache_elements_per_token.argtypes = [P(mla_config)]
    lib.mla_mha_cache_elements_per_token.restype = c_size_t
    lib.mla_workspace_size.argtypes = [P(mla_config), c_int32, c_int32, c_int32, c_int32, P(c_size_t)]
    lib.mla_workspace_size.restype = c_int32
    lib.mla_compress_kv.argtypes = [P(mla_config), P(mla_weights), c_void_p, c_int32, c_void_p, c_void_p,
                                    c_int32, P(mla_cache), c_void_p, c_size_t, c_void_p]
    lib.mla_compress_kv.restype = c_int32
    lib.mla_prefill.argtypes = [P(mla_config), P(mla_weights), c_void_p, c_int32, c_int32, P(mla_cache),
                                c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.mla_prefill.restype = c_int32
    lib.mla_decode.argtypes = [P(mla_config), P(mla_weights), c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                               c_int32, P(mla_cache), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.mla_decode.restype = c_int32
    lib.mla_decode_noalloc.argtypes = [P(mla_config), P(mla_weights), c_void_p, c_int32, c_int32, c_void_p,
                                       c_void_p, c_int32, P(mla_cache), c_void_p, c_void_p, c_void_p]
    lib.mla_decode_noalloc.restype = c_int32
    lib.mla_status_string.argtypes = [c_int32]
    lib.mla_status_string.restype = c_char_p
    lib.mla_version.argtypes = []
    lib.mla_version.restype = c_char_p
    lib.mla_timing_enable.argtypes = [c_int32]
    lib.mla_timing_enable.restype = c_int32
    lib.mla_timing_read.argtypes = [P(c_char_p), P(c_double), P(c_int64), c_int32]
    lib.mla_timing_read.restype = c_int32
    return lib


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = load(LIB_PATH)
    return _LIB


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def _check(fn: str, code: int):
    if code != 0:
        raise MlaError(fn, code)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# Struct builders
# ---------------------------------------------------------------------------

def make_config(dims, dtype: str, cache: str = "layer", weights: str = "layer") -> mla_config:
    return mla_config(dims.d_model, dims.n_heads, dims.d_nope, dims.d_rope, dims.d_v, dims.d_c, dims.d_cq,
                      MLA_BF16 if dtype == "bf16" else MLA_FP32, float(dims.rope_base),
                      float(getattr(dims, "yarn_factor", 1.0)), float(getattr(dims, "yarn_beta_slow", 1.0)),
                      float(getattr(dims, "yarn_beta_fast", 32.0)), int(getattr(dims, "yarn_orig_len", 4096)),
                      MLA_CACHE_FP8_E4M3 if cache == "fp8" else MLA_CACHE_LAYER,
                      MLA_WEIGHTS_FP8_BLOCK if weights == "fp8" else MLA_WEIGHTS_LAYER)


def make_weights(w: Dict[str, object], scales: Optional[Dict[str, object]] = None) -> mla_weights:
    """Weight pointers by name; `scales` (by weight name) gives the block
    scales of the FP8 projections."""
    scales = scales or {}
    return mla_weights(*[_ptr(w.get(n)) for n in WEIGHT_NAMES], *[_ptr(scales.get(n)) for n in SCALE_NAMES])


def make_cache(pool, *, max_len: int = 0, block_size: int = 0, n_blocks: int = 0, block_table=None,
               max_blocks_per_seq: int = 0) -> mla_cache:
    return mla_cache(_ptr(pool), block_size, n_blocks, _ptr(block_table), max_blocks_per_seq, max_len)


# ---------------------------------------------------------------------------
# The ABI calls, same names
# ---------------------------------------------------------------------------

def mla_cache_bytes_per_token(cfg: mla_config) -> int:
    return _lib().mla_cache_bytes_per_token(ctypes.byref(cfg))


def mla_mha_cache_elements_per_token(cfg: mla_config) -> int:
    return _lib().mla_mha_cache_elements_per_token(ctypes.byref(cfg))


def mla_workspace_size(cfg: mla_config, op: int, batch: int, len_or_nq: int, max_cache_len: int = 0) -> int:
    out = c_size_t(0)
    _check("mla_workspace_size",
           _lib().mla_workspace_size(ctypes.byref(cfg), op, batch, len_or_nq, max_cache_len, ctypes.byref(out)))
    return out.value


def mla_compress_kv(cfg, w: mla_weights, h, n: int, seq_idx, pos, batch: int, cache: mla_cache, workspace=None,
                    workspace_bytes: int = 0, stream=None):
    _check("mla_compress_kv", _lib().mla_compress_kv(ctypes.byref(cfg), ctypes.byref(w), _ptr(h), n,
                                                     _ptr(seq_idx), _ptr(pos), batch, ctypes.byref(cache),
                                                     _ptr(workspace), workspace_bytes, _stream(stream)))


def mla_prefill(cfg, w: mla_weights, h, batch: int, length: int, cache: mla_cache, u, o_heads, workspace,
                workspace_bytes: int, stream=None):
    _check("mla_prefill", _lib().mla_prefill(ctypes.byref(cfg), ctypes.byref(w), _ptr(h), batch, length,
                                             ctypes.byref(cache), _ptr(u), _ptr(o_heads), _ptr(workspace),
                                             workspace_bytes, _stream(stream)))


def _host_i32(a):
    """A host int32 array for a *_host argument: (ctypes pointer, keep-alive
    object), or (None, None)."""
    if a is None:
        return None, None
    import numpy as np
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr.ctypes.data_as(c_void_p), arr


def mla_decode(cfg, w: mla_weights, h, batch: int, n_q: int, cache_lens, max_cache_len: int, cache: mla_cache,
               u, o_heads, workspace, workspace_bytes: int, stream=None, cache_lens_host=None):
    lens_host, _keep = _host_i32(cache_lens_host)
    _check("mla_decode", _lib().mla_decode(ctypes.byref(cfg), ctypes.byref(w), _ptr(h), batch, n_q,
                                           _ptr(cache_lens), lens_host, max_cache_len, ctypes.byref(cache),
                                           _ptr(u), _ptr(o_heads), _ptr(workspace), workspace_bytes,
                                           _stream(stream)))


MLA_NOALLOC_WORKSPACE_BYTES = 128 << 20


def mla_decode_noalloc(cfg, w: mla_weights, h, batch: int, n_q: int, cache_lens, max_cache_len: int,
                       cache: mla_cache, u, o_heads, stream=None, cache_lens_host=None):
    lens_host, _keep = _host_i32(cache_lens_host)
    _check("mla_decode_noalloc", _lib().mla_decode_noalloc(ctypes.byref(cfg), ctypes.byref(w), _ptr(h), batch, n_q,
                                                           _ptr(cache_lens), lens_host, max_cache_len,
                                                           ctypes.byref(cache), _ptr(u), _ptr(o_heads),
                                                           _stream(stream)))


def mla_status_string(code: int) -> str:
    return _lib().mla_status_string(code).decode()


def mla_version() -> str:
    return _lib().mla_version().decode()


def mla_timing_enable(on: bool):
    _check("mla_timing_enable", _lib().mla_timing_enable(1 if on else 0))


def mla_timing_read(cap: int = 64) -> Dict[str, tuple]:
    names = (c_char_p * cap)()
    ms = (c_double * cap)()
    cnt = (c_int64 * cap)()
    n = _lib().mla_timing_read(names, ms, cnt, cap)
    if n < 0:
        raise MlaError("mla_timing_read", n)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n, cap))}
