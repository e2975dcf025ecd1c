"""ctypes binding of libsparse_attn.so (see include/sparse_attn.h).

Argument marshalling only: every step of the computation runs in the
library.  Functions keep the C names.  Tensor arguments may be torch
tensors (their ``data_ptr()`` is passed) or raw integer device addresses.
A non-OK status raises ``SparseAttnError`` carrying the status code.

The library is loaded after ``torch`` so that it binds to the HIP runtime
torch already loaded (same SONAME), sharing devices and streams with it.
If the library is missing this module raises on first use -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime first)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")

SA_OK = 0
SA_ERR_SPEC = -1
SA_ERR_RANGE = -2
SA_ERR_SHAPE = -3
SA_ERR_UNSUPPORTED = -4
SA_ERR_NULL = -5
SA_ERR_ALIAS = -6
SA_ERR_HIP = -7
SA_ERR_ALIGN = -8
SA_ERR_NOMEM = -9
SA_ERR_SCRATCH = -10
SA_DECODE_SCRATCH_BYTES = 4 << 20

SA_TILE_EMPTY, SA_TILE_FULL, SA_TILE_PARTIAL = 0, 1, 2
SA_DTYPE_BF16, SA_DTYPE_F32 = 0, 1
SA_MAX_GLOBAL_RANGES = 64

EXPORTED = [
    "sparse_attn_fwd", "sparse_attn_fwd_f32", "sparse_attn_parse", "sparse_attn_count",
    "sparse_attn_tile_map", "sparse_attn_tile_shape", "sparse_attn_plan_info", "sparse_attn_plan_info_bh",
    "sparse_attn_strerror", "sparse_attn_release_cache", "sparse_attn_decode",
    "sparse_attn_decode_cache_rows", "sparse_attn_fwd_lse", "sparse_attn_fwd_lse_f32",
    "sparse_attn_bwd", "sparse_attn_bwd_f32", "sparse_attn_decode_noalloc",
]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class sa_mask(ctypes.Structure):
    _fields_ = [
        ("causal", ctypes.c_int32), ("has_radius", ctypes.c_int32),
        ("window", ctypes.c_int64), ("radius", ctypes.c_int64),
        ("stride", ctypes.c_int64), ("phase", ctypes.c_int64),
        ("n_global", ctypes.c_int32), ("dilation", ctypes.c_int32),
        ("global_lo", ctypes.c_int64 * SA_MAX_GLOBAL_RANGES),
        ("global_hi", ctypes.c_int64 * SA_MAX_GLOBAL_RANGES),
        ("block", ctypes.c_int64), ("n_random", ctypes.c_int32), ("seed", ctypes.c_uint32),
    ]


class sa_plan_info(ctypes.Structure):
    _fields_ = [
        ("bq", ctypes.c_int32), ("bk", ctypes.c_int32),
        ("n_qb", ctypes.c_int32), ("n_kb", ctypes.c_int32),
        ("subsequences", ctypes.c_int32), ("split_parts", ctypes.c_int32),
        ("inplace_tiles", ctypes.c_int64), ("masked_tiles", ctypes.c_int64),
        ("gathered_tiles", ctypes.c_int64), ("gathered_keys", ctypes.c_int64),
        ("executed_cells", ctypes.c_int64), ("allowed_cells", ctypes.c_int64),
    ]


_lib = None


def load():
    """Load (once) and return the library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with `python -m block_sparse_masked_spec_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, cs = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_char_p
    fwd_args = [vp, vp, vp, vp, i32, i32, i32, i32, cs, vp]
    lib.sparse_attn_fwd.argtypes = fwd_args
    lib.sparse_attn_fwd.restype = i32
    lib.sparse_attn_fwd_f32.argtypes = fwd_args
    lib.sparse_attn_fwd_f32.restype = i32
    lib.sparse_attn_parse.argtypes = [cs, ctypes.POINTER(sa_mask)]
    lib.sparse_attn_parse.restype = i32
    lib.sparse_attn_count.argtypes = [cs, i32, ctypes.POINTER(i64), vp]
    lib.sparse_attn_count.restype = i32
    lib.sparse_attn_tile_map.argtypes = [cs, i32, i32, i32, vp]
    lib.sparse_attn_tile_map.restype = i32
    lib.sparse_attn_tile_shape.argtypes = [cs, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.sparse_attn_tile_shape.restype = i32
    lib.sparse_attn_plan_info.argtypes = [cs, i32, i32, i32, ctypes.POINTER(sa_plan_info)]
    lib.sparse_attn_plan_info.restype = i32
    lib.sparse_attn_plan_info_bh.argtypes = [cs, i32, i32, i32, i32, i32, ctypes.POINTER(sa_plan_info)]
    lib.sparse_attn_plan_info_bh.restype = i32
    lib.sparse_attn_strerror.argtypes = [i32]
    lib.sparse_attn_strerror.restype = cs
    lse_args = [vp, vp, vp, vp, vp, i32, i32, i32, i32, cs, vp]
    lib.sparse_attn_fwd_lse.argtypes = lse_args
    lib.sparse_attn_fwd_lse.restype = i32
    lib.sparse_attn_fwd_lse_f32.argtypes = lse_args
    lib.sparse_attn_fwd_lse_f32.restype = i32
    bwd_args = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, cs, vp]
    lib.sparse_attn_bwd.argtypes = bwd_args
    lib.sparse_attn_bwd.restype = i32
    lib.sparse_attn_bwd_f32.argtypes = bwd_args
    lib.sparse_attn_bwd_f32.restype = i32
    lib.sparse_attn_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, cs, vp]
    lib.sparse_attn_decode.restype = i32
    lib.sparse_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, cs, vp]
    lib.sparse_attn_decode_noalloc.restype = i32
    lib.sparse_attn_decode_cache_rows.argtypes = [cs, i32, ctypes.POINTER(i64)]
    lib.sparse_attn_decode_cache_rows.restype = i32
    lib.sparse_attn_release_cache.argtypes = []
    lib.sparse_attn_release_cache.restype = None
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().sparse_attn_strerror(int(status)).decode()


def _check(status: int, where: str) -> int:
    if status != SA_OK:
        raise SparseAttnError(status, where)
    return status


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream_handle(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _spec(s) -> bytes:
    return s.encode() if isinstance(s, str) else s


def sparse_attn_fwd(Q, K, V, O, B, H, T, d, mask_spec, stream=None):
    """bf16 forward; stream defaults to torch's current stream."""
    return _check(load().sparse_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), B, H, T, d,
                                         _spec(mask_spec), _stream_handle(stream)),
                  "sparse_attn_fwd")


def sparse_attn_fwd_f32(Q, K, V, O, B, H, T, d, mask_spec, stream=None):
    """fp32 forward; stream defaults to torch's current stream."""
    return _check(load().sparse_attn_fwd_f32(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), B, H, T, d,
                                             _spec(mask_spec), _stream_handle(stream)),
                  "sparse_attn_fwd_f32")


def sparse_attn_parse(mask_spec) -> sa_mask:
    m = sa_mask()
    _check(load().sparse_attn_parse(_spec(mask_spec), ctypes.byref(m)), "sparse_attn_parse")
    return m


def sparse_attn_count(mask_spec, T, row_counts=False):
    """Returns E, or (E, int32 numpy row counts) when row_counts is True."""
    import numpy as np
    total = ctypes.c_int64(0)
    rows = np.zeros(max(T, 1), dtype=np.int32) if row_counts else None
    _check(load().sparse_attn_count(_spec(mask_spec), T, ctypes.byref(total),
                                    rows.ctypes.data if row_counts else None),
           "sparse_attn_count")
    return (total.value, rows[:T]) if row_counts else total.value


def sparse_attn_tile_map(mask_spec, T, bq, bk):
    """Returns a uint8 numpy array [ceil(T/bq), ceil(T/bk)] of SA_TILE_*."""
    import numpy as np
    nqb, nkb = -(-T // bq) if bq > 0 else 0, -(-T // bk) if bk > 0 else 0
    out = np.zeros(max(nqb * nkb, 1), dtype=np.uint8)
    _check(load().sparse_attn_tile_map(_spec(mask_spec), T, bq, bk, out.ctypes.data),
           "sparse_attn_tile_map")
    return out[:nqb * nkb].reshape(nqb, nkb)


def sparse_attn_tile_shape(mask_spec, d, dtype=SA_DTYPE_BF16):
    """(bq, bk) of the forward for mask_spec (None: token-level specs)."""
    bq, bk = ctypes.c_int(0), ctypes.c_int(0)
    spec = None if mask_spec is None else _spec(mask_spec)
    _check(load().sparse_attn_tile_shape(spec, d, dtype, ctypes.byref(bq), ctypes.byref(bk)),
           "sparse_attn_tile_shape")
    return bq.value, bk.value


def sparse_attn_plan_info(mask_spec, T, d, dtype=SA_DTYPE_BF16) -> dict:
    info = sa_plan_info()
    _check(load().sparse_attn_plan_info(_spec(mask_spec), T, d, dtype, ctypes.byref(info)),
           "sparse_attn_plan_info")
    return {name: getattr(info, name) for name, _ in sa_plan_info._fields_}


def sparse_attn_plan_info_bh(mask_spec, B, H, T, d, dtype=SA_DTYPE_BF16) -> dict:
    info = sa_plan_info()
    _check(load().sparse_attn_plan_info_bh(_spec(mask_spec), B, H, T, d, dtype, ctypes.byref(info)),
           "sparse_attn_plan_info_bh")
    return {name: getattr(info, name) for name, _ in sa_plan_info._fields_}


def sparse_attn_fwd_lse(Q, K, V, O, LSE, B, H, T, d, mask_spec, stream=None):
    """bf16 forward that also writes the fp32 log-sum-exp [B, H, T]."""
    return _check(load().sparse_attn_fwd_lse(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B, H,
                                             T, d, _spec(mask_spec), _stream_handle(stream)),
                  "sparse_attn_fwd_lse")


def sparse_attn_fwd_lse_f32(Q, K, V, O, LSE, B, H, T, d, mask_spec, stream=None):
    return _check(load().sparse_attn_fwd_lse_f32(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), B,
                                                 H, T, d, _spec(mask_spec), _stream_handle(stream)),
                  "sparse_attn_fwd_lse_f32")


def sparse_attn_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, T, d, mask_spec, stream=None):
    """bf16 backward: writes dQ, dK, dV."""
    return _check(load().sparse_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE),
                                         _ptr(dQ), _ptr(dK), _ptr(dV), B, H, T, d, _spec(mask_spec),
                                         _stream_handle(stream)),
                  "sparse_attn_bwd")


def sparse_attn_bwd_f32(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, T, d, mask_spec, stream=None):
    return _check(load().sparse_attn_bwd_f32(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                             _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV), B, H, T, d,
                                             _spec(mask_spec), _stream_handle(stream)),
                  "sparse_attn_bwd_f32")


def sparse_attn_decode(Q, K_cache, V_cache, O, pos, B, H, Hkv, n_new, C, d, mask_spec,
                       stream=None):
    """bf16 windowed decode against ring-buffer caches; pos is a device
    int32 tensor [B]; stream defaults to torch's current stream."""
    return _check(load().sparse_attn_decode(_ptr(Q), _ptr(K_cache), _ptr(V_cache), _ptr(O),
                                            _ptr(pos), B, H, Hkv, n_new, C, d, _spec(mask_spec),
                                            _stream_handle(stream)),
                  "sparse_attn_decode")


def sparse_attn_decode_noalloc(Q, K_cache, V_cache, O, pos, B, H, Hkv, n_new, C, d, mask_spec,
                               stream=None):
    """sparse_attn_decode with its partials in the library's static scratch
    (allocates nothing); stream defaults to torch's current stream."""
    return _check(load().sparse_attn_decode_noalloc(_ptr(Q), _ptr(K_cache), _ptr(V_cache), _ptr(O),
                                                    _ptr(pos), B, H, Hkv, n_new, C, d,
                                                    _spec(mask_spec), _stream_handle(stream)),
                  "sparse_attn_decode_noalloc")


def sparse_attn_decode_cache_rows(mask_spec, n_new=1) -> int:
    rows = ctypes.c_int64(0)
    _check(load().sparse_attn_decode_cache_rows(_spec(mask_spec), n_new, ctypes.byref(rows)),
           "sparse_attn_decode_cache_rows")
    return rows.value


def sparse_attn_strerror(status):
    return strerror(status)


def sparse_attn_release_cache():
    load().sparse_attn_release_cache()
