"""Oracle for masked sparse attention (forward) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package never imports the product: the two share no code, no header and
no constant.  The only thing both sides see is the seeded input generator
(``block_sparse_masked_spec_amd.inputs``), which holds none of the method's
arithmetic.

What it computes (fp64, no rounding of the result):

* ``allowed(i, j)``, ``row_set``, ``count`` and ``tile_map`` -- the mask rule,
  pair by pair, in ``sa_oracle.c``.
* ``forward_rows`` -- for each requested (head, query) row: S_i by scanning
  every key, scores q.k/sqrt(d), max, exp-sum and the renormalised weighted
  sum of values ("Sparse attention", glossary.selfmadequant.com, section
  "Choose the available reads").
* ``backward`` -- dQ, dK, dV for an upstream gradient dO: the chain rule
  through the renormalised softmax, row by row (pinned by finite differences
  of ``forward_rows``, by autograd through a dense masked softmax, and by the
  identities sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i).
* ``dense_forward`` -- a second, independent formulation for tiny inputs: a
  materialised boolean mask, full score matrix, -inf fill, softmax, matmul
  (the naive recipe of "Sparse and sliding-window attention", getnybble.com,
  section "Implementation").

Mask-spec text is parsed here by ``parse_spec`` (written independently of the
product's parser).  Grammar: ``causal`` or ``bidir``, then ``;``-separated
clauses ``window=W`` (causal; 0 = unlimited), ``radius=R`` (bidir),
``dilation=G`` (G >= 1: the local keys sit G apart, "Attention variants",
section 6, dilated-mask exercise), ``stride=S``, ``phase=P`` (0 <= P < S),
``global=a,b:c,...`` (single indices or half-open ranges).  Block mode
(BigBird, "Sparse and sliding-window attention", section "Block-sparse
attention: BigBird"): ``blocks;block=S`` then ``radius=`` (in blocks,
default 0), ``random=R`` (random key blocks per query block, <= 4096),
``seed=X``, ``stride``/``phase``/``global`` as above.

Pins (each in ``tests/test_oracle_pins.py``): the pages' printed cell counts
and per-row key sets (``tests/golden/page_facts.json``), the closed form
E = n*w - w*(w-1)/2, torch's CPU ``scaled_dot_product_attention`` in fp64 for
cases that reduce to a library routine (causal, full, a tril/triu band), the
w = 1 identity, the q = 0 mean over the pages' printed sets, shift and affine
invariants, and a negative test (no renormalisation).  No function here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


# --------------------------------------------------------------------------
# spec parsing (independent of the product's parser)
# --------------------------------------------------------------------------
class OracleSpecError(ValueError):
    pass


@dataclass
class OracleMask:
    causal: bool
    window: int = 0            # causal: 0 = unlimited
    radius: int | None = None  # bidir: None = unlimited
    stride: int = 0
    phase: int = 0
    dilation: int = 1          # local keys sit `dilation` apart
    globals_: list = field(default_factory=list)  # list of (lo, hi) half-open
    block: int = 0             # > 0: block mode (radius counts blocks)
    random: int = 0            # block mode: random key blocks per query block
    seed: int = 0              # block mode: random stream seed

    def global_set(self, T):
        s = set()
        for lo, hi in self.globals_:
            s.update(range(lo, min(hi, T)))
        return s


_INT = re.compile(r"^[0-9]+$")


def parse_spec(spec: str) -> OracleMask:
    text = "".join(spec.split())
    if not text:
        raise OracleSpecError("empty spec")
    parts = text.split(";")
    head = parts[0]
    if head not in ("causal", "bidir", "blocks"):
        raise OracleSpecError(f"mode must be causal, bidir or blocks, got {head!r}")
    m = OracleMask(causal=(head == "causal"))
    blocks = head == "blocks"
    seen = set()
    for clause in parts[1:]:
        if "=" not in clause:
            raise OracleSpecError(f"bad clause {clause!r}")
        key, val = clause.split("=", 1)
        if key in seen:
            raise OracleSpecError(f"duplicate key {key!r}")
        seen.add(key)
        if key == "global":
            ranges = []
            for item in val.split(","):
                if ":" in item:
                    a, b = item.split(":", 1)
                    if not (_INT.match(a) and _INT.match(b)) or int(a) >= int(b) \
                            or int(b) >= 2 ** 31:
                        raise OracleSpecError(f"bad global range {item!r}")
                    ranges.append((int(a), int(b)))
                else:
                    if not _INT.match(item) or int(item) >= 2 ** 31:
                        raise OracleSpecError(f"bad global index {item!r}")
                    ranges.append((int(item), int(item) + 1))
            m.globals_ = ranges
            continue
        if not _INT.match(val) or int(val) >= 2 ** 31:
            raise OracleSpecError(f"bad integer {val!r}")
        v = int(val)
        if blocks and key in ("window", "dilation"):
            raise OracleSpecError(f"{key} is not a block-mode clause")
        if not blocks and key in ("block", "random", "seed"):
            raise OracleSpecError(f"{key} needs block mode")
        if key == "window":
            if not m.causal:
                raise OracleSpecError("window needs causal")
            m.window = v
        elif key == "radius":
            if m.causal:
                raise OracleSpecError("radius needs bidir")
            m.radius = v
        elif key == "block":
            if v < 1:
                raise OracleSpecError("block must be >= 1")
            m.block = v
        elif key == "random":
            if v > 4096:
                raise OracleSpecError("random must be <= 4096")
            m.random = v
        elif key == "seed":
            m.seed = v
        elif key == "stride":
            m.stride = v
        elif key == "phase":
            m.phase = v
        elif key == "dilation":
            if v < 1:
                raise OracleSpecError("dilation must be >= 1")
            m.dilation = v
        else:
            raise OracleSpecError(f"unknown key {key!r}")
    if blocks:
        if m.block == 0:
            raise OracleSpecError("block mode needs block=")
        if m.radius is None:
            m.radius = 0
    if "phase" in seen and m.stride == 0:
        raise OracleSpecError("phase needs stride > 0")
    if m.stride and not (0 <= m.phase < m.stride):
        raise OracleSpecError("phase must be below stride")
    return m


# --------------------------------------------------------------------------
# the C core
# --------------------------------------------------------------------------
class _CMask(ctypes.Structure):
    _fields_ = [
        ("causal", ctypes.c_int32),
        ("has_radius", ctypes.c_int32),
        ("window", ctypes.c_int64),
        ("radius", ctypes.c_int64),
        ("stride", ctypes.c_int64),
        ("phase", ctypes.c_int64),
        ("n_global", ctypes.c_int32),
        ("dilation", ctypes.c_int32),
        ("global_lo", ctypes.POINTER(ctypes.c_int64)),
        ("global_hi", ctypes.POINTER(ctypes.c_int64)),
        ("block", ctypes.c_int64),
        ("n_random", ctypes.c_int64),
        ("seed", ctypes.c_uint64),
    ]


def build(force: bool = True) -> str:
    """Compile sa_oracle.c into oracle/liboracle.so with gcc (fp64, OpenMP)."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
             "-std=c11", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        lib.oracle_allowed.argtypes = [P(_CMask), ctypes.c_int64, ctypes.c_int64]
        lib.oracle_allowed.restype = ctypes.c_int
        lib.oracle_allowed_T.argtypes = [P(_CMask), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        lib.oracle_allowed_T.restype = ctypes.c_int
        lib.oracle_splitmix64.argtypes = [P(ctypes.c_uint64)]
        lib.oracle_splitmix64.restype = ctypes.c_uint64
        lib.oracle_random_blocks.argtypes = [P(_CMask), ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_random_blocks.restype = ctypes.c_int64
        lib.oracle_row_set.argtypes = [P(_CMask), ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_row_set.restype = ctypes.c_int64
        lib.oracle_count.argtypes = [P(_CMask), ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_count.restype = ctypes.c_int64
        lib.oracle_tile_map.argtypes = [P(_CMask), ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_tile_map.restype = None
        lib.oracle_forward_rows.argtypes = [
            P(_CMask), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_forward_rows.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [
            P(_CMask), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _cmask(m: OracleMask):
    """Return a C struct for ``m`` plus the arrays it points into (keep alive)."""
    lo = np.array([a for a, _ in m.globals_] or [0], dtype=np.int64)
    hi = np.array([b for _, b in m.globals_] or [0], dtype=np.int64)
    c = _CMask(
        causal=1 if m.causal else 0,
        has_radius=0 if m.radius is None else 1,
        window=m.window,
        radius=0 if m.radius is None else m.radius,
        stride=m.stride,
        phase=m.phase,
        n_global=len(m.globals_),
        dilation=m.dilation,
        global_lo=lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        global_hi=hi.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        block=m.block,
        n_random=m.random,
        seed=m.seed,
    )
    return c, (lo, hi)


def _as_mask(spec_or_mask):
    return parse_spec(spec_or_mask) if isinstance(spec_or_mask, str) else spec_or_mask


def allowed(spec, i: int, j: int, T: int | None = None) -> bool:
    """The rule for one pair; block mode needs T (it fixes the key blocks)."""
    m = _as_mask(spec)
    c, keep = _cmask(m)
    if m.block:
        if T is None:
            raise ValueError("block mode needs T")
        return bool(_load().oracle_allowed_T(ctypes.byref(c), T, i, j))
    return bool(_load().oracle_allowed(ctypes.byref(c), i, j))


def splitmix64(state: int, n: int) -> list:
    """The first n outputs of SplitMix64 started from `state`."""
    st = ctypes.c_uint64(state)
    return [int(_load().oracle_splitmix64(ctypes.byref(st))) for _ in range(n)]


def random_blocks(spec, T: int, qb: int) -> list:
    """Rand(qb): the random key blocks of query block qb, in draw order."""
    m = _as_mask(spec)
    c, keep = _cmask(m)
    out = np.zeros(max(m.random, 1) + (-(-T // max(m.block, 1))), dtype=np.int64)
    n = _load().oracle_random_blocks(ctypes.byref(c), T, qb, out.ctypes.data)
    return out[:n].tolist()


def row_set(spec, T: int, i: int) -> list:
    m = _as_mask(spec)
    c, keep = _cmask(m)
    out = np.zeros(max(T, 1), dtype=np.int64)
    n = _load().oracle_row_set(ctypes.byref(c), T, i, out.ctypes.data)
    return out[:n].tolist()


def count(spec, T: int, per_row: bool = False):
    m = _as_mask(spec)
    c, keep = _cmask(m)
    rows = np.zeros(max(T, 1), dtype=np.int64) if per_row else None
    total = _load().oracle_count(ctypes.byref(c), T, rows.ctypes.data if per_row else None)
    return (int(total), rows[:T]) if per_row else int(total)


def tile_map(spec, T: int, bq: int, bk: int) -> np.ndarray:
    m = _as_mask(spec)
    c, keep = _cmask(m)
    nqb, nkb = -(-T // bq), -(-T // bk)
    out = np.zeros(nqb * nkb, dtype=np.uint8)
    _load().oracle_tile_map(ctypes.byref(c), T, bq, bk, out.ctypes.data)
    return out.reshape(nqb, nkb)


def forward_rows(spec, Q, K, V, rows=None):
    """Forward pass in fp64 for selected rows.

    Q, K, V: arrays or CPU tensors of shape [B, H, T, d] (any float dtype; the
    stored values are widened exactly).  ``rows``: iterable of (b, h, i) or
    None for every row.  Returns (O [n_rows, d] fp64, lse [n_rows], |S_i|
    [n_rows]); with rows=None, O is shaped [B, H, T, d].
    """
    m = _as_mask(spec)
    q = _to_f32(Q)
    k = _to_f32(K)
    v = _to_f32(V)
    B, H, T, d = q.shape
    if rows is None:
        flat = np.arange(B * H * T, dtype=np.int64)
    else:
        flat = np.array([(b * H + h) * T + i for (b, h, i) in rows], dtype=np.int64)
    n = flat.size
    O = np.zeros((max(n, 1), d), dtype=np.float64)
    lse = np.zeros(max(n, 1), dtype=np.float64)
    nset = np.zeros(max(n, 1), dtype=np.int64)
    c, keep = _cmask(m)
    rc = _load().oracle_forward_rows(
        ctypes.byref(c), q.ctypes.data, k.ctypes.data, v.ctypes.data,
        B * H, T, d, flat.ctypes.data, n, O.ctypes.data, lse.ctypes.data,
        nset.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_forward_rows failed (row out of range or no memory)")
    O, lse, nset = O[:n], lse[:n], nset[:n]
    if rows is None:
        return O.reshape(B, H, T, d), lse.reshape(B, H, T), nset.reshape(B, H, T)
    return O, lse, nset


def backward(spec, Q, K, V, dO):
    """Gradients (dQ, dK, dV) of the forward for upstream gradient dO, fp64,
    each [B, H, T, d].  The chain rule through the softmax over each S_i,
    written out in sa_oracle.c."""
    m = _as_mask(spec)
    q, k, v, g = (_to_f32(x) for x in (Q, K, V, dO))
    B, H, T, d = q.shape
    dq = np.zeros((B, H, T, d), dtype=np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    c, keep = _cmask(m)
    rc = _load().oracle_backward(ctypes.byref(c), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                 g.ctypes.data, B * H, T, d, dq.ctypes.data, dk.ctypes.data,
                                 dv.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_backward failed (no memory)")
    return dq, dk, dv


def threads() -> int:
    return int(_load().oracle_threads())


def _to_f32(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.ndim != 4:
        raise ValueError("expected [B, H, T, d]")
    return x


# --------------------------------------------------------------------------
# dense formulation for tiny inputs
# --------------------------------------------------------------------------
def dense_mask(spec, T: int) -> np.ndarray:
    """Boolean [T, T] matrix, True = may attend, built as whole-array rules:
    the local rule, OR the strided columns, OR whole global rows and columns,
    then AND the causal triangle ("Attention variants", section 4, "Build it
    from scratch": masks are unions of simple rules over index grids)."""
    m = _as_mask(spec)
    i, j = np.indices((T, T))
    if m.block:
        qb, kb = i // m.block, j // m.block
        mask = np.abs(qb - kb) <= m.radius
        nqb = -(-T // m.block)
        rnd = np.zeros((nqb, nqb), dtype=bool)
        for b in range(nqb):
            rnd[b, random_blocks(m, T, b)] = True
        mask |= rnd[qb, kb]
        if m.stride:
            mask |= (j % m.stride) == m.phase
        g = sorted(m.global_set(T))
        if g:
            mask[:, g] = True
            mask[g, :] = True
        return mask
    g_ = m.dilation
    if m.causal:
        local = (i - j < m.window * g_) if m.window else np.ones((T, T), bool)
    else:
        local = (np.abs(i - j) <= m.radius * g_) if m.radius is not None else np.ones((T, T), bool)
    local &= (np.abs(i - j) % g_) == 0
    mask = local.copy()
    if m.stride:
        mask |= (j % m.stride) == m.phase
    g = sorted(m.global_set(T))
    if g:
        mask[:, g] = True
        mask[g, :] = True
    if m.causal:
        mask &= j <= i
    return mask


def dense_forward(spec, Q, K, V):
    """Materialise all scores, fill excluded ones with -inf, softmax, matmul
    -- fp64, [B, H, T, d] in and out.  For T up to a few hundred."""
    q = _to_f32(Q).astype(np.float64)
    k = _to_f32(K).astype(np.float64)
    v = _to_f32(V).astype(np.float64)
    T, d = q.shape[2], q.shape[3]
    mask = dense_mask(spec, T)
    scores = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(d)
    scores = np.where(mask, scores, -np.inf)
    mx = scores.max(axis=-1, keepdims=True)
    w = np.exp(scores - mx)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.matmul(w, v)
