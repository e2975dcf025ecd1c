"""GPU parity at the longest sequence the library accepts, T = SA_MAX_T =
2^22, checked on sampled rows against the fp64 oracle.

Two layers, one head each:

* a causal window of 256 keys at d = 128 ("Sparse and sliding-window
  attention", getnybble.com, section "Sliding window attention"): K and V of
  the sequence then span exactly 1 GiB each, the largest byte offset the
  kernels' 32-bit buffer addressing has to reach;
* a bidirectional band with strided landmark keys and 64 global tokens at
  d = 64 ("Sparse Attention", ai360xpert.com, "How It Actually Works"): the
  global rows read all 2^22 keys, so their query block is split into many
  work items that the merge kernel combines, and every other row reads the
  strided and global columns as gathered keys.

Rows checked: the first and last 300, rows on both sides of the middle and
of every power-of-two row up to T, the global rows (eight of them), and 300
seeded random rows.  Tolerance as for every bf16 forward: elementwise
max |O - O*| <= 2e-2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_masked_spec_amd import inputs

pytestmark = pytest.mark.gpu

BF16_ATOL = 2e-2
T_MAX = 1 << 22


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def sample_rows(T, extra, seed):
    rows = set(range(300)) | set(range(T - 300, T)) | set(extra)
    p = 1
    while p < T:
        rows |= {p - 2, p - 1, p, p + 1}
        p *= 2
    rows |= set(range(T // 2 - 70, T // 2 + 70))
    rows |= {int(x) for x in np.random.default_rng(seed).integers(0, T, size=300)}
    return sorted(r for r in rows if 0 <= r < T)


@pytest.mark.parametrize("spec,d,seed,global_rows", [
    ("causal;window=256", 128, 11, []),
    ("bidir;radius=64;stride=65536;global=0:64", 64, 12, [0, 1, 17, 31, 32, 50, 62, 63]),
])
def test_forward_at_max_length(gpu, spec, d, seed, global_rows):
    T = T_MAX
    assert gpu.sparse_attn_count(spec, T) > 0
    with pytest.raises(RuntimeError):  # the library's limit: one row more is a shape error
        gpu.sparse_attn_count(spec, T + 1)
    announce(f"fwd max length bf16 B=1 H=1 T={T} d={d} seed={seed} spec={spec}")
    q, k, v = inputs.qkv(1, 1, T, d, "bf16", seed)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    od = torch.empty_like(qd)
    gpu.sparse_attn_fwd(qd, kd, vd, od, 1, 1, T, d, spec)
    torch.cuda.synchronize()
    o = od.cpu()
    del qd, kd, vd, od
    rows = sample_rows(T, global_rows, seed)
    ref, _, nset = oracle.forward_rows(spec, q, k, v, rows=[(0, 0, i) for i in rows])
    got = o[0, 0, rows].double().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    announce(f"max length {spec} d={d}: {len(rows)} rows (up to {int(nset.max())} keys each), "
             f"max abs err {err:.3e}")
    assert err <= BF16_ATOL, f"max abs err {err:.3e} > {BF16_ATOL}"
