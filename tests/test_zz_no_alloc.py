"""The allocation-free decode entry point (sparse_attn_decode_noalloc)
against the allocating one (sparse_attn_decode): same kernels and key
splits, so the outputs must be bitwise equal.  Two calls in a row on the
same stream, the second with a smaller input, so the second reuses the
static scratch the first left behind; a third call past the scratch limit
is refused before any device work."""
import sys

import numpy as np
import pytest
import torch

from block_sparse_masked_spec_amd import inputs

pytestmark = pytest.mark.gpu


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def decode_pair(gpu, spec, B, H, Hkv, n_new, C, d, seed):
    """Run both entry points on one set of ring caches; return the outputs."""
    rng = np.random.default_rng(seed)
    rows = gpu.sparse_attn_decode_cache_rows(spec, n_new)
    assert rows <= C
    pos = [int(x) for x in rng.integers(C, 4 * C, size=B)]
    _, kc, vc = inputs.qkv(B, Hkv, C, d, "bf16", seed)
    q = inputs.qkv(B, H, n_new, d, "bf16", seed + 1)[0]
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    o_ref, o_na = torch.empty_like(qd), torch.empty_like(qd)
    announce(f"decode_noalloc B={B} H={H} Hkv={Hkv} n_new={n_new} C={C} d={d} spec={spec}")
    gpu.sparse_attn_decode(qd, kd, vd, o_ref, posd, B, H, Hkv, n_new, C, d, spec)
    gpu.sparse_attn_decode_noalloc(qd, kd, vd, o_na, posd, B, H, Hkv, n_new, C, d, spec)
    return o_ref, o_na


def test_noalloc_decode_matches_decode_on_two_calls(gpu):
    # Call 1: the window-4096 serving shape with 16 sequences (32 query heads
    # over 8 KV heads): 128 key groups get 4 key splits, 1.06 MB of partials
    # in the static scratch.
    r1, n1 = decode_pair(gpu, "causal;window=4096", 16, 32, 8, 1, 4096, 128, seed=3)
    # Call 2, smaller, right behind it on the same stream: 6 key splits over
    # a 1500-key window with 3 new tokens, d=64.
    r2, n2 = decode_pair(gpu, "causal;window=1500", 4, 8, 2, 3, 2000, 64, seed=4)
    torch.cuda.synchronize()
    for r, n, what in [(r1, n1, "call 1"), (r2, n2, "call 2")]:
        assert torch.isfinite(n.float()).all(), what
        assert torch.equal(r, n), f"{what}: max diff {(r.float() - n.float()).abs().max().item()}"


def test_noalloc_decode_refuses_past_the_scratch_limit(gpu):
    """B=511, H=8, Hkv=1, d=128, window 4096: 511 key groups of 8 queries
    get 2 key splits, 4.25 MB of partials, above the 4 MiB scratch:
    SA_ERR_SCRATCH, with the output untouched."""
    B, H, Hkv, C, d = 511, 8, 1, 4096, 128
    need = B * H * 1 * 2 * (d + 2) * 4
    assert need > gpu.SA_DECODE_SCRATCH_BYTES
    q = torch.zeros(B, H, 1, d, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    posd = torch.full((B,), C, dtype=torch.int32, device="cuda")
    # The caches are never read (the call is refused first): stand-in
    # addresses far from O, so that no alias check fires instead.
    kc, vc = o.data_ptr() + (1 << 40), o.data_ptr() + (2 << 40)
    with pytest.raises(gpu.SparseAttnError) as e:
        gpu.sparse_attn_decode_noalloc(q, kc, vc, o, posd, B, H, Hkv, 1, C, d, "causal;window=4096")
    assert e.value.status == gpu.SA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (o == 3.0).all()
