"""GPU parity of the forward's log-sum-exp output and of the backward pass
(dQ, dK, dV) against the fp64 oracle.

Tolerances:
* LSE (fp32 output): |lse - lse*| <= 1e-4 for fp32 inputs (scores and sums
  in fp32); <= 2^-8 for bf16, where the fast forward sums the weights after
  rounding them to bf16 (each within 2^-9 relative, so log l moves by at most
  about 2^-9) -- the same weights that multiply V and normalise O.
* fp32 gradients: max |g - g*| <= 1e-4 * max(1, max |g*|) per tensor (the
  floor covers gradients that vanish exactly, like T = 1, where the terms
  are O(1) with N(0,1) inputs), and per row <= 1e-3 of that row's max.  The weights are rebuilt from the fp32 LSE
  (relative error a few fp32 ulps times the score magnitude, about 1e-6) and
  the products accumulate in fp32; a row of dQ or dK is a sum whose
  coefficients ds_ij sum to zero, so a row with a small gradient keeps the
  absolute error of its larger terms and its own relative error grows.
* bf16 gradients: max |g - g*| <= 3e-2 * max(1, max |g*|) per tensor.  The
  MFMA operands P and dS are rounded to bf16 (relative 2^-9 each), the
  outputs too, and a key's gradient sums up to T such terms.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from block_sparse_masked_spec_amd import inputs
from spec_fuzz import random_spec

pytestmark = pytest.mark.gpu

SPECS = [
    "causal",
    "causal;window=7",
    "causal;window=100;stride=32;phase=5",
    "causal;window=3;stride=5;global=0,77:80",
    "bidir",
    "bidir;radius=40;stride=16",
    "bidir;radius=5;global=0:3,150,299",
    "causal;window=9;dilation=2",
    "blocks;block=64;radius=1;random=3;seed=0;global=0:8",
]


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def run(gpu, spec, q, k, v, g):
    """Forward with LSE, then backward, on the GPU; returns CPU tensors."""
    B, H, T, d = q.shape
    announce(f"bwd {q.dtype} B={B} H={H} T={T} d={d} spec={spec}")
    qd, kd, vd, gd = (x.cuda() for x in (q, k, v, g))
    od = torch.empty_like(qd)
    lse = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
    if q.dtype == torch.bfloat16:
        gpu.sparse_attn_fwd_lse(qd, kd, vd, od, lse, B, H, T, d, spec)
        gpu.sparse_attn_bwd(qd, kd, vd, od, gd, lse, dq, dk, dv, B, H, T, d, spec)
    else:
        gpu.sparse_attn_fwd_lse_f32(qd, kd, vd, od, lse, B, H, T, d, spec)
        gpu.sparse_attn_bwd_f32(qd, kd, vd, od, gd, lse, dq, dk, dv, B, H, T, d, spec)
    torch.cuda.synchronize()
    return od.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def check_grad(got, ref, dtype, what):
    g = got.double().numpy()
    assert np.isfinite(g).all(), f"non-finite {what}"
    if dtype == "bf16":
        tol = 3e-2 * max(1.0, np.abs(ref).max())
        err = np.abs(g - ref).max()
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.3e}"
        return err / tol
    err = np.abs(g - ref).max()
    assert err <= 1e-4 * max(1.0, np.abs(ref).max()), f"{what}: max abs err {err:.3e}"
    g2, r2 = g.reshape(-1, g.shape[-1]), ref.reshape(-1, ref.shape[-1])
    scale = np.maximum(np.abs(r2).max(-1), 1e-30)
    rowrel = (np.abs(g2 - r2).max(-1) / scale)
    rowrel = rowrel[np.abs(r2).max(-1) > 1e-3].max(initial=0.0)
    assert rowrel <= 1e-3, f"{what}: row-normwise rel err {rowrel:.3e}"
    return rowrel


def full_check(gpu, spec, B, H, T, d, dtype, seed):
    q, k, v = inputs.qkv(B, H, T, d, dtype, seed)
    g = inputs.qkv(B, H, T, d, dtype, seed + 500)[0]
    o, lse, dq, dk, dv = run(gpu, spec, q, k, v, g)
    _, lse_ref, _ = oracle.forward_rows(spec, q, k, v)
    lse_tol = 2.0 ** -8 if dtype == "bf16" else 1e-4
    assert np.abs(lse.double().numpy() - lse_ref).max() <= lse_tol, f"lse {spec}"
    # the backward's upstream inputs are the GPU's own O (as in training)
    rq, rk, rv = oracle.backward(spec, q, k, v, g)
    worst = 0.0
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        worst = max(worst, check_grad(got, ref, dtype, f"{nm} {spec} T={T} d={d} {dtype}"))
    return worst


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("spec", SPECS)
def test_backward_small_ragged(gpu, spec, d, dtype):
    """T=300: 3 query blocks, 3 key blocks of the dK/dV pass, ragged tails."""
    full_check(gpu, spec, 2, 2, 300, d, dtype, seed=zlib.crc32(f"{spec}/{d}".encode()) % 1000)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 128, 129, 257])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_edge_lengths(gpu, T, dtype):
    for spec in ["causal;window=5;stride=7", "bidir;radius=9;global=0"]:
        full_check(gpu, spec, 1, 2, T, 64, dtype, seed=T)



@pytest.mark.parametrize("T", [1, 63, 64, 65, 130, 257])
def test_backward_block_mode_64_row_tiles(gpu, T):
    """Block mode with 64-key blocks at bf16 d = 64 runs the backward on
    64-query and 64-key blocks (two waves per workgroup)."""
    specs = ["blocks;block=64;radius=1;random=2;seed=4"]
    if T >= 3:
        specs.append("blocks;block=64;random=3;seed=1;stride=29;global=0:3")
    for spec in specs:
        assert gpu.sparse_attn_plan_info(spec, T, 64)["bq"] == 64
        full_check(gpu, spec, 2, 2, T, 64, "bf16", seed=T)

@pytest.mark.parametrize("cap", [1, 2, 3])
@pytest.mark.parametrize("spec,T,d", [
    ("bidir;radius=64;stride=16;phase=0;global=0:128", 700, 64),
    ("causal;window=64;stride=8;phase=3;global=5:9", 500, 128),
    ("causal;window=100;global=300:340", 650, 128),
    ("blocks;block=64;radius=1;random=3;seed=0;global=0:128", 900, 64),
])
def test_backward_split_forced(gpu, monkeypatch, spec, T, d, cap):
    """Every query block (dQ pass) and key block (dK/dV pass) above `cap`
    tiles split into items whose partials the merge kernels sum."""
    monkeypatch.setenv("SA_FWD_SPLIT_TILES", str(cap))
    full_check(gpu, spec, 2, 2, T, d, "bf16", seed=cap)


def test_backward_global_rows_automatic(gpu):
    """Global rows 0..127 of a 2K bidirectional layer: their query block and
    the key blocks of the global columns read every tile, so both passes
    split them by themselves."""
    full_check(gpu, "bidir;radius=64;stride=16;phase=0;global=0:128", 1, 3, 2048, 128, "bf16", seed=7)


@pytest.mark.parametrize("case", range(80))
def test_backward_random_specs(gpu, case):
    """Seeded random specs (all modes and fields, ragged lengths up to 600):
    forward LSE and dQ, dK, dV against the oracle, bf16 d = 64 / 128 on the
    fast kernels and fp32 or small d on the generic ones."""
    import random
    rng = random.Random(5000 + case)
    T = rng.randrange(1, 600)
    spec = random_spec(rng, T)
    B, H = rng.randrange(1, 3), rng.randrange(1, 3)
    if case % 4 == 3:
        d, dtype = rng.choice([16, 32, 64]), "f32"
    else:
        d, dtype = rng.choice([64, 128]), "bf16"
    full_check(gpu, spec, B, H, T, d, dtype, seed=case)


def test_backward_window_layer_2k(gpu):
    """B=1, H=4, T=2048, d=128, causal window 256: every gradient compared."""
    full_check(gpu, "causal;window=256", 1, 4, 2048, 128, "bf16", seed=3)


def test_backward_is_deterministic(gpu):
    q, k, v = inputs.qkv(1, 4, 1024, 128, "bf16", 4)
    g = inputs.qkv(1, 4, 1024, 128, "bf16", 5)[0]
    a = run(gpu, "causal;window=200;stride=64", q, k, v, g)
    b = run(gpu, "causal;window=200;stride=64", q, k, v, g)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def heads_check(spec, tensors, outputs, heads):
    """Full-size backward, already run on the GPU: the listed (b, h) pairs
    checked in full (every row of LSE and dQ, every key of dK and dV)
    against the fp64 oracle."""
    q, k, v, g = tensors
    o, lse, dq, dk, dv = outputs
    for b, h in heads:
        announce(f"oracle bwd {spec} b={b} h={h}")
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs, gs = (x[sl] for x in (q, k, v, g))
        _, lse_ref, _ = oracle.forward_rows(spec, qs, ks, vs)
        assert np.abs(lse[sl].double().numpy() - lse_ref).max() <= 2.0 ** -8, f"lse b={b} h={h}"
        rq, rk, rv = oracle.backward(spec, qs, ks, vs, gs)
        check_grad(dq[sl], rq, "bf16", f"dQ {spec} b={b} h={h}")
        check_grad(dk[sl], rk, "bf16", f"dK {spec} b={b} h={h}")
        check_grad(dv[sl], rv, "bf16", f"dV {spec} b={b} h={h}")


def full_size(gpu, spec, B, H, T, d, seed):
    q, k, v = inputs.qkv(B, H, T, d, "bf16", seed)
    g = inputs.qkv(B, H, T, d, "bf16", seed + 500)[0]
    return (q, k, v, g), run(gpu, spec, q, k, v, g)


MISTRAL = "causal;window=4096"


@pytest.fixture(scope="module")
def mistral_bwd(gpu):
    """The 32K-window layer (B=1, H=32, T=32768, d=128) forward with LSE and
    backward, run once on the GPU in full."""
    return full_size(gpu, MISTRAL, 1, 32, 32768, 128, seed=0)


def test_backward_mistral_32k_window_full_size_heads_0_17(mistral_bwd):
    heads_check(MISTRAL, *mistral_bwd, heads=[(0, 0), (0, 17)])


def test_backward_mistral_32k_window_full_size_heads_9_31(mistral_bwd):
    """Two more whole heads, the last one included: a fault confined to
    later query blocks or to one XCD's slice of the heads shows here."""
    heads_check(MISTRAL, *mistral_bwd, heads=[(0, 9), (0, 31)])


def test_backward_bigbird_4k_full_size(gpu):
    """The 4K BigBird layer at full size (B=8, H=12, T=4096, d=64, 64-row
    plans): three (b, h) slices compared in full."""
    spec = "blocks;block=64;radius=1;random=3;seed=0;global=0:128"
    heads_check(spec, *full_size(gpu, spec, 8, 12, 4096, 64, seed=1),
                heads=[(0, 0), (3, 7), (7, 11)])


def test_backward_longformer_16k_full_size(gpu):
    """The Longformer 16K layer at full size (B=1, H=16, T=16384, d=64):
    band, strided landmark keys and 128 global rows, whose plan splits the
    global-row query block and runs the strided keys as gathered key blocks
    in the dK/dV pass.  Three whole heads, the first and last included,
    compared in full."""
    spec = "bidir;radius=256;stride=16;phase=0;global=0:128"
    heads_check(spec, *full_size(gpu, spec, 1, 16, 16384, 64, seed=2),
                heads=[(0, 0), (0, 7), (0, 15)])


def test_backward_at_max_length(gpu):
    """T = SA_MAX_T = 2^22 (the longest sequence the library accepts), d = 128,
    causal window of 256: Q, K, V, dO and each gradient of the sequence span
    exactly 1 GiB.  The window rule depends on i - j only, so the oracle run
    on a slice [a, b) of the sequence alone gives exact values for the rows
    whose keys all lie in the slice (dQ and LSE of rows i >= a + 255, every
    row when a = 0) and for the keys whose queries and those queries' keys
    all lie in it (dK and dV of keys a + 255 <= j < b - 255, without the
    first bound when a = 0 and without the second when b = T).  Slices at
    the start, the middle and the end of the sequence are checked."""
    T, d, W = 1 << 22, 128, 256
    spec = f"causal;window={W}"
    q, k, v = inputs.qkv(1, 1, T, d, "bf16", 13)
    g = inputs.qkv(1, 1, T, d, "bf16", 513)[0]
    _, lse, dq, dk, dv = run(gpu, spec, q, k, v, g)
    for a, b in ((0, 4096), (T // 2 - 2048, T // 2 + 2048), (T - 4096, T)):
        announce(f"oracle bwd {spec} T={T} slice {a}..{b}")
        sl = (slice(None), slice(None), slice(a, b))
        qs, ks, vs, gs = (x[sl].contiguous() for x in (q, k, v, g))
        _, lse_ref, _ = oracle.forward_rows(spec, qs, ks, vs)
        rq, rk, rv = oracle.backward(spec, qs, ks, vs, gs)
        r0 = 0 if a == 0 else W - 1            # first exact row (slice index)
        k1 = (b - a) if b == T else (b - a) - (W - 1)  # one past the last exact key
        assert np.abs(lse[0, 0, a + r0:b].double().numpy() - lse_ref[0, 0, r0:]).max() <= 2.0 ** -8
        check_grad(dq[:, :, a + r0:b], rq[:, :, r0:], "bf16", f"dQ max length rows {a + r0}..{b - 1}")
        check_grad(dk[:, :, a + r0:a + k1], rk[:, :, r0:k1], "bf16", f"dK max length keys {a + r0}..{a + k1 - 1}")
        check_grad(dv[:, :, a + r0:a + k1], rv[:, :, r0:k1], "bf16", f"dV max length keys {a + r0}..{a + k1 - 1}")
