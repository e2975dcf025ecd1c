"""GPU parity of windowed decode against the fp64 oracle.

Decode reads a ring-buffer cache: position t of sequence b sits in row t mod
C.  The expected value of new token i is the oracle's forward row over the
sequence of live positions, with each KV head's keys and values repeated for
the query heads that share it.  Cache rows that hold no live position are
filled with large values, so reading one would show.
Tolerance as for the bf16 forward: elementwise |O - O*| <= 2e-2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_masked_spec_amd import inputs

pytestmark = pytest.mark.gpu

BF16_ATOL = 2e-2


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def ring_rows(pos_b, C):
    """Ring row of window slot x (x = 0..C-1 stands for position
    pos_b - C + 1 + x), and the first slot whose position is >= 0."""
    x = np.arange(C)
    return (pos_b + 1 + x) % C, max(0, C - 1 - pos_b)


def run_decode(gpu, spec, B, H, Hkv, n_new, C, d, pos, seed, check_rows=None):
    """Random keys/values for the C most recent positions of each sequence
    (slot x is position pos - C + 1 + x), written into the ring; decode the
    last n_new tokens; compare with the oracle's rows for those tokens.

    The oracle gets the sequence of live positions.  Where pos >= C that is
    the full sequence shifted by pos - C + 1; for a window rule this leaves
    every row's allowed set unchanged, because the rule depends on i - j
    only and the cache holds the whole window (C >= reach + n_new)."""
    G = H // Hkv
    _, kv_k, kv_v = inputs.qkv(B, Hkv, C, d, "bf16", seed)
    q_new = inputs.qkv(B, H, n_new, d, "bf16", seed + 1000)[0]
    kc = inputs.scaled(kv_v.flip(2), 60.0)  # large junk in rows with no live position
    vc = inputs.scaled(kv_k.flip(2), 60.0)
    for b in range(B):
        rows, x0 = ring_rows(int(pos[b]), C)
        live = torch.from_numpy(rows[x0:])
        kc[b][:, live] = kv_k[b][:, x0:]
        vc[b][:, live] = kv_v[b][:, x0:]
    announce(f"decode B={B} H={H} Hkv={Hkv} n_new={n_new} C={C} d={d} spec={spec}")
    qd, kd, vd = q_new.cuda(), kc.cuda(), vc.cuda()
    od = torch.empty_like(qd)
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    gpu.sparse_attn_decode(qd, kd, vd, od, posd, B, H, Hkv, n_new, C, d, spec)
    torch.cuda.synchronize()
    got = od.cpu()
    assert torch.isfinite(got.float()).all()
    worst = 0.0
    for b in (range(B) if check_rows is None else check_rows):
        _, x0 = ring_rows(int(pos[b]), C)
        Lp = C - x0                                  # live positions, shifted to 0..Lp-1
        kx = kv_k[b][:, x0:].repeat_interleave(G, dim=0)[None]
        vx = kv_v[b][:, x0:].repeat_interleave(G, dim=0)[None]
        qx = torch.zeros(1, H, Lp, d, dtype=torch.bfloat16)
        qx[0, :, Lp - n_new:] = q_new[b]
        rows = [(0, h, Lp - n_new + t) for h in range(H) for t in range(n_new)]
        ref, _, _ = oracle.forward_rows(spec, qx, kx, vx, rows=rows)
        g = got[b].reshape(H * n_new, d).double().numpy()
        err = np.abs(g - ref).max()
        worst = max(worst, err)
        assert err <= BF16_ATOL, f"b={b} pos={pos[b]}: max abs err {err:.3e}"
    return worst


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_window_cache_exactly_w_rows(gpu, d):
    """C = w: the cache holds exactly the window; wrapped and unwrapped rings."""
    run_decode(gpu, "causal;window=64", 4, 8, 2, 1, 64, d, [200, 64, 63, 10], seed=d)


def test_cache_larger_than_window_masks_live_rows(gpu):
    """Live positions older than the window are in the cache and must be
    excluded by the rule."""
    run_decode(gpu, "causal;window=16", 3, 4, 4, 1, 40, 128, [100, 39, 20], seed=1)


@pytest.mark.parametrize("n_new", [2, 3, 5])
def test_several_new_tokens(gpu, n_new):
    C = 16 + n_new - 1
    run_decode(gpu, "causal;window=16", 2, 6, 3, n_new, C, 64, [150, C + 3], seed=n_new)


def test_dilated_window(gpu):
    """One new token visits only its grid; several use the mask."""
    spec = "causal;window=8;dilation=3"
    run_decode(gpu, spec, 3, 4, 2, 1, 22, 128, [100, 21, 30], seed=3)
    run_decode(gpu, spec, 2, 4, 2, 2, 23, 64, [77, 40], seed=4)


def test_unlimited_window_full_context(gpu):
    """window=0 with the whole context cached (pos < C)."""
    run_decode(gpu, "causal", 2, 4, 1, 1, 300, 128, [299, 150], seed=5)
    run_decode(gpu, "causal", 1, 2, 2, 3, 300, 64, [250], seed=6)


@pytest.mark.parametrize("H,Hkv", [(16, 1), (4, 4), (32, 8), (12, 4)])
def test_head_grouping(gpu, H, Hkv):
    """G = H / Hkv query heads per KV head, including more than 8 queries per
    KV head (several query chunks) and plain multi-head (G = 1)."""
    run_decode(gpu, "causal;window=32", 2, H, Hkv, 1, 32, 128, [80, 31], seed=H)


def test_key_splits_long_cache(gpu):
    """A long window on few sequences runs many key splits through the
    workspace and the merge kernel."""
    run_decode(gpu, "causal;window=3000", 1, 8, 2, 1, 3000, 128, [5000], seed=7)
    run_decode(gpu, "causal;window=3000", 1, 8, 2, 2, 3001, 64, [3001], seed=8)


def test_mistral_decode_batch_every_sequence(gpu):
    """B=64, H=32, Hkv=8, d=128, window 4096, C=4096: the bench shape, in the
    launch configuration the bench times; every sequence's 32 new rows
    checked against the oracle."""
    rng = np.random.default_rng(0)
    pos = [int(x) for x in rng.integers(4096, 9000, size=64)]
    pos[0], pos[1] = 4095, 4096
    worst = run_decode(gpu, "causal;window=4096", 64, 32, 8, 1, 4096, 128, pos, seed=9)
    announce(f"decode bench shape, all 64 sequences: max abs err {worst:.3e}")


@pytest.mark.parametrize("case", range(40))
def test_decode_random_shapes(gpu, case):
    """Seeded random decode calls: window (or unlimited, then every position
    still cached), dilation, head grouping, new-token count, head size,
    cache length at or above the minimum, and per-sequence positions before
    and long after the ring wraps."""
    import random
    rng = random.Random(7000 + case)
    d = rng.choice([16, 32, 64, 128])
    H, Hkv = rng.choice([(1, 1), (4, 1), (8, 2), (6, 3), (16, 4), (32, 8)])
    n_new = rng.choice([1, 1, 1, 2, 3, 5])
    dil = rng.choice([1, 1, 2, 3])
    B = rng.randrange(1, 5)
    if rng.random() < 0.15:
        spec = "causal;window=0" + (f";dilation={dil}" if dil > 1 else "")
        C = rng.randrange(n_new, 1500)
        hi = C  # unlimited window: the cache holds the whole context
    else:
        spec = f"causal;window={rng.randrange(1, 800)}" + (f";dilation={dil}" if dil > 1 else "")
        C = gpu.sparse_attn_decode_cache_rows(spec, n_new) + rng.randrange(0, 300)
        hi = C + 3000
    pos = [rng.randrange(n_new - 1, hi) for _ in range(B)]
    run_decode(gpu, spec, B, H, Hkv, n_new, C, d, pos, seed=case)


def test_decode_and_forward_last_rows_match_the_oracle(gpu):
    """Decode of the last token and the forward's last row, on the same
    inputs (MHA, full sequence in the cache), each against the oracle's row;
    the two GPU results are also within the sum of their bounds of each
    other (a consistency check, not the parity criterion)."""
    B, H, T, d, spec, C = 2, 4, 512, 128, "causal;window=128", 128
    q, k, v = inputs.qkv(B, H, T, d, "bf16", 10)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    of = torch.empty_like(qd)
    announce(f"fwd + decode last row B={B} H={H} T={T} spec={spec}")
    gpu.sparse_attn_fwd(qd, kd, vd, of, B, H, T, d, spec)
    t = torch.arange(T - C, T)
    kc = torch.empty(B, H, C, d, dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    kc[:, :, t % C] = k[:, :, t]
    vc[:, :, t % C] = v[:, :, t]
    od = torch.empty(B, H, 1, d, dtype=torch.bfloat16, device="cuda")
    posd = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    gpu.sparse_attn_decode(qd[:, :, T - 1:].contiguous(), kc.cuda(), vc.cuda(), od, posd,
                           B, H, H, 1, C, d, spec)
    torch.cuda.synchronize()
    rows = [(b, h, T - 1) for b in range(B) for h in range(H)]
    ref, _, _ = oracle.forward_rows(spec, q, k, v, rows=rows)
    dec = od[:, :, 0].cpu().double().numpy().reshape(-1, d)
    fwd = of[:, :, T - 1].cpu().double().numpy().reshape(-1, d)
    assert np.abs(dec - ref).max() <= BF16_ATOL
    assert np.abs(fwd - ref).max() <= BF16_ATOL
    assert np.abs(dec - fwd).max() <= 2 * BF16_ATOL


def test_decode_on_a_side_stream_and_release(gpu):
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run_decode(gpu, "causal;window=3000", 1, 4, 1, 1, 3000, 128, [4000], seed=11)
    torch.cuda.synchronize()
    gpu.sparse_attn_release_cache()
    run_decode(gpu, "causal;window=3000", 1, 4, 1, 1, 3000, 128, [4000], seed=11)
