"""Seeded random mask specs for the GPU parity fuzz tests (test helper; no
method arithmetic: it only writes spec text of the grammar)."""


def random_spec(rng, T):
    """A spec of the grammar with random fields (globals inside [0, T))."""
    mode = rng.choice(["causal", "bidir", "blocks"])
    if mode == "blocks":
        spec = (f"blocks;block={rng.choice([16, 32, 48, 64, 64, 96, 128])};radius={rng.randrange(3)}"
                f";random={rng.randrange(5)};seed={rng.randrange(1000)}")
    elif mode == "bidir":
        spec = "bidir" + (f";radius={rng.randrange(200)}" if rng.random() < 0.8 else "")
        if rng.random() < 0.2:
            spec += f";dilation={rng.randrange(1, 5)}"
    else:
        spec = f"causal;window={rng.randrange(1, 500) if rng.random() < 0.85 else 0}"
        if rng.random() < 0.25:
            spec += f";dilation={rng.randrange(1, 5)}"
    if rng.random() < 0.5:
        st = rng.randrange(2, 70)
        spec += f";stride={st};phase={rng.randrange(st)}"
    if rng.random() < 0.5:
        rs = []
        for _ in range(rng.randrange(1, 4)):
            a = rng.randrange(T)
            rs.append(f"{a}:{min(T, a + 1 + rng.randrange(max(1, T // 6)))}" if rng.random() < 0.7 else str(a))
        spec += ";global=" + ",".join(rs)
    return spec
