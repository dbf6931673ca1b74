"""Planted slips for the oracle mutation check: (name, original text, mutated text)."""

MUTANTS = [
    ("dropped scale", "s = float(scale) * (qrows @ kh.T)", "s = (qrows @ kh.T)"),
    ("exponent sign", "e = np.exp(z - m)", "e = np.exp(m - z)"),
    ("transposed weights", "o = a @ vh", "o = a.T @ vh[: a.shape[0]]"),
    ("keys used as values", "o = a @ vh", "o = a @ kh"),
    ("max over wrong axis", "m = z.max(axis=1, keepdims=True)", "m = z.max(axis=0, keepdims=True)"),
    ("sum over wrong axis", "l = e.sum(axis=1, keepdims=True)", "l = e.sum(axis=0, keepdims=True)"),
    ("strict causal", "vis &= j <= rows[:, None]", "vis &= j < rows[:, None]"),
    ("causal upper triangle", "vis &= j <= rows[:, None]", "vis &= j >= rows[:, None]"),
    ("padding off by one", "vis &= j < int(key_len)", "vis &= j <= int(key_len)"),
    ("interleaved head map", "g = h // G", "g = h % Hkv"),
    ("lse without max", "lse = (m + np.log(l))[:, 0]", "lse = np.log(l)[:, 0]"),
    ("unweighted merge", "w = np.exp(lse_part - M)", "w = np.ones_like(lse_part)"),
    ("merge lse without max", "lse = (M + np.log(den))[..., 0]", "lse = np.log(den)[..., 0]"),
    ("short split chunks", "chunk = -(-Sk // num_splits)", "chunk = max(1, Sk // num_splits)"),
    ("split ignores padding", "vis = vis_all[:, lo:hi]", "vis = np.ones_like(vis_all[:, lo:hi])"),
]
