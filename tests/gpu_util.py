"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch


def np_(t):
    """Device tensor -> numpy (bf16 is widened to float32 exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def rel_fro(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def assert_finite(*arrs):
    for a in arrs:
        a = np.asarray(a, dtype=np.float64)
        assert np.isfinite(a).all(), "NaN/Inf in a GPU output"


def say(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------- full-size sampling
def sample_rows(r0, r1, rng, block=64, extra=8):
    """Rows of one expert to check: all of them up to 2 blocks; else the first and last row
    of every 64-row block (so every m-tile of the GEMMs and both its edges) plus a few at
    random."""
    if r1 - r0 <= 2 * block:
        return np.arange(r0, r1)
    starts = np.arange(r0, r1, block)
    ends = np.minimum(starts + block - 1, r1 - 1)
    return np.unique(np.concatenate([starts, ends, rng.integers(r0, r1, extra)]))


def sample_cols(n, rng, block=64, per=4):
    """Columns to check: `per` distinct random columns from every 64-column block, so every
    weight-row tile of the GEMMs is hit."""
    cols = [b + rng.choice(min(block, n - b), size=min(per, n - b), replace=False) for b in range(0, n, block)]
    return np.sort(np.concatenate(cols))


def check_every_expert(offsets, tok, A_all, h_got, y_got, h_in_rows, deq13, deq2, F, H, round_h, tol_h,
                       tol_y=1e-5, seed=0):
    """Both GEMMs of every active expert against the oracle on identical operands: for each
    expert, sampled rows (sample_rows) x sampled columns (sample_cols) of h = SwiGLU(A W13^T)
    and of Y = h_in W2^T. deq13(e, idx) / deq2(e, idx) give the float64 weight rows idx of the
    expert's W13 / W2 (dequantized by the oracle from the GPU's codes); h_in_rows(rows) the
    down GEMM's float64 input rows; round_h the rounding of h as the GPU stores it. Every
    expert must be within tol_h (h) and tol_y (Y) relative Frobenius error on its sample."""
    from oracle import moe as omoe
    rng = np.random.default_rng(seed)
    act = np.nonzero(np.diff(offsets))[0]
    worst = [0.0, 0.0]
    for e in act:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        rows = sample_rows(r0, r1, rng)
        ch = sample_cols(F, rng)
        G = A_all[tok[rows]] @ deq13(int(e), np.concatenate([ch, F + ch])).T
        rh = rel_fro(np.asarray(h_got[np.ix_(rows, ch)], np.float64), round_h(omoe.swiglu(G)))
        cy = sample_cols(H, rng)
        ry = rel_fro(np.asarray(y_got[np.ix_(rows, cy)], np.float64), h_in_rows(rows) @ deq2(int(e), cy).T)
        assert rh <= tol_h and ry <= tol_y, f"expert {e} ({r1 - r0} rows): rel(h) {rh:.2e} rel(Y) {ry:.2e}"
        worst = [max(worst[0], rh), max(worst[1], ry)]
    say(f"{len(act)} experts checked: worst rel(h) {worst[0]:.2e} rel(Y) {worst[1]:.2e}")
    return len(act)


def bf16_ulp(v):
    """Spacing of bfloat16 numbers at |v| (8 significant bits; the subnormal spacing 2^-133
    below 2^-126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(np.maximum(e, -126.0) - 7.0), 2.0 ** -133)


def assert_reduce_elementwise(got, y, slot_to_row, w):
    """The weighted reduce element by element: the kernel sums k products in float32 in
    ascending j and rounds once to bf16, the oracle sums in float64 and rounds once, so
    |got - want| <= one bf16 ulp (two half-ulp roundings) + the float32 summation bound
    k * 2^-23 * sum_j |w_j y_j| (a margin of 2 on k u). NaN must match NaN."""
    from oracle import moe as omoe
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = w.shape[1]
    want = omoe.bf16_round(omoe.unpermute_reduce(y, slot_to_row, w))
    mag = omoe.unpermute_reduce(np.abs(y), slot_to_row, np.abs(w))
    got = np.asarray(got, dtype=np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    tol = bf16_ulp(np.maximum(np.abs(want), np.abs(got))) + k * 2.0 ** -23 * mag
    err = np.abs(got - want)
    bad = fin & (err > tol)
    assert not bad.any(), f"{bad.sum()} reduce outputs off by more than 1 bf16 ulp (worst {err[bad].max():.3e})"
    return want
