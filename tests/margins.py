"""Encode margins for the tests: how clearly each (vector, head, segment)
decides its nearest codeword.

The margin is the float64 gap between the second-smallest and the smallest
squared Euclidean distance to the codewords.  Where it exceeds 1e-4 the
GPU's fp32 decision and the oracle's float64 one cannot differ, so codes
are compared bit for bit only on inputs whose every margin clears it
(ties built on purpose are the one exception, and the tests that build them
leave those entries out).
"""
import numpy as np

MIN_MARGIN = 1e-4


def encode_margins(x, cb, block=4096):
    """float64 best-vs-second distance gap, [N, H, M], for x fp16 [N, H, D]
    and cb fp16 [H, M, K, ds]; blockwise, so large N stays in memory."""
    N, H, D = x.shape
    _, M, K, ds = cb.shape
    c = cb.astype(np.float64)
    out = np.empty((N, H, M))
    for lo in range(0, N, block):
        hi = min(N, lo + block)
        xs = x[lo:hi].astype(np.float64).reshape(hi - lo, H, M, ds)
        for h in range(H):
            for m in range(M):
                # |x|^2 - 2 x.c + |c|^2: float64 keeps it within ~1e-13 of the
                # direct sum at these magnitudes, far below MIN_MARGIN
                xm = xs[:, h, m]
                d = (xm * xm).sum(-1)[:, None] - 2.0 * (xm @ c[h, m].T) + (c[h, m] ** 2).sum(-1)[None]
                part = np.partition(d, 1, axis=1)
                out[lo:hi, h, m] = part[:, 1] - part[:, 0]
    return out


def assert_clear_margins(x, cb, what="", mask=None):
    """Every margin (where mask is True, if given) is above MIN_MARGIN."""
    g = encode_margins(x, cb)
    if mask is not None:
        g = g[mask]
    assert g.size == 0 or g.min() > MIN_MARGIN, \
        f"{what}: an encode margin of {g.min():.3e} is below {MIN_MARGIN}: regenerate the case"
    return float(g.min()) if g.size else float("inf")


def assert_lloyd_margins(x, cb_init, n_iter, oracle, what=""):
    """The margins of every assignment of an n_iter Lloyd run from cb_init
    (the oracle's iterations, step by step): each must clear MIN_MARGIN for a
    bit-exact comparison of the whole run to be meaningful."""
    cb = cb_init.copy()
    for it in range(int(n_iter) + 1):
        assert_clear_margins(x, cb, f"{what} assignment {it}")
        if it == n_iter:
            break
        cb, _ = oracle.codebook_update(x, oracle.encode(x, cb), cb)
