"""The V histogram's fixed point, emulated on the CPU.

The score kernels add every token's softmax weight p_t = 2^(s_t - m_c) to
32-bit integer bins as u_t = round(p_t * 2^S) (LDS float atomics are slow on
gfx950).  S is taken per (chunk, head) from the chunk's mass
l_c = sum_t p_t: rows of 16 tokens are summed in fp32, each row sum is
rounded up to a multiple of 2^-16 and added as an integer, and
S = 30 - ceil(log2 of that estimate), clamped to [14, 30].  The bins are
then read back as fp32, times 2^-S, split into fp16 high and low parts and
contracted with the fp16 V codebook (exact products, wide sums).

This file runs that arithmetic step by step in NumPy on softmax
distributions with one dominant "sink" token (the sharp case of the chunked
softmax of the PAM page, section 2.2.3 (1), and of the online rescaling of
the memory-wall chapter, section 1.4.3 (5.1)), next to the exact float64
attention, for chunks of 1024, 2048 and 4096 tokens.  It also runs the
capacity-based scale S = 31 - log2(T) (a bin can never overflow, whatever
the mass) on the same inputs, to show that these inputs are sharp enough to
break a 1e-3 bar when the scale ignores the mass.
"""
import math

import numpy as np
import pytest

LOG2E = 1.4426950408889634


def _clz32(x):
    return 32 - int(x).bit_length()


def mass_shift(p32):
    """S from the rows' rounded-up fixed-point sums (the kernels' fix_shift)."""
    T = p32.size
    rows = np.zeros(-(-T // 16) * 16, np.float32)
    rows[:T] = p32
    row_sums = rows.reshape(-1, 16).sum(axis=1, dtype=np.float32)
    lest = int(np.ceil(row_sums.astype(np.float64) * 65536.0).sum())
    x = lest - 1 if lest > 65536 else 65535
    return 30 - 16 + _clz32(x)


def emulate(s_nat, vcodes, vcb, shift):
    """o / l of one (chunk, head) as the kernels compute it.

    s_nat fp64 [T] natural-log scores; vcodes int [T, M]; vcb fp16 [M, K, ds];
    shift: "mass" (the kernels) or "capacity" (31 - log2 T, for contrast)."""
    T = s_nat.size
    M, K, ds = vcb.shape
    s2 = (s_nat * LOG2E).astype(np.float32)                 # base-2 scores, fp32
    m = s2.max()
    p = np.exp2(s2 - m).astype(np.float32)                  # 2^(s - m_c) <= 1
    S = mass_shift(p) if shift == "mass" else 31 - int(math.log2(T))
    scaled = (p.astype(np.float64) * 2.0 ** S).astype(np.float32)     # exact
    u = np.floor(scaled + np.float32(0.5)).astype(np.int64)             # fma(p, 2^S, 0.5), truncated
    bins = np.zeros((M, K), np.int64)
    for mm in range(M):
        np.add.at(bins[mm], vcodes[:, mm], u)
    assert bins.sum(axis=1).max() < 2 ** 31, "a segment's bins exceed 31 bits"
    l = float(bins[0].sum()) * 2.0 ** -S
    f = (bins.astype(np.float32) * np.float32(2.0 ** -S)).astype(np.float32)
    hi = f.astype(np.float16)
    lo = (f - hi.astype(np.float32)).astype(np.float16)
    w = hi.astype(np.float64) + lo.astype(np.float64)        # what the matrix cores weight
    o = np.concatenate([w[mm] @ vcb[mm].astype(np.float64) for mm in range(M)])
    return o / l


def exact(s_nat, vcodes, vcb):
    M, K, ds = vcb.shape
    p = np.exp(s_nat - s_nat.max())
    v = np.concatenate([vcb[mm].astype(np.float64)[vcodes[:, mm]] for mm in range(M)], axis=1)
    return (p @ v) / p.sum()


def sink_case(rng, T, lead, spread):
    """One token `lead` nats above T - 1 others spread uniformly over
    `spread` nats; random V codes; an N(0, 1) fp16 V codebook (M = 4)."""
    s = -lead - rng.uniform(0.0, spread, size=T)
    s[rng.integers(T)] = 0.0
    vcodes = rng.integers(0, 256, size=(T, 4))
    vcb = rng.standard_normal((4, 256, 32)).astype(np.float16)
    return s, vcodes, vcb


CASES = [(T, lead, spread) for T in (1024, 2048, 4096)
         for lead, spread in ((12.0, 0.0), (13.0, 0.05), (15.0, 0.05), (16.0, 0.0), (12.0, 2.0))]


@pytest.mark.parametrize("T,lead,spread", CASES)
def test_mass_scaled_fixed_point_on_sink_softmax(T, lead, spread):
    rng = np.random.default_rng(int(T + lead * 10 + spread * 100))
    s, vc, vcb = sink_case(rng, T, lead, spread)
    ref = exact(s, vc, vcb)
    got = emulate(s, vc, vcb, "mass")
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err <= 2e-4, f"T={T} lead={lead}: {err:.2e} of max|out|"


def test_uniform_and_random_scores():
    """Flat and N(0, 1)-like chunks (the common case): l_c ~ T, S = 30 -
    log2 T, the bins near their bound and still no overflow."""
    rng = np.random.default_rng(5)
    for T in (1024, 4096):
        for s in (np.zeros(T), rng.normal(0.0, 1.0, T), rng.normal(0.0, 3.0, T)):
            vc = rng.integers(0, 256, size=(T, 4))
            vcb = rng.standard_normal((4, 256, 32)).astype(np.float16)
            ref = exact(s, vc, vcb)
            err = np.abs(emulate(s, vc, vcb, "mass") - ref).max() / np.abs(ref).max()
            assert err <= 2e-4


def test_shift_rule():
    """S = 30 - ceil(log2 l_c) from the estimate, clamped to [14, 30]."""
    one = np.zeros(16, np.float32)
    one[3] = 1.0
    assert mass_shift(one) == 30                     # l = 1
    two = one.copy()
    two[5] = 1.0
    assert mass_shift(two) == 29                     # l = 2 -> ceil(log2) = 1
    assert mass_shift(np.full(4096, 1.0, np.float32)) == 18      # l = 4096
    assert mass_shift(np.full(4096, 0.999, np.float32)) == 18
    assert mass_shift(np.full(65536, 1.0, np.float32)) == 14     # the clamp's floor
    just_above = one.copy()
    just_above[7] = 2.0 ** -20
    assert mass_shift(just_above) == 29              # rounded up: never underestimates


def test_capacity_scale_breaks_on_sink_softmax():
    """The same inputs with S = 31 - log2(T): the sub-quantum weights of the
    4095 clustered tokens are rounded as a block, and the output misses the
    1e-3 bar -- the case the mass-based scale exists for."""
    worst = 0.0
    for lead, spread in ((12.0, 0.0), (13.0, 0.05), (14.0, 0.05), (15.0, 0.05)):
        rng = np.random.default_rng(int(lead * 10))
        s, vc, vcb = sink_case(rng, 4096, lead, spread)
        ref = exact(s, vc, vcb)
        worst = max(worst, np.abs(emulate(s, vc, vcb, "capacity") - ref).max() / np.abs(ref).max())
    assert worst > 1e-3
