"""GPU parity for codebook learning (Lloyd iterations) through the C ABI.

The update step sums every member exactly and rounds one double-precision
mean to fp16, as the oracle does, so codebooks are compared bit for bit;
codes are bit-exact as for encode.  Inputs come from the seeded generators
(vectors around the codewords of a generating codebook, a perturbed start).
"""
import sys

import numpy as np
import pytest

import oracle
from margins import assert_clear_margins, assert_lloyd_margins
from synth import gen

torch = pytest.importorskip("torch")
pq = pytest.importorskip("decode_attention_product_amd")

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[kmeans] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pq.load_library()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def same_bits(got, ref):
    np.testing.assert_array_equal(np.asarray(got).view(np.uint16), np.asarray(ref).view(np.uint16))


UPDATE = [
    # (N, H, M, n_used)
    (1, 1, 4, None),
    (32, 8, 4, None),      # the pages' sample size: most codewords empty
    (32, 8, 8, None),
    (1000, 2, 8, 50),
    (4096, 32, 4, 200),    # a prefill-sized sample over 32 heads
]


@pytest.mark.parametrize("N,H,M,n_used", UPDATE)
def test_update_matches_oracle(N, H, M, n_used):
    say(f"update N={N} H={H} M={M} used={n_used}")
    case = gen.kmeans_case(np.random.default_rng(900 + N + M), N, H, M, sigma=0.1,
                           init_sigma=0.3, n_used=n_used)
    x, cb0 = case["x"], case["cb_init"]
    assert_clear_margins(x, cb0, "update assignment")
    codes = oracle.encode(x, cb0)
    ref, ref_counts = oracle.codebook_update(x, codes, cb0)
    cb = dev(cb0)
    counts = torch.zeros((H, M, 256), dtype=torch.int32, device="cuda")
    pq.pq_codebook_update(dev(x), dev(codes), cb, counts)
    torch.cuda.synchronize()
    same_bits(cb.cpu().numpy(), ref)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_counts)


def test_update_rounding_cases():
    """Means that fall exactly between two fp16 values (normal and subnormal),
    at the top of the fp16 range, of mixed signs and at -0; the other
    segments random."""
    cases = [  # codeword -> member values (every dim of segment 0)
        [1.0, 1.0 + 2**-10],                  # tie -> 1.0 (even)
        [1.0 + 2**-10, 1.0 + 2 * 2**-10],     # tie -> 1 + 2^-9 (even)
        [1.0, 1.0, 1.0 + 2**-10],             # below the tie -> 1.0
        [2**-24, 2 * 2**-24],                 # subnormal tie -> 2^-23
        [65504.0, 65504.0, 65504.0],
        [-3.0, 5.0],
        [2**-24, 0.0],                        # tie between 0 and 2^-24 -> 0
        [-(2**-24), 0.0],                     # -> -0
        [0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.7],
        [-65504.0, 65504.0, 1.5],
    ]
    rng = np.random.default_rng(950)
    rows, code0 = [], []
    for k, vals in enumerate(cases):
        for v in vals:
            rows.append(v)
            code0.append(3 * k + 1)
    N, H, M = len(rows), 1, 4
    x = rng.standard_normal((N, H, 128)).astype(np.float16)
    x[:, 0, :32] = np.array(rows, dtype=np.float16)[:, None]
    codes = rng.integers(0, 256, (N, H, M), dtype=np.uint8)
    codes[:, 0, 0] = code0
    cb0 = rng.standard_normal((H, M, 256, 32)).astype(np.float16)
    ref, _ = oracle.codebook_update(x, codes, cb0)
    cb = dev(cb0)
    pq.pq_codebook_update(dev(x), dev(codes), cb)
    torch.cuda.synchronize()
    got = cb.cpu().numpy()
    same_bits(got, ref)
    assert got[0, 0, 1, 0] == 1.0 and got[0, 0, 4, 0] == 1.0 + 2**-9
    assert got[0, 0, 10, 0] == 2**-23 and got[0, 0, 13, 0] == 65504.0
    assert got[0, 0, 22].view(np.uint16)[0] == 0x8000


KMEANS = [
    # (N, H, M, n_used, n_iter)
    (32, 8, 4, None, 0),
    (32, 8, 4, None, 5),
    (512, 4, 8, 64, 3),
    (2048, 8, 4, 128, 8),
]


@pytest.mark.parametrize("N,H,M,n_used,n_iter", KMEANS)
def test_kmeans_matches_oracle(N, H, M, n_used, n_iter):
    say(f"kmeans N={N} H={H} M={M} used={n_used} iters={n_iter}")
    case = gen.kmeans_case(np.random.default_rng(1000 + N + n_iter), N, H, M, sigma=0.05,
                           init_sigma=0.25, n_used=n_used)
    x, cb0 = case["x"], case["cb_init"]
    assert_lloyd_margins(x, cb0, n_iter, oracle, "kmeans")
    ref_cb, ref_codes = oracle.kmeans(x, cb0, n_iter)
    cb = dev(cb0)
    _, codes = pq.pq_kmeans(dev(x), cb, n_iter)
    torch.cuda.synchronize()
    same_bits(cb.cpu().numpy(), ref_cb)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)


def test_kmeans_strided_sample_from_a_cache_and_order_independence():
    """The sample is the first 32 tokens of request 1 of a [B, H, L, D] K
    tensor, read in place through strides; shuffling the sample's vectors
    gives the same codebook."""
    B, H, L, D, M, N = 3, 4, 64, 128, 4, 32
    case = gen.kmeans_case(np.random.default_rng(1100), B * L, H, M, sigma=0.05, init_sigma=0.25,
                           n_used=24)
    kv = np.ascontiguousarray(case["x"].reshape(B, L, H, D).transpose(0, 2, 1, 3))   # [B, H, L, D]
    sample = np.ascontiguousarray(kv[1, :, :N].transpose(1, 0, 2))                  # [N, H, D]
    assert_lloyd_margins(sample, case["cb_init"], 4, oracle, "strided sample")
    ref_cb, ref_codes = oracle.kmeans(sample, case["cb_init"], 4)
    kv_d = dev(kv)
    x_view = kv_d[1, :, :N].transpose(0, 1)           # [N, H, D] view, strides (D, L*D, 1)
    codes = torch.zeros((N, H, M), dtype=torch.uint8, device="cuda")
    desc = pq.PQEncodeDesc(N, H, D, M, 256, D, L * D, H * M, M, codes.numel())
    cb = dev(case["cb_init"])
    st = pq.load_library().pq_kmeans(pq.ctypes.byref(desc), x_view.data_ptr(), cb.data_ptr(), 4,
                                     codes.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    same_bits(cb.cpu().numpy(), ref_cb)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)
    perm = np.random.default_rng(1101).permutation(N)
    cb2 = dev(case["cb_init"])
    pq.pq_kmeans(dev(sample[perm]), cb2, 4)
    torch.cuda.synchronize()
    same_bits(cb2.cpu().numpy(), ref_cb)


def test_learned_codebooks_then_encode_and_decode():
    """The whole flow at a small size: learn K and V codebooks on the first 32
    tokens, encode the prefill with them into the cache, decode one token;
    every step against the oracle's."""
    B, H, L, M, N = 2, 4, 256, 4, 32
    rng = np.random.default_rng(1200)
    kc = gen.kmeans_case(rng, B * L, H, M, sigma=0.1, init_sigma=0.3, n_used=48)
    vc = gen.kmeans_case(rng, B * L, H, M, sigma=0.1, init_sigma=0.3, n_used=48)
    q = (rng.standard_normal((B, H, 128)).astype(np.float16))
    lens = np.array([L, 150], np.int32)
    assert_lloyd_margins(kc["x"][:N], kc["cb_init"], 3, oracle, "K sample")
    assert_lloyd_margins(vc["x"][:N], vc["cb_init"], 3, oracle, "V sample")
    ref_kcb, _ = oracle.kmeans(kc["x"][:N], kc["cb_init"], 3)
    ref_vcb, _ = oracle.kmeans(vc["x"][:N], vc["cb_init"], 3)
    assert_clear_margins(kc["x"], ref_kcb, "prefill K with learned codebook")
    assert_clear_margins(vc["x"], ref_vcb, "prefill V with learned codebook")
    kcb, vcb = dev(kc["cb_init"]), dev(vc["cb_init"])
    pq.pq_kmeans(dev(kc["x"][:N]), kcb, 3)
    pq.pq_kmeans(dev(vc["x"][:N]), vcb, 3)
    torch.cuda.synchronize()
    same_bits(kcb.cpu().numpy(), ref_kcb)
    same_bits(vcb.cpu().numpy(), ref_vcb)
    # prefill: token t of request b is row b*L + t of the samples
    kcodes = torch.zeros((B, H, L, M), dtype=torch.uint8, device="cuda")
    vcodes = torch.zeros((B, H, L, M), dtype=torch.uint8, device="cuda")
    slots = dev(np.concatenate([b * H * L + np.arange(L) for b in range(B)]).astype(np.int64))
    desc = pq.cache_encode_desc(B * L, B, H, L, n_sub=M)
    pq.pq_encode(dev(kc["x"]), kcb, kcodes, slots=slots, desc=desc)
    pq.pq_encode(dev(vc["x"]), vcb, vcodes, slots=slots, desc=desc)
    out = pq.pq_attn_decode(dev(q), kcodes, vcodes, kcb, vcb, dev(lens))
    torch.cuda.synchronize()
    ref_kc = oracle.encode(kc["x"], ref_kcb).reshape(B, L, H, M).transpose(0, 2, 1, 3)
    ref_vc = oracle.encode(vc["x"], ref_vcb).reshape(B, L, H, M).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(kcodes.cpu().numpy(), ref_kc)
    np.testing.assert_array_equal(vcodes.cpu().numpy(), ref_vc)
    ref = oracle.decode_attention(q, ref_kc, ref_vc, ref_kcb, ref_vcb, lens)
    got = out.cpu().numpy()
    err = np.abs(got - ref).max()
    say(f"learned-codebook decode: max|d| = {err:.3e}, max|ref| = {np.abs(ref).max():.3e}")
    assert err <= 1e-3 * np.abs(ref).max()


@pytest.mark.parametrize("N,M,n_iter", [(8192, 8, 3), (8200, 4, 2)])
def test_kmeans_at_and_past_the_one_launch_size(N, M, n_iter):
    """8192 vectors: the last size learned in one launch; 8200: the per-
    iteration launches.  Both as the oracle, bit for bit."""
    say(f"kmeans N={N} M={M} iters={n_iter}")
    case = gen.kmeans_case(np.random.default_rng(1300 + N), N, 2, M, sigma=0.05, init_sigma=0.25,
                           n_used=100)
    assert_lloyd_margins(case["x"], case["cb_init"], n_iter, oracle, "kmeans")
    ref_cb, ref_codes = oracle.kmeans(case["x"], case["cb_init"], n_iter)
    cb = dev(case["cb_init"])
    _, codes = pq.pq_kmeans(dev(case["x"]), cb, n_iter)
    torch.cuda.synchronize()
    same_bits(cb.cpu().numpy(), ref_cb)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)


def test_kmeans_many_equals_single_calls():
    """K and V samples learned in one call give what two pq_kmeans calls give,
    and the oracle's."""
    say("kmeans_many: K and V of 8 heads, 64 vectors, 4 iterations")
    rng = np.random.default_rng(1400)
    cases = [gen.kmeans_case(rng, 64, 8, 4, sigma=0.1, init_sigma=0.3) for _ in range(2)]
    xs = [dev(c["x"]) for c in cases]
    many = [dev(c["cb_init"]) for c in cases]
    _, codes = pq.pq_kmeans_many(xs, many, 4)
    single = [dev(c["cb_init"]) for c in cases]
    single_codes = [pq.pq_kmeans(x, cb, 4)[1] for x, cb in zip(xs, single)]
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        assert_lloyd_margins(c["x"], c["cb_init"], 4, oracle, f"plane {i}")
        ref_cb, ref_codes = oracle.kmeans(c["x"], c["cb_init"], 4)
        same_bits(many[i].cpu().numpy(), ref_cb)
        same_bits(single[i].cpu().numpy(), ref_cb)
        np.testing.assert_array_equal(codes[i].cpu().numpy(), ref_codes)
        np.testing.assert_array_equal(single_codes[i].cpu().numpy(), ref_codes)


def test_kmeans_one_launch_rounding_cases():
    """A Lloyd iteration inside the one-launch kernel on clusters whose means
    fall exactly between two fp16 values (normal, subnormal, large, negative)
    or at the top of the range: segment 0 of every vector is a constant
    vector near one chosen codeword; the other segments are codewords exactly,
    so every assignment is unambiguous."""
    clusters = [  # (centre, member values)
        (0.0, [2**-24, 2 * 2**-24]),            # subnormal tie -> 2^-23
        (1.0, [1.0, 1.0 + 2**-10]),             # tie -> 1.0
        (2.0, [2.0 + 2**-9, 2.0 + 2 * 2**-9]),  # tie -> 2 + 2^-8 (even)
        (100.0, [100.0, 100.0 + 2**-4]),        # tie -> 100
        (-3.0, [-3.0, -3.0 - 2**-9]),           # tie -> -3
        (65504.0, [65504.0, 65504.0]),
        (-500.0, [-500.0, -499.75, -499.5]),
    ]
    rng = np.random.default_rng(1500)
    H, M, D = 1, 4, 128
    cb0 = rng.standard_normal((H, M, 256, 32)).astype(np.float16)
    cb0[0, 0] = np.float16(20000.0) + np.arange(256, dtype=np.float16)[:, None]   # far away
    rows = []
    for i, (centre, members) in enumerate(clusters):
        cb0[0, 0, 10 + 20 * i] = centre
        rows += members
    N = len(rows)
    x = np.empty((N, H, D), np.float16)
    x[:, 0, :32] = np.array(rows, np.float16)[:, None]
    for m in range(1, M):   # exact codewords
        x[:, 0, 32 * m:32 * (m + 1)] = cb0[0, m, rng.integers(0, 256, N)]
    assert_lloyd_margins(x, cb0, 1, oracle, "rounding clusters")
    ref_cb, ref_codes = oracle.kmeans(x, cb0, 1)
    cb = dev(cb0)
    _, codes = pq.pq_kmeans(dev(x), cb, 1)
    torch.cuda.synchronize()
    got = cb.cpu().numpy()
    same_bits(got, ref_cb)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)
    assert got[0, 0, 10, 0] == 2**-23 and got[0, 0, 30, 0] == 1.0
    assert got[0, 0, 50, 0] == 2.0 + 2**-8 and got[0, 0, 70, 0] == 100.0
    assert got[0, 0, 90, 0] == -3.0 and got[0, 0, 110, 0] == 65504.0
