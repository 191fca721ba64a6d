"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each test ties one part of the oracle to the pages' printed numbers, to an
algebraic identity computed another way, to a closed form on a tiny input,
or to a library routine (torch's CPU attention, scipy's distances).  The
cases are chosen so that a plausible slip in the oracle (a dropped scale, a
swapped subspace order, a transposed codebook, K and V mixed up, the wrong
GQA head map, a missing max in the merge) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return json.load(f)


def _small(seed=0, B=2, Hq=4, Hkv=2, L=37, M=4, D=128, lens=None):
    return gen.random_case(seed, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_len=L,
                           n_sub=M, head_dim=D, lens=lens)[1]


# --------------------------------------------------------------------------
# P1-P3: the pages' printed sizes pin the cache layout and the codebook size
# --------------------------------------------------------------------------

def test_compression_ratio_64_to_1():
    f = _facts()["compression"]
    inp = gen.workload_inputs(2, with_encode=False)
    one_vec_codes = inp["k_codes"][0, 0, 0]               # M uint8 indices
    one_vec_dense = oracle.reconstruct(inp["k_codes"][0, 0, :1], inp["k_cb"][0])
    assert one_vec_codes.nbytes == f["pq_bytes"]
    assert one_vec_dense.astype(np.float16).nbytes == f["dense_bytes"]
    assert f["dense_bytes"] // f["pq_bytes"] == f["ratio"]


def test_dense_footprint_page_sizing():
    """B=4, L=2048, H=32, D=128 fp16 K+V is 134,217,728 B per layer; the PQ
    code arrays of the same workload are 64x smaller."""
    facts = _facts()
    inp = gen.workload_inputs(2, with_encode=False)
    B, H, L, M = inp["k_codes"].shape
    w = gen.WORKLOADS[2]
    assert (B, H, L) == (facts["dense_kv_step"]["batch"], facts["dense_kv_step"]["heads"],
                         facts["dense_kv_layer"]["seq_len"])
    k_hat = oracle.reconstruct(inp["k_codes"][0, 0], inp["k_cb"][0])      # [L, D]
    assert k_hat.shape == (L, w.head_dim)
    dense_layer = 2 * B * H * k_hat.astype(np.float16).nbytes             # K and V
    assert dense_layer == facts["dense_kv_layer"]["bytes"]
    assert dense_layer // L == facts["dense_kv_step"]["bytes"]
    assert round(dense_layer * facts["dense_kv_model"]["layers"] / 1e9, 1) == \
        facts["dense_kv_model"]["printed_gb"]
    code_bytes = inp["k_codes"].nbytes + inp["v_codes"].nbytes
    assert code_bytes == dense_layer // facts["compression"]["ratio"] == 2_097_152


def test_codebook_size_64kb():
    f = _facts()["codebook"]
    inp = gen.workload_inputs(2, with_encode=False)
    assert inp["k_cb"].shape[1:] == (f["n_sub"], f["n_codes"], f["sub_dim"])
    assert inp["k_cb"][0].nbytes == f["bytes"] == f["printed_kb"] * 1024


def test_gqa_shape():
    f = _facts()["gqa"]
    w = gen.WORKLOADS[3]
    assert (w.n_q_heads, w.n_kv_heads, w.group) == (f["q_heads"], f["kv_heads"], f["q_per_kv"])


# --------------------------------------------------------------------------
# P4: lookup-table scores equal reconstruct-then-dot (AQPIM page, 4 vs 4.1)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M", [2, 4, 8])
def test_lookup_scores_equal_reconstruct_dot(M):
    inp = _small(seed=M, M=M, L=50)
    q, kc, cb = inp["q"], inp["k_codes"], inp["k_cb"]
    D = q.shape[-1]
    ds = D // M
    scale = oracle.default_scale(D)
    b, h, g = 1, 3, 1                        # h=3 reads KV head 3 // 2 = 1
    # lookup form, written out independently of the oracle
    qs = q[b, h].astype(np.float64).reshape(M, ds)
    lut = np.einsum("mj,mkj->mk", qs, cb[g].astype(np.float64))         # [M, K]
    s_lut = scale * lut[np.arange(M)[None, :], kc[b, g].astype(np.intp)].sum(axis=1)
    # the oracle's reconstruction, dotted
    s_rec = scale * oracle.reconstruct(kc[b, g], cb[g]) @ q[b, h].astype(np.float64)
    np.testing.assert_allclose(s_rec, s_lut, rtol=0, atol=1e-12)
    # and the oracle's softmax weights agree with the softmax of the lookups
    p = oracle.attention_weights(q[b, h], oracle.reconstruct(kc[b, g], cb[g]), scale)
    e = np.exp(s_lut - s_lut.max())
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# P5: softmax weights are a distribution
# --------------------------------------------------------------------------

def test_weights_sum_to_one():
    inp = _small(seed=5, L=300)
    k_hat = oracle.reconstruct(inp["k_codes"][0, 1], inp["k_cb"][1])
    for h in range(inp["q"].shape[1]):
        p = oracle.attention_weights(inp["q"][0, h], k_hat, oracle.default_scale(128))
        assert abs(p.sum() - 1.0) <= 1e-12
        assert (p > 0).all()


# --------------------------------------------------------------------------
# P6: chunk statistics merged by the reduction equal one pass (PAM page 2.2.3)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 7, 16, 2048, 61])
def test_split_merge_equals_single_pass(chunk):
    inp = _small(seed=11, L=61, lens=[61, 23])
    args = [inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")]
    ref = oracle.decode_attention(*args)
    m, l, o = oracle.chunk_partials(*args, chunk=chunk)
    got = oracle.merge_partials(m, l, o)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    # chunks wholly past lens are empty: (-inf, 0, 0)
    C = m.shape[-1]
    for c in range(C):
        if c * chunk >= 23:
            assert np.isneginf(m[1, :, c]).all() and (l[1, :, c] == 0).all() and (o[1, :, c] == 0).all()


def test_uneven_splits_merge():
    """Token ranges cut at random points (as if held by different devices)."""
    rng = np.random.default_rng(3)
    inp = _small(seed=12, B=1, L=97, lens=[97])
    args = [inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb")]
    ref = oracle.decode_attention(*args, inp["lens"])
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 97), size=4, replace=False))
        edges = [0, *cuts.tolist(), 97]
        ms, ls, os_ = [], [], []
        for a, b in zip(edges[:-1], edges[1:]):
            sub = [args[0], args[1][:, :, a:b], args[2][:, :, a:b], args[3], args[4]]
            m, l, o = oracle.chunk_partials(*sub, np.array([b - a]), chunk=b - a)
            ms.append(m), ls.append(l), os_.append(o)
        got = oracle.merge_partials(np.concatenate(ms, -1), np.concatenate(ls, -1),
                                    np.concatenate(os_, -2))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_merge_is_shift_invariant_and_needs_the_max():
    """Adding a constant to every score leaves the output unchanged; the merge
    must rescale by exp(m_c - m*) (a merge that forgets m_c fails here)."""
    rng = np.random.default_rng(0)
    m = rng.normal(size=(3, 5)) * 10
    l = rng.uniform(0.5, 2, size=(3, 5))
    o = rng.normal(size=(3, 5, 4))
    out = oracle.merge_partials(m, l, o)
    manual = np.zeros((3, 4))
    for i in range(3):
        w = np.exp(m[i] - m[i].max())
        manual[i] = (w[:, None] * o[i]).sum(0) / (w * l[i]).sum()
    np.testing.assert_allclose(out, manual, rtol=1e-13)
    # a chunk whose max is 30 above the others dominates completely
    m2 = np.array([[0.0, 30.0]])
    l2 = np.array([[1.0, 1.0]])
    o2 = np.array([[[1.0], [2.0]]])
    assert abs(oracle.merge_partials(m2, l2, o2)[0, 0] - 2.0) < 1e-12


# --------------------------------------------------------------------------
# P7: V through per-codeword probability histograms equals sum_t p_t V_t
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M", [4, 8])
def test_histogram_v_identity(M):
    inp = _small(seed=20 + M, M=M, L=80, lens=[80, 41])
    q, kc, vc, kcb, vcb, lens = (inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens"))
    out = oracle.decode_attention(q, kc, vc, kcb, vcb, lens)
    D = q.shape[-1]
    ds, K = D // M, vcb.shape[2]
    G = q.shape[1] // kcb.shape[0]
    for b in range(q.shape[0]):
        L = int(lens[b])
        for h in range(q.shape[1]):
            g = h // G
            p = oracle.attention_weights(q[b, h], oracle.reconstruct(kc[b, g, :L], kcb[g]),
                                         oracle.default_scale(D))
            hist = np.zeros((M, K))
            for m in range(M):
                np.add.at(hist[m], vc[b, g, :L, m].astype(np.intp), p)
            o = np.concatenate([hist[m] @ vcb[g, m].astype(np.float64) for m in range(M)])
            np.testing.assert_allclose(out[b, h], o, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P8: closed forms and brute force on tiny inputs
# --------------------------------------------------------------------------

def _vhat_loop(vc_row, vcb_g):
    """One V vector rebuilt by an explicit loop over subspaces."""
    M = vcb_g.shape[0]
    out = []
    for m in range(M):
        out.extend(float(x) for x in vcb_g[m, int(vc_row[m])])
    return np.array(out)


def test_single_token_returns_its_value():
    inp = _small(seed=30, L=9, lens=[1, 1])
    out = oracle.decode_attention(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")))
    for b in range(2):
        for h in range(4):
            g = h // 2
            np.testing.assert_array_equal(out[b, h], _vhat_loop(inp["v_codes"][b, g, 0], inp["v_cb"][g]))


def test_zero_query_gives_mean_of_values():
    inp = _small(seed=31, L=17)
    inp["q"][:] = 0
    out = oracle.decode_attention(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")))
    for b in range(2):
        for h in range(4):
            g = h // 2
            mean = np.mean([_vhat_loop(inp["v_codes"][b, g, t], inp["v_cb"][g]) for t in range(17)], axis=0)
            np.testing.assert_allclose(out[b, h], mean, rtol=0, atol=1e-13)


def test_equal_keys_give_mean_of_values():
    inp = _small(seed=32, L=13)
    inp["k_codes"][:] = inp["k_codes"][:, :, :1, :]   # every token has the same K
    out = oracle.decode_attention(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")))
    mean = np.mean([_vhat_loop(inp["v_codes"][0, 1, t], inp["v_cb"][1]) for t in range(13)], axis=0)
    np.testing.assert_allclose(out[0, 2], mean, rtol=0, atol=1e-13)


def test_two_tokens_sigmoid():
    inp = _small(seed=33, B=1, Hq=1, Hkv=1, L=2)
    q, kc, vc, kcb, vcb = (inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb"))
    scale = 1 / math.sqrt(128)
    s = []
    for t in range(2):
        acc = 0.0
        for m in range(4):
            for j in range(32):
                acc += float(q[0, 0, m * 32 + j]) * float(kcb[0, m, int(kc[0, 0, t, m]), j])
        s.append(scale * acc)
    p0 = 1 / (1 + math.exp(-(s[0] - s[1])))
    v0, v1 = _vhat_loop(vc[0, 0, 0], vcb[0]), _vhat_loop(vc[0, 0, 1], vcb[0])
    out = oracle.decode_attention(q, kc, vc, kcb, vcb, np.array([2]))
    np.testing.assert_allclose(out[0, 0], p0 * v0 + (1 - p0) * v1, rtol=0, atol=1e-13)


def test_brute_force_tiny_loops():
    """B=1, H=1, M=2, K=4, D=4, L<=4, written as plain loops."""
    rng = np.random.default_rng(34)
    D, M, K = 4, 2, 4
    ds = D // M
    kcb = rng.standard_normal((1, M, K, ds)).astype(np.float16)
    vcb = rng.standard_normal((1, M, K, ds)).astype(np.float16)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    for L in range(1, 5):
        kc = rng.integers(0, K, (1, 1, 4, M), dtype=np.uint8)
        vc = rng.integers(0, K, (1, 1, 4, M), dtype=np.uint8)
        scores = []
        for t in range(L):
            acc = 0.0
            for d in range(D):
                m, j = divmod(d, ds)
                acc += float(q[0, 0, d]) * float(kcb[0, m, kc[0, 0, t, m], j])
            scores.append(acc / math.sqrt(D))
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        z = sum(w)
        expect = [0.0] * D
        for t in range(L):
            for d in range(D):
                m, j = divmod(d, ds)
                expect[d] += w[t] / z * float(vcb[0, m, vc[0, 0, t, m], j])
        got = oracle.decode_attention(q, kc, vc, kcb, vcb, np.array([L]))
        np.testing.assert_allclose(got[0, 0], expect, rtol=0, atol=1e-14)


def test_tokens_past_lens_do_not_matter_and_empty_gives_zero():
    inp = _small(seed=35, L=40, lens=[17, 0])
    args = [inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")]
    ref = oracle.decode_attention(*args)
    assert (ref[1] == 0).all()
    inp["k_codes"][:, :, 17:] ^= 0x5A
    inp["v_codes"][:, :, 17:] ^= 0xA5
    again = oracle.decode_attention(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")))
    np.testing.assert_array_equal(again, ref)
    # lens beyond the capacity is clamped
    clamp = oracle.decode_attention(*args[:5], np.array([40, 0]))
    big = oracle.decode_attention(*args[:5], np.array([1000, -3]))
    np.testing.assert_array_equal(big, clamp)


def test_gqa_head_map():
    """Query head h attends KV head h // G: head 5 of 8 with 2 KV heads
    equals single-head attention over KV head 1's cache."""
    inp = _small(seed=36, B=1, Hq=8, Hkv=2, L=21)
    full = oracle.decode_attention(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")))
    one = oracle.decode_attention(inp["q"][:, 5:6], inp["k_codes"][:, 1:2], inp["v_codes"][:, 1:2],
                                  inp["k_cb"][1:2], inp["v_cb"][1:2], inp["lens"])
    np.testing.assert_array_equal(full[:, 5], one[:, 0])
    other = oracle.decode_attention(inp["q"][:, 5:6], inp["k_codes"][:, 0:1], inp["v_codes"][:, 0:1],
                                    inp["k_cb"][0:1], inp["v_cb"][0:1], inp["lens"])
    assert np.abs(full[:, 5] - other[:, 0]).max() > 1e-3


# --------------------------------------------------------------------------
# P9: special case that is dense attention -> torch's CPU SDPA in float64
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 4])
def test_identity_codes_reduce_to_dense_attention(M):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(40 + M)
    D, K, L = 128, 256, 200
    ds = D // M
    kcb = rng.standard_normal((1, M, K, ds)).astype(np.float16)
    vcb = rng.standard_normal((1, M, K, ds)).astype(np.float16)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    codes = np.repeat(np.arange(L, dtype=np.uint8)[:, None], M, axis=1)[None, None]  # codes[t, m] = t
    out = oracle.decode_attention(q, codes, codes, kcb, vcb, np.array([L]))
    # token t is row t of every codebook, segments side by side
    Kd = np.concatenate([kcb[0, m, :L] for m in range(M)], axis=1).astype(np.float64)
    Vd = np.concatenate([vcb[0, m, :L] for m in range(M)], axis=1).astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)).view(1, 1, 1, D),
        torch.from_numpy(Kd).view(1, 1, L, D), torch.from_numpy(Vd).view(1, 1, L, D))
    np.testing.assert_allclose(out[0, 0], ref.view(D).numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P10: encode = nearest codeword
# --------------------------------------------------------------------------

def _fp64_distances(x, cb):
    N, H, D = x.shape
    _, M, K, ds = cb.shape
    xs = x.astype(np.float64).reshape(N, H, M, ds)
    c = cb.astype(np.float64)
    return ((xs[:, :, :, None, :] - c[None]) ** 2).sum(-1)      # [N, H, M, K]


def test_encode_recovers_source_codes_tiny_workload():
    inp = gen.workload_inputs(1)
    for x, cb, src in ((inp["x_k"], inp["k_cb"], inp["src_k"]), (inp["x_v"], inp["v_cb"], inp["src_v"])):
        codes = oracle.encode(x, cb)
        np.testing.assert_array_equal(codes, src)
        d = np.sort(_fp64_distances(x, cb), axis=-1)
        assert (d[..., 1] - d[..., 0]).min() > 1e-4


def test_encode_matches_scipy_cdist():
    """scipy's float64 squared-Euclidean distances, argmin per row: the same
    codes on every row (both sides decide in float64; unstructured vectors,
    so some decisions are close calls)."""
    spatial = pytest.importorskip("scipy.spatial")
    rng = np.random.default_rng(50)
    H, M, K, ds = 3, 4, 256, 32
    cb = rng.standard_normal((H, M, K, ds)).astype(np.float16)
    x = rng.standard_normal((300, H, M * ds)).astype(np.float16)     # far from codewords
    codes = oracle.encode(x, cb)
    gaps = []
    for h in range(H):
        for m in range(M):
            d = spatial.distance.cdist(x[:, h, m * ds:(m + 1) * ds].astype(np.float64),
                                       cb[h, m].astype(np.float64), "sqeuclidean")
            np.testing.assert_array_equal(codes[:, h, m], d.argmin(1))
            srt = np.sort(d, axis=1)
            gaps.append((srt[:, 1] - srt[:, 0]).min())
    assert min(gaps) < 1e-1          # the case does hold close calls


def test_encode_decides_in_float64():
    """A decision that float32 distances get wrong: two codewords whose
    distances to x differ by 2^-30 (far below float32's resolution at that
    size) -- the oracle must pick the nearer one."""
    cb = np.zeros((1, 1, 4, 2), dtype=np.float16)
    x = np.zeros((1, 1, 2), dtype=np.float16)
    x[0, 0] = [np.float16(1024.0), np.float16(0.0)]
    cb[0, 0, 0] = [np.float16(0.0), np.float16(2.0 ** -15)]        # |x-c|^2 = 2^20 + 2^-30
    cb[0, 0, 1] = [np.float16(0.0), np.float16(0.0)]               # |x-c|^2 = 2^20
    cb[0, 0, 2:] = np.float16(-1000.0)
    d0 = (1024.0 ** 2) + 2.0 ** -30
    assert np.float32(d0) == np.float32(1024.0 ** 2)                # float32 would tie -> index 0
    assert oracle.encode(x, cb)[0, 0, 0] == 1


def test_encode_ties_take_lowest_index():
    rng = np.random.default_rng(51)
    cb = rng.standard_normal((1, 2, 8, 4)).astype(np.float16)
    cb[0, 0, 6] = cb[0, 0, 2]
    cb[0, 1, 7] = cb[0, 1, 5]
    x = np.concatenate([cb[0, 0, 6], cb[0, 1, 7]])[None, None, :]
    np.testing.assert_array_equal(oracle.encode(x, cb)[0, 0], [2, 5])


def test_encode_ragged_workload_sample():
    """A sample of the ragged workload's prefill vectors (sigma = 0.1)."""
    w = gen.WORKLOADS[5]
    rng = gen.rng_for(5)
    cb = gen.codebooks(rng, w.n_kv_heads, w.n_sub, w.n_codes, w.sub_dim)
    x, src = gen.noisy_codewords(rng, cb, 64, w.encode_sigma)
    np.testing.assert_array_equal(oracle.encode(x, cb), src)
    d = np.sort(_fp64_distances(x, cb), axis=-1)
    assert (d[..., 1] - d[..., 0]).min() > 1e-2


# --------------------------------------------------------------------------
# P11: the tiny workload's shapes
# --------------------------------------------------------------------------

def test_tiny_workload_shapes():
    inp = gen.workload_inputs(1)
    assert inp["q"].shape == (1, 8, 128) and inp["q"].dtype == np.float16
    assert inp["k_cb"].shape == (8, 4, 256, 32) and inp["k_cb"].dtype == np.float16
    assert inp["k_codes"].shape == (1, 8, 512, 4) and inp["k_codes"].dtype == np.uint8
    out = oracle.decode_attention(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")))
    assert out.shape == (1, 8, 128)
    assert np.isfinite(out).all()
    assert abs(oracle.default_scale(128) - 1 / math.sqrt(128)) < 1e-15


# --------------------------------------------------------------------------
# Paged code cache: the same attention with codes read through a block table
# --------------------------------------------------------------------------

_ATTN = ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")


@pytest.mark.parametrize("P", [1, 4, 16])
def test_paged_equals_dense_through_shuffled_pages(P):
    """Pages scattered in random order by the generator and read back through
    the table give exactly the dense cache's attention (ragged lens, an empty
    request, a full one)."""
    inp = _small(seed=60 + P, B=4, Hq=4, Hkv=2, L=48, lens=[48, 0, 17, 33])
    dense = oracle.decode_attention(*(inp[k] for k in _ATTN))
    kp, vp, table, _ = gen.paged_cache(np.random.default_rng(70 + P), inp["k_codes"],
                                       inp["v_codes"], inp["lens"], P)
    paged = oracle.decode_attention_paged(inp["q"], kp, vp, inp["k_cb"], inp["v_cb"],
                                          table, inp["lens"], P)
    np.testing.assert_array_equal(paged, dense)


def test_paged_tiny_loops():
    """B=1, H=1, M=2, K=4, D=4, P=2, 3 tokens in pages [3, 0] of a 4-page
    pool, written as plain loops over the pool."""
    rng = np.random.default_rng(80)
    D, M, K, P = 4, 2, 4, 2
    ds = D // M
    kcb = rng.standard_normal((1, M, K, ds)).astype(np.float16)
    vcb = rng.standard_normal((1, M, K, ds)).astype(np.float16)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    kp = rng.integers(0, K, (1, 4 * P, M), dtype=np.uint8)
    vp = rng.integers(0, K, (1, 4 * P, M), dtype=np.uint8)
    table = np.array([[3, 0, 99]], dtype=np.int32)      # third entry unused
    where = [6, 7, 0]                                    # token -> pool slot, by hand
    scores = []
    for t in range(3):
        acc = 0.0
        for d in range(D):
            m, j = divmod(d, ds)
            acc += float(q[0, 0, d]) * float(kcb[0, m, kp[0, where[t], m], j])
        scores.append(acc / math.sqrt(D))
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    expect = [0.0] * D
    for t in range(3):
        for d in range(D):
            m, j = divmod(d, ds)
            expect[d] += w[t] / sum(w) * float(vcb[0, m, vp[0, where[t], m], j])
    got = oracle.decode_attention_paged(q, kp, vp, kcb, vcb, table, np.array([3]), P)
    np.testing.assert_allclose(got[0, 0], expect, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(oracle.paged_slots(table, np.array([3]), 0, P, 6), where)


def test_paged_shared_page_and_unused_entries():
    """Two requests may name the same page (a shared prefix); entries past a
    request's last page are never read, whatever they hold."""
    inp = _small(seed=81, B=2, Hq=2, Hkv=1, L=32, lens=[20, 9])
    inp["k_codes"][1, :, :8] = inp["k_codes"][0, :, :8]   # request 1 shares request 0's first page
    inp["v_codes"][1, :, :8] = inp["v_codes"][0, :, :8]
    dense = oracle.decode_attention(*(inp[k] for k in _ATTN))
    P = 8
    kp = np.zeros((1, 5 * P, 4), np.uint8)
    vp = np.zeros((1, 5 * P, 4), np.uint8)
    table = np.array([[2, 4, 0, 2**31 - 1], [2, 1, -7, 12345]], dtype=np.int32)
    for b, pages in ((0, [2, 4, 0]), (1, [2, 1])):
        for j, page in enumerate(pages):
            kp[0, page * P:(page + 1) * P] = inp["k_codes"][b, 0, j * P:(j + 1) * P]
            vp[0, page * P:(page + 1) * P] = inp["v_codes"][b, 0, j * P:(j + 1) * P]
    paged = oracle.decode_attention_paged(inp["q"], kp, vp, inp["k_cb"], inp["v_cb"], table,
                                          inp["lens"], P)
    np.testing.assert_array_equal(paged, dense)


# --------------------------------------------------------------------------
# Codebook learning: Lloyd iterations per head and segment
# --------------------------------------------------------------------------

def test_codebook_update_by_hand():
    """H=1, M=1, D=2, K=4: means of hand-placed points, an empty codeword that
    keeps its value, and a mean that needs rounding to fp16."""
    x = np.array([[[0, 0]], [[0, 2]], [[10, 0]], [[10, 2]], [[5, 5]],
                  [[1, 1]], [[2, 2]], [[2, 2]]], dtype=np.float16)
    codes = np.array([0, 0, 1, 1, 3, 2, 2, 2], dtype=np.uint8).reshape(8, 1, 1)
    cb = np.array([[[[0, 0], [9, 9], [7, 7], [6, 6]]]], dtype=np.float16)
    new, counts = oracle.codebook_update(x[:5], codes[:5], cb)
    np.testing.assert_array_equal(new[0, 0], np.array([[0, 1], [10, 1], [7, 7], [5, 5]], np.float16))
    np.testing.assert_array_equal(counts[0, 0], [2, 2, 0, 1])
    new, counts = oracle.codebook_update(x, codes, cb)
    # (1 + 2 + 2) / 3 = 5/3 lies between fp16 neighbours 1706/1024 and 1707/1024 and nearer the second
    assert float(new[0, 0, 2, 0]) == 1 + 683 / 1024
    assert counts[0, 0, 2] == 3


def _objective(x, cb, codes):
    """Sum of squared distances of every segment to its codeword, in fp64."""
    N, H, D = x.shape
    _, M, K, ds = cb.shape
    xs = x.astype(np.float64).reshape(N, H, M, ds)
    c = cb.astype(np.float64)[np.arange(H)[None, :, None], np.arange(M)[None, None, :],
                              codes.astype(np.intp)]
    return float(((xs - c) ** 2).sum())


def test_codebook_update_matches_sklearn_lloyd():
    """One Lloyd iteration of scikit-learn's KMeans from the same start, per
    (head, segment), on data where no cluster goes empty: the same labels
    and, after rounding to fp16, centres within one fp16 step."""
    skc = pytest.importorskip("sklearn.cluster")
    rng = np.random.default_rng(90)
    case = gen.kmeans_case(rng, 480, 2, 4, n_codes=16, sigma=0.2, init_sigma=0.3)
    x, cb0 = case["x"], case["cb_init"]
    codes = oracle.encode(x, cb0)
    new, counts = oracle.codebook_update(x, codes, cb0)
    assert (counts > 0).all()
    ds = 32
    for h in range(2):
        for m in range(4):
            pts = x[:, h, m * ds:(m + 1) * ds].astype(np.float64)
            km = skc.KMeans(n_clusters=16, init=cb0[h, m].astype(np.float64), n_init=1, max_iter=1,
                            algorithm="lloyd", tol=0.0).fit(pts)
            sk_labels = np.argmin(((pts[:, None, :] - cb0[h, m].astype(np.float64)[None]) ** 2).sum(-1), 1)
            np.testing.assert_array_equal(codes[:, h, m], sk_labels)
            ref = km.cluster_centers_.astype(np.float16)
            step = np.spacing(np.abs(ref)).astype(np.float64)
            assert (np.abs(new[h, m].astype(np.float64) - ref.astype(np.float64)) <= step).all()


def test_kmeans_lowers_the_objective_and_finds_the_generating_codebook():
    rng = np.random.default_rng(91)
    case = gen.kmeans_case(rng, 2048, 2, 8, n_codes=256, sigma=0.05, init_sigma=0.25, n_used=64)
    x, cb = case["x"], case["cb_init"]
    objs = [_objective(x, cb, oracle.encode(x, cb))]
    for _ in range(4):
        cb, codes = oracle.kmeans(x, cb, 1)
        objs.append(_objective(x, cb, codes))
    # each step lowers the objective, up to fp16 rounding of the centroids
    rounding = x.shape[0] * x.shape[1] * 128 * 2e-3 * 2.0 ** -10
    assert all(b <= a + rounding for a, b in zip(objs, objs[1:]))
    assert objs[-1] < 0.5 * objs[0]
    np.testing.assert_array_equal(codes, case["src"])
    used = cb[:, :, :64].astype(np.float64)
    assert np.abs(used - case["cb_true"][:, :, :64]).max() < 0.05
    # codewords nobody chose keep their starting values
    np.testing.assert_array_equal(cb[:, :, 64:], case["cb_init"][:, :, 64:])


def test_kmeans_fixed_point_and_segment_independence():
    """Vectors that are exactly codewords are a fixed point; swapping two
    segments of the data and the codebook swaps the results."""
    rng = np.random.default_rng(92)
    case = gen.kmeans_case(rng, 300, 1, 4, n_codes=256, sigma=0.0, init_sigma=0.0, n_used=40)
    cb, codes = oracle.kmeans(case["x"], case["cb_true"], 2)
    np.testing.assert_array_equal(cb, case["cb_true"])
    np.testing.assert_array_equal(codes, case["src"])
    case = gen.kmeans_case(rng, 200, 1, 4, n_codes=256, sigma=0.1, init_sigma=0.3, n_used=30)
    a_cb, a_codes = oracle.kmeans(case["x"], case["cb_init"], 2)
    xs = case["x"].reshape(200, 1, 4, 32)[:, :, [1, 0, 2, 3]].reshape(200, 1, 128)
    b_cb, b_codes = oracle.kmeans(xs, case["cb_init"][:, [1, 0, 2, 3]], 2)
    np.testing.assert_array_equal(b_cb, a_cb[:, [1, 0, 2, 3]])
    np.testing.assert_array_equal(b_codes, a_codes[:, :, [1, 0, 2, 3]])


# --------------------------------------------------------------------------
# FP8 codebooks (AQPIM page, section 4.2: codebooks as a low-precision float
# such as FP8): the E4M3 decode and what it implies
# --------------------------------------------------------------------------

def test_fp8_e4m3_values_by_hand():
    """Bytes whose values follow from the format's fields by hand: sign,
    exponent (bias 7), mantissa, the subnormal range, the largest value and
    the NaN encoding."""
    cases = {
        0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x30: 0.5, 0x3F: 1.875,
        0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
        0x07: 7 * 2.0 ** -9, 0x04: 2.0 ** -7, 0x77: 1.875 * 2.0 ** 7, 0x78: 256.0,
    }
    b = np.array(list(cases), dtype=np.uint8)
    got = oracle.fp8_e4m3_to_float64(b)
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    neg0 = oracle.fp8_e4m3_to_float64(np.array([0x80], np.uint8))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0
    assert np.isnan(oracle.fp8_e4m3_to_float64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_fp8_e4m3_decode_matches_torch():
    """All 256 bytes against torch's own float8_e4m3fn -> float64 conversion."""
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("this torch has no float8_e4m3fn")
    b = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_e4m3_to_float64(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_fp8_values_are_fp16_values():
    """Every finite E4M3 value survives a round trip through fp16 -- the
    fact the GPU path rests on (it converts codebooks to fp16 on load)."""
    v = oracle.fp8_e4m3_to_float64(np.arange(256, dtype=np.uint8))
    v = v[~np.isnan(v)]
    np.testing.assert_array_equal(v.astype(np.float16).astype(np.float64), v)


def test_fp8_codebook_is_half_the_page_size():
    """At M=4, K=256, 32 dims an FP8 codebook set is 32 KB, half of the
    page's 64 KB fp16 figure."""
    f = _facts()["codebook"]
    cb8 = gen.codebooks_fp8(np.random.default_rng(60), 2, f["n_sub"], f["n_codes"], f["sub_dim"])
    assert cb8.dtype == np.uint8 and cb8[0].nbytes * 2 == f["bytes"] == 65536


def test_fp8_generator_rounds_to_nearest():
    """The generator's bytes decode to the E4M3 value nearest the drawn
    normal (checked against all 254 finite values)."""
    rng = np.random.default_rng(61)
    cb8 = gen.codebooks_fp8(rng, 1, 1, 256, 8)
    x = np.random.default_rng(61).standard_normal((1, 1, 256, 8), dtype=np.float32).astype(np.float64)
    table = oracle.fp8_e4m3_to_float64(np.arange(256, dtype=np.uint8))
    finite = table[~np.isnan(table)]
    got = oracle.fp8_e4m3_to_float64(cb8)
    best = np.abs(x[..., None] - finite).min(axis=-1)
    np.testing.assert_array_equal(np.abs(x - got), best)
