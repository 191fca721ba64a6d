"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Bars: encode codes bit-exact; attention outputs within
max|gpu - oracle| <= 1e-3 * max|oracle| over the whole output tensor of a call.
Every input comes from the seeded generators; no expected value comes from
the GPU.
"""
import sys

import numpy as np
import pytest

import oracle
from margins import assert_clear_margins
from synth import gen

torch = pytest.importorskip("torch")
pq = pytest.importorskip("decode_attention_product_amd")

pytestmark = pytest.mark.gpu

TOL = 1e-3


def say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pq.load_library()       # raises if the library is missing: no silent fallback


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_inputs(inp):
    return [dev(inp[k]) for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")]


def oracle_out(inp, **kw):
    return oracle.decode_attention(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")), **kw)


def assert_attn_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    if scale == 0:
        assert err == 0, f"{what}: expected zeros, max |got| = {err}"
        return
    say(f"{what}: max|d| = {err:.3e}, max|ref| = {scale:.3e}, ratio {err / scale:.2e}")
    assert err <= TOL * scale, f"{what}: max|d| {err:.3e} > {TOL} * {scale:.3e}"


def decode_gpu(inp, chunk=0):
    t = gpu_inputs(inp)
    out = pq.pq_attn_decode(*t, chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

def test_tiny_workload_decode_and_encode():
    say("workload tiny: decode B=1 H=8 L=512 M=4; encode 8 heads x (K, V)")
    inp = gen.workload_inputs(1)
    assert_attn_close(decode_gpu(inp), oracle_out(inp), "tiny decode")
    for x, cb, src in ((inp["x_k"], inp["k_cb"], inp["src_k"]), (inp["x_v"], inp["v_cb"], inp["src_v"])):
        assert_clear_margins(x, cb, "tiny encode")
        codes = torch.empty((x.shape[0], x.shape[1], cb.shape[1]), dtype=torch.uint8, device="cuda")
        pq.pq_encode(dev(x), dev(cb), codes)
        torch.cuda.synchronize()
        got = codes.cpu().numpy()
        np.testing.assert_array_equal(got, oracle.encode(x, cb))
        np.testing.assert_array_equal(got, src)


def test_page_sizing_workload():
    say("workload page-sizing: B=4 H=32 L=2048 M=4")
    inp = gen.workload_inputs(2, with_encode=False)
    assert_attn_close(decode_gpu(inp), oracle_out(inp), "page-sizing decode")


def test_gqa_workload():
    say("workload gqa: B=8 Hq=64 Hkv=8 L=8192 M=8 (library-picked chunks, as benchmarked)")
    inp = gen.workload_inputs(3, with_encode=False)
    assert_attn_close(decode_gpu(inp), oracle_out(inp), "gqa decode")


def test_long_context_workload():
    say("workload long-splitk: B=1 Hq=64 Hkv=8 L=131072 M=4 T=2048")
    inp = gen.workload_inputs(4, with_encode=False)
    w = gen.WORKLOADS[4]
    t = gpu_inputs(inp)
    desc = pq.attn_desc(t[0], t[1], t[3], chunk=w.chunk)
    assert pq.pq_attn_num_chunks(desc) == 64
    out = pq.pq_attn_decode(*t, desc=desc)
    torch.cuda.synchronize()
    ref = oracle_out(inp)
    assert_attn_close(out.cpu().numpy(), ref, "long-splitk decode")
    # the 64 chunk records themselves, on a sample of query heads
    pm, pl, po = pq.pq_attn_partials(*t, desc=desc)
    torch.cuda.synchronize()
    rm, rl, ro = oracle.chunk_partials(inp["q"][:, :2], inp["k_codes"][:, :1], inp["v_codes"][:, :1],
                                       inp["k_cb"][:1], inp["v_cb"][:1], inp["lens"], chunk=w.chunk)
    np.testing.assert_allclose(pm.cpu().numpy()[:, :2], rm, rtol=0, atol=1e-4)
    np.testing.assert_allclose(pl.cpu().numpy()[:, :2], rl, rtol=2e-4, atol=0)
    assert_attn_close(po.cpu().numpy()[:, :2], ro, "long-splitk partial o (heads 0-1)")


def test_ragged_workload_encode_then_decode():
    """Prefill: encode every prefill token's K and V straight into the code
    cache, then one decode step over the ragged cache."""
    say("workload ragged: 64 requests (45x512 + 19x4096), H=32, prefill encode of 6,455,296 vectors")
    w = gen.WORKLOADS[5]
    inp = gen.workload_inputs(5)
    B, H, L, M = w.batch, w.n_kv_heads, w.max_len, w.n_sub
    lens = inp["lens"]
    slots = dev(inp["slots"])
    N = int(lens.sum())
    kc = dev(inp["k_codes"])           # padding positions keep their random codes
    vc = dev(inp["v_codes"])
    desc = pq.cache_encode_desc(N, B, H, L, n_sub=M)
    pq.pq_encode(dev(inp["x_k"]), dev(inp["k_cb"]), kc, slots=slots, desc=desc)
    pq.pq_encode(dev(inp["x_v"]), dev(inp["v_cb"]), vc, slots=slots, desc=desc)
    torch.cuda.synchronize()
    kc_h, vc_h = kc.cpu().numpy(), vc.cpu().numpy()
    # expected cache: generator's source indices at the prefill places,
    # the original random codes elsewhere
    exp_k, exp_v = inp["k_codes"].copy(), inp["v_codes"].copy()
    b_of = np.repeat(np.arange(B), lens)
    t_of = np.concatenate([np.arange(l) for l in lens])
    exp_k[b_of, :, t_of] = inp["src_k"]
    exp_v[b_of, :, t_of] = inp["src_v"]
    np.testing.assert_array_equal(kc_h, exp_k)
    np.testing.assert_array_equal(vc_h, exp_v)
    # and the oracle's own encode agrees on a sample of vectors
    rng = np.random.default_rng(7)
    idx = np.sort(rng.choice(N, size=3000, replace=False))
    assert_clear_margins(inp["x_k"][idx], inp["k_cb"], "ragged encode sample (K)")
    assert_clear_margins(inp["x_v"][idx], inp["v_cb"], "ragged encode sample (V)")
    np.testing.assert_array_equal(oracle.encode(inp["x_k"][idx], inp["k_cb"]), kc_h[b_of[idx], :, t_of[idx]])
    np.testing.assert_array_equal(oracle.encode(inp["x_v"][idx], inp["v_cb"]), vc_h[b_of[idx], :, t_of[idx]])
    say("ragged: decode over the encoded cache")
    out = pq.pq_attn_decode(dev(inp["q"]), kc, vc, dev(inp["k_cb"]), dev(inp["v_cb"]), dev(lens))
    torch.cuda.synchronize()
    ref = oracle.decode_attention(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], lens)
    assert_attn_close(out.cpu().numpy(), ref, "ragged decode")


# --------------------------------------------------------------------------
# Edge cases: ragged lengths around chunk edges, every group size, both M
# --------------------------------------------------------------------------

EDGE = [
    # (G, M, Lmax, chunk, lens)
    (1, 4, 64, 0, [0, 1, 63, 64]),
    (2, 4, 272, 16, [15, 16, 17, 0]),
    (4, 8, 528, 256, [255, 256, 257, 528]),
    (8, 8, 1040, 1024, [1023, 1024, 1025, 1]),
    (8, 4, 2048, 7, [7, 6, 8, 2000]),
    (1, 8, 4096, 0, [4096, 3000, 1, 2]),
    (4, 4, 1536, 1536, [1536, 1535, 0, 700]),
    (8, 8, 4096, 4096, [4096, 4095, 2049, 1]),     # more than one pass per chunk
]


@pytest.mark.parametrize("G,M,Lmax,chunk,lens", EDGE)
def test_edge_shapes(G, M, Lmax, chunk, lens):
    say(f"edge G={G} M={M} Lmax={Lmax} chunk={chunk} lens={lens}")
    Hkv = 2
    _, inp = gen.random_case(100 + G * 10 + M, batch=len(lens), n_q_heads=G * Hkv,
                             n_kv_heads=Hkv, max_len=Lmax, n_sub=M, lens=lens)
    t = gpu_inputs(inp)
    out = pq.pq_attn_decode(*t, chunk=chunk)
    torch.cuda.synchronize()
    ref = oracle_out(inp)
    assert_attn_close(out.cpu().numpy(), ref, f"edge G={G} M={M}")
    for b, l in enumerate(lens):
        if l == 0:
            assert (out[b] == 0).all()


@pytest.mark.parametrize("chunk", [16, 100, 256])
def test_partials_match_oracle(chunk):
    say(f"partials chunk={chunk}")
    _, inp = gen.random_case(200 + chunk, batch=2, n_q_heads=8, n_kv_heads=2, max_len=512,
                             n_sub=4, lens=[512, 130])
    t = gpu_inputs(inp)
    pm, pl, po = pq.pq_attn_partials(*t, chunk=chunk)
    torch.cuda.synchronize()
    rm, rl, ro = oracle.chunk_partials(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")),
                                       chunk=chunk)
    pm, pl, po = pm.cpu().numpy(), pl.cpu().numpy(), po.cpu().numpy()
    empty = np.isneginf(rm)
    assert (np.isneginf(pm) == empty).all()
    assert (pl[empty] == 0).all() and (po[empty] == 0).all()
    np.testing.assert_allclose(pm[~empty], rm[~empty], rtol=0, atol=1e-4)
    np.testing.assert_allclose(pl[~empty], rl[~empty], rtol=2e-4, atol=0)
    assert_attn_close(po, ro, f"partial o chunk={chunk}")


def test_reduce_matches_oracle_merge():
    say("reduce on random statistics")
    rng = np.random.default_rng(9)
    rows, C, D = 37, 11, 128
    m = rng.normal(size=(rows, C)).astype(np.float32) * 5
    l = rng.uniform(0.5, 3, size=(rows, C)).astype(np.float32)
    o = rng.normal(size=(rows, C, D)).astype(np.float32)
    m[3, :] = -np.inf
    l[3, :] = 0
    o[3] = 0
    m[5, 2:] = -np.inf
    l[5, 2:] = 0
    o[5, 2:] = 0
    out = pq.pq_attn_reduce(dev(m), dev(l), dev(o))
    torch.cuda.synchronize()
    ref = oracle.merge_partials(m, l, o)
    assert (out[3] == 0).all()
    assert_attn_close(out.cpu().numpy(), ref, "reduce")


def test_token_shards_merge_like_one_call():
    """Token-parallel split (PAM page, section 2.2.3 (2)) emulated on one GPU:
    each shard of the token range is its own cache; their chunk statistics,
    laid side by side, merge to the single-call result."""
    say("token shards -> partials -> reduce")
    B, Hq, Hkv, L, M = 3, 16, 2, 1024, 4
    _, inp = gen.random_case(300, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_len=L, n_sub=M,
                             lens=[1024, 700, 333])
    ref = oracle_out(inp)
    full = decode_gpu(inp)
    cuts = [0, 256, 512 + 64, 1024]
    ms, ls, os_ = [], [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sh_lens = np.clip(inp["lens"] - a, 0, b - a).astype(np.int32)
        t = [dev(inp["q"]), dev(inp["k_codes"][:, :, a:b]), dev(inp["v_codes"][:, :, a:b]),
             dev(inp["k_cb"]), dev(inp["v_cb"]), dev(sh_lens)]
        pm, pl, po = pq.pq_attn_partials(*t, chunk=128)
        ms.append(pm), ls.append(pl), os_.append(po)
    out = pq.pq_attn_reduce(torch.cat(ms, -1).contiguous(), torch.cat(ls, -1).contiguous(),
                            torch.cat(os_, -2).contiguous())
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), ref, "shards vs oracle")
    assert_attn_close(out.cpu().numpy(), full, "shards vs one call")


# --------------------------------------------------------------------------
# Robustness
# --------------------------------------------------------------------------

def test_tokens_past_lens_are_not_read():
    say("codes past lens changed on the device")
    _, inp = gen.random_case(400, batch=2, n_q_heads=4, n_kv_heads=1, max_len=1024, n_sub=4,
                             lens=[600, 17])
    t = gpu_inputs(inp)
    a = pq.pq_attn_decode(*t).clone()
    t[1][0, :, 600:] ^= 0x33          # request 0 attends 600 tokens
    t[2][0, :, 600:] ^= 0x5C
    t[1][1, :, 17:] ^= 0x11           # request 1 attends 17
    t[2][1, :, 17:] ^= 0xC3
    b = pq.pq_attn_decode(*t)
    torch.cuda.synchronize()
    assert_attn_close(b.cpu().numpy(), oracle_out(inp), "after changing padding")
    assert_attn_close(a.cpu().numpy(), b.cpu().numpy().astype(np.float64), "before vs after")


def test_repeat_and_two_streams():
    say("repeated calls on two streams")
    inp = gen.workload_inputs(2, with_encode=False)
    t = gpu_inputs(inp)
    ref = oracle_out(inp)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for i in range(6):
        s = s1 if i % 2 == 0 else s2
        with torch.cuda.stream(s):
            outs.append(pq.pq_attn_decode(*t, stream=s))
    torch.cuda.synchronize()
    for o in outs:
        assert_attn_close(o.cpu().numpy(), ref, "repeat")


def test_lens_clamped_and_empty_batch_rows():
    say("lens beyond capacity and negative")
    _, inp = gen.random_case(500, batch=3, n_q_heads=8, n_kv_heads=4, max_len=256, n_sub=8,
                             lens=[256, 0, 100])
    ref = oracle_out(inp)
    inp2 = dict(inp)
    inp2["lens"] = np.array([100000, -5, 100], dtype=np.int32)
    got = decode_gpu(inp2)
    assert_attn_close(got, ref, "clamped lens")
    assert (got[1] == 0).all()


def test_encode_strided_slots_and_out_of_range():
    say("encode through slots into a cache; out-of-range slots skipped")
    rng = np.random.default_rng(600)
    B, H, L, M = 3, 4, 64, 8
    cb = gen.codebooks(rng, H, M, 256, 128 // M)
    x, src = gen.noisy_codewords(rng, cb, 10, 0.05)
    assert_clear_margins(x, cb, "slot encode")
    cache = np.full((B, H, L, M), 0xEE, dtype=np.uint8)
    slots = np.array([0, 5, 63, 64 * 4 + 1, 2 * H * L + 7, 2 * H * L + 8, 2 * H * L + 63,
                      -1, B * H * L, 1 << 40], dtype=np.int64)
    c = dev(cache)
    desc = pq.cache_encode_desc(10, B, H, L, n_sub=M)
    pq.pq_encode(dev(x), dev(cb), c, slots=dev(slots), desc=desc)
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    exp = cache.copy()
    for n, s in enumerate(slots[:7]):
        b, t = divmod(int(s), H * L)
        exp[b, :, t] = src[n]
    # slot B*H*L - ... : only in-buffer places are written
    np.testing.assert_array_equal(got, exp)
    np.testing.assert_array_equal(oracle.encode(x, cb), src)


def test_encode_ties_lowest_index():
    say("encode ties")
    rng = np.random.default_rng(601)
    cb = gen.codebooks(rng, 2, 4, 256, 32)
    cb[1, 2, 200] = cb[1, 2, 17]
    cb[0, 0, 255] = cb[0, 0, 3]
    x = np.zeros((2, 2, 128), dtype=np.float16)
    x[0, 1, 64:96] = cb[1, 2, 17]
    x[1, 0, 0:32] = cb[0, 0, 3]
    built_tie = np.zeros((2, 2, 4), dtype=bool)
    built_tie[0, 1, 2] = built_tie[1, 0, 0] = True
    assert_clear_margins(x, cb, "encode ties (other segments)", mask=~built_tie)
    codes = torch.empty((2, 2, 4), dtype=torch.uint8, device="cuda")
    pq.pq_encode(dev(x), dev(cb), codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    assert got[0, 1, 2] == 17 and got[1, 0, 0] == 3
    np.testing.assert_array_equal(got, oracle.encode(x, cb))


def test_encode_zero_score_ties_lowest_index():
    """Zero codewords against a zero segment all score exactly 0 (as -0 or +0,
    however the sums round; the segment of vector 1 is negative zeros); the
    lowest of them must win whether the others sit in the same lane, in
    another lane or in the other half of the codebook."""
    say("encode zero-score ties")
    rng = np.random.default_rng(602)
    cb = gen.codebooks(rng, 1, 4, 256, 32)
    for m, ks in {0: (21, 5, 200), 1: (200, 77), 2: (250, 44, 40)}.items():
        cb[0, m, list(ks)] = 0
    x, _ = gen.noisy_codewords(rng, cb, 3, 0.05)
    x[0, 0, :96] = 0
    x[1, 0, 32:64] = np.float16(-0.0)
    built_tie = np.zeros((3, 1, 4), dtype=bool)
    built_tie[0, 0, :3] = built_tie[1, 0, 1] = True
    assert_clear_margins(x, cb, "encode zero ties (other segments)", mask=~built_tie)
    codes = torch.empty((3, 1, 4), dtype=torch.uint8, device="cuda")
    pq.pq_encode(dev(x), dev(cb), codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    assert list(got[0, 0, :3]) == [5, 77, 40] and got[1, 0, 1] == 77
    np.testing.assert_array_equal(got, oracle.encode(x, cb))


def test_encode_many_matches_single_calls():
    """K and V of a batch of new tokens in one launch (pq_encode_many) give
    exactly what two pq_encode calls give, into a cache through slots."""
    say("encode_many: K and V planes in one launch")
    rng = np.random.default_rng(602)
    B, H, L, M = 4, 8, 64, 8
    kcb = gen.codebooks(rng, H, M, 256, 128 // M)
    vcb = gen.codebooks(rng, H, M, 256, 128 // M)
    xk, srck = gen.noisy_codewords(rng, kcb, B, 0.05)
    xv, srcv = gen.noisy_codewords(rng, vcb, B, 0.05)
    assert_clear_margins(xk, kcb, "encode_many K")
    assert_clear_margins(xv, vcb, "encode_many V")
    slots = np.arange(B, dtype=np.int64) * H * L + np.array([0, 5, 63, 17])
    kc1, vc1 = dev(np.zeros((B, H, L, M), np.uint8)), dev(np.zeros((B, H, L, M), np.uint8))
    kc2, vc2 = dev(np.zeros((B, H, L, M), np.uint8)), dev(np.zeros((B, H, L, M), np.uint8))
    desc = pq.cache_encode_desc(B, B, H, L, n_sub=M)
    s = dev(slots)
    pq.pq_encode_many([dev(xk), dev(xv)], [dev(kcb), dev(vcb)], [kc1, vc1], slots=s, desc=desc)
    pq.pq_encode(dev(xk), dev(kcb), kc2, slots=s, desc=desc)
    pq.pq_encode(dev(xv), dev(vcb), vc2, slots=s, desc=desc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kc1.cpu().numpy(), kc2.cpu().numpy())
    np.testing.assert_array_equal(vc1.cpu().numpy(), vc2.cpu().numpy())
    got_k = kc1.cpu().numpy()[np.arange(B), :, slots % L]
    np.testing.assert_array_equal(got_k, oracle.encode(xk, kcb))
    np.testing.assert_array_equal(got_k, srck)
    np.testing.assert_array_equal(vc1.cpu().numpy()[np.arange(B), :, slots % L], srcv)


# --------------------------------------------------------------------------
# Decode step with the new token appended (one launch: encode + attend + merge)
# --------------------------------------------------------------------------

def step_expected(inp, xk, xv, lens):
    """The cache after appending the new token at slot lens[b] - 1 (codes from
    the oracle's encode) and the oracle's attention over it."""
    exp_k, exp_v = inp["k_codes"].copy(), inp["v_codes"].copy()
    assert_clear_margins(xk, inp["k_cb"], "new token K")
    assert_clear_margins(xv, inp["v_cb"], "new token V")
    ck, cv = oracle.encode(xk, inp["k_cb"]), oracle.encode(xv, inp["v_cb"])
    L = exp_k.shape[2]
    for b, l in enumerate(lens):
        l = min(max(int(l), 0), L)
        if l >= 1:
            exp_k[b, :, l - 1] = ck[b]
            exp_v[b, :, l - 1] = cv[b]
    ref = oracle.decode_attention(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], lens)
    return exp_k, exp_v, ref


def run_step(inp, xk, xv, lens, chunk=0, ws=None):
    q, kcb, vcb = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"])
    kc, vc = dev(inp["k_codes"]), dev(inp["v_codes"])
    desc = pq.attn_desc(q, kc, kcb, chunk=chunk)
    if ws is None:
        ws = pq.step_workspace(desc, q.device)
    out = pq.pq_attn_decode_step(q, dev(xk), dev(xv), kc, vc, kcb, vcb, dev(np.asarray(lens, np.int32)),
                                 desc=desc, workspace=ws)
    torch.cuda.synchronize()
    return desc, ws, kc.cpu().numpy(), vc.cpu().numpy(), out.cpu().numpy()


def check_counters_zero(desc, ws):
    if ws is None:
        return
    rec = pq.pq_attn_workspace_bytes(desc)
    n = pq.pq_attn_step_workspace_bytes(desc) - rec     # every counter (and padding)
    assert n >= desc.batch * desc.n_kv_heads * 4
    assert (ws[rec:rec + n] == 0).all(), "arrival counters not left at zero"


@pytest.mark.parametrize("chunk", [0, 2048])
def test_step_gqa_workload(chunk):
    """The library's choice (the query heads of a KV head split over four
    workgroups of two, one chunk each: no merge) and the token split into
    four chunks of 2048 merged in the launch."""
    say(f"step on the gqa workload (B=8 Hq=64 Hkv=8 L=8192 M=8, chunk {chunk or 'library'})")
    inp = gen.workload_inputs(3, with_encode=False)
    xk, sk, xv, sv = gen.step_tokens(np.random.default_rng(3001), inp["k_cb"], inp["v_cb"], 8)
    lens = inp["lens"]
    desc, ws, kc, vc, out = run_step(inp, xk, xv, lens, chunk=chunk)
    assert pq.pq_attn_num_chunks(desc) == (1 if chunk == 0 else 4)
    exp_k, exp_v, ref = step_expected(inp, xk, xv, lens)
    np.testing.assert_array_equal(kc, exp_k)
    np.testing.assert_array_equal(vc, exp_v)
    np.testing.assert_array_equal(kc[np.arange(8), :, lens - 1], sk)
    assert_attn_close(out, ref, "gqa step")
    check_counters_zero(desc, ws)


HEAD_SPLIT = [
    # (G, M, B, Hkv, L, lens, C): shapes the library splits by query heads
    # (G/2 workgroups of two per (request, KV head)), with one chunk or, with
    # one request, several (records and the in-launch merge per head part)
    (8, 8, 8, 8, 8192, [8192, 1, 0, 8191, 4096, 1025, 7000, 2], 1),
    (8, 4, 32, 2, 4096, None, 1),
    (4, 8, 16, 8, 2048, None, 1),
    (4, 4, 24, 8, 8192, None, 1),
    (8, 8, 1, 8, 8192, [8192], 8),
    (8, 4, 1, 8, 8192, [5001], 8),
]


@pytest.mark.parametrize("G,M,B,Hkv,L,lens,C", HEAD_SPLIT)
def test_head_split_decode_and_step(G, M, B, Hkv, L, lens, C):
    rng = np.random.default_rng(3950 + G + M + B)
    if lens is None:
        lens = rng.integers(0, L + 1, B)
        lens[:3] = [L, 1, 0]
    lens = np.asarray(lens, np.int32)
    say(f"head split G={G} M={M} B={B} Hkv={Hkv} L={L}")
    _, inp = gen.random_case(3960 + G * M + B, batch=B, n_q_heads=G * Hkv, n_kv_heads=Hkv,
                             max_len=L, n_sub=M, lens=lens)
    t = gpu_inputs(inp)
    desc = pq.attn_desc(t[0], t[1], t[3])
    assert pq.pq_attn_num_chunks(desc) == C
    assert (pq.pq_attn_workspace_bytes(desc) == 0) == (C == 1)
    out = pq.pq_attn_decode(*t, desc=desc)
    pm, pl, po = pq.pq_attn_partials(*t, desc=desc)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), oracle_out(inp), f"head split decode G={G} M={M}")
    rm, rl, ro = oracle.chunk_partials(*(inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")),
                                       chunk=-(-L // C))
    empty = np.isneginf(rm)
    assert (np.isneginf(pm.cpu().numpy()) == empty).all()
    np.testing.assert_allclose(pm.cpu().numpy()[~empty], rm[~empty], rtol=0, atol=1e-4)
    np.testing.assert_allclose(pl.cpu().numpy()[~empty], rl[~empty], rtol=2e-4, atol=0)
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(3970 + G + M), inp["k_cb"], inp["v_cb"], B)
    d2, ws, kc, vc, out2 = run_step(inp, xk, xv, lens)
    exp_k, exp_v, ref = step_expected(inp, xk, xv, lens)
    np.testing.assert_array_equal(kc, exp_k)
    np.testing.assert_array_equal(vc, exp_v)
    assert_attn_close(out2, ref, f"head split step G={G} M={M}")
    for b, l in enumerate(lens):
        if l == 0:
            assert (out2[b] == 0).all()
    check_counters_zero(d2, ws)


def test_step_long_context_workload():
    say("step on the long-context workload (B=1 Hq=64 Hkv=8 L=131072 M=4, 64 chunks merged in the launch)")
    w = gen.WORKLOADS[4]
    inp = gen.workload_inputs(4, with_encode=False)
    xk, sk, xv, sv = gen.step_tokens(np.random.default_rng(3002), inp["k_cb"], inp["v_cb"], 1)
    lens = inp["lens"]
    desc, ws, kc, vc, out = run_step(inp, xk, xv, lens, chunk=w.chunk)
    assert pq.pq_attn_num_chunks(desc) == 64
    exp_k, exp_v, ref = step_expected(inp, xk, xv, lens)
    np.testing.assert_array_equal(kc[0, :, lens[0] - 1], exp_k[0, :, lens[0] - 1])
    np.testing.assert_array_equal(vc[0, :, lens[0] - 1], exp_v[0, :, lens[0] - 1])
    np.testing.assert_array_equal(kc[0, :, lens[0] - 1], sk[0])
    assert_attn_close(out, ref, "long-context step")
    check_counters_zero(desc, ws)


def test_step_matches_encode_then_decode():
    """The fused step gives the codes of pq_encode_many and the output of
    pq_attn_decode over the same cache."""
    say("step vs encode_many + decode (tiny and page-sizing shapes)")
    for wid, chunk in ((1, 0), (2, 256)):
        inp = gen.workload_inputs(wid, with_encode=False)
        B, Hkv, L, M = inp["k_codes"].shape
        xk, _, xv, _ = gen.step_tokens(np.random.default_rng(3100 + wid), inp["k_cb"], inp["v_cb"], B)
        lens = np.minimum(inp["lens"], L - 3)
        desc, ws, kc, vc, out = run_step(inp, xk, xv, lens, chunk=chunk)
        kc2, vc2 = dev(inp["k_codes"]), dev(inp["v_codes"])
        edesc = pq.cache_encode_desc(B, B, Hkv, L, n_sub=M)
        slots = dev(np.arange(B, dtype=np.int64) * Hkv * L + (lens.astype(np.int64) - 1))
        pq.pq_encode_many([dev(xk), dev(xv)], [dev(inp["k_cb"]), dev(inp["v_cb"])], [kc2, vc2],
                          slots=slots, desc=edesc)
        out2 = pq.pq_attn_decode(dev(inp["q"]), kc2, vc2, dev(inp["k_cb"]), dev(inp["v_cb"]),
                                 dev(lens), chunk=chunk)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(kc, kc2.cpu().numpy())
        np.testing.assert_array_equal(vc, vc2.cpu().numpy())
        _, _, ref = step_expected(inp, xk, xv, lens)
        assert_attn_close(out, ref, f"step wid={wid}")
        assert_attn_close(out, out2.cpu().numpy().astype(np.float64), f"step vs two calls wid={wid}")
        check_counters_zero(desc, ws)


STEP_EDGE = [
    # (G, M, Lmax, chunk, lens): the new token at chunk starts and ends, empty requests
    (8, 8, 4096, 1024, [1, 1024, 1025, 4096]),
    (8, 4, 3072, 1024, [0, 2048, 2049, 3000]),
    (4, 8, 2048, 512, [512, 513, 0, 7]),
    (2, 4, 1024, 256, [256, 1, 1024, 300]),
    (1, 8, 512, 0, [512, 1, 0, 255]),
    (1, 4, 4096, 2048, [4096, 2048, 2049, 0]),
    # more than 8 chunks: the merging workgroup's spread record loads
    (8, 4, 4096, 128, [1, 4096, 2049, 0]),
    (4, 8, 2048, 64, [100, 2048, 1, 1500]),
    (2, 8, 1536, 128, [1536, 129, 0, 700]),
    (1, 4, 2048, 128, [2048, 1, 1000, 0]),
    (1, 4, 4096, 1024, [4096, 1, 3000, 0]),   # partial tiles fill the whole table region
]


@pytest.mark.parametrize("G,M,Lmax,chunk,lens", STEP_EDGE)
def test_step_edges(G, M, Lmax, chunk, lens):
    say(f"step edge G={G} M={M} Lmax={Lmax} chunk={chunk} lens={lens}")
    Hkv = 2
    _, inp = gen.random_case(3200 + G * 10 + M, batch=len(lens), n_q_heads=G * Hkv,
                             n_kv_heads=Hkv, max_len=Lmax, n_sub=M, lens=lens)
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(3300 + G + M), inp["k_cb"], inp["v_cb"],
                                   len(lens))
    lens = np.asarray(lens, np.int32)
    desc, ws, kc, vc, out = run_step(inp, xk, xv, lens, chunk=chunk)
    exp_k, exp_v, ref = step_expected(inp, xk, xv, lens)
    np.testing.assert_array_equal(kc, exp_k)
    np.testing.assert_array_equal(vc, exp_v)
    assert_attn_close(out, ref, f"step edge G={G} M={M}")
    for b, l in enumerate(lens):
        if l == 0:
            assert (out[b] == 0).all()
    check_counters_zero(desc, ws)


TWO_CHUNK = [
    # (G, Hkv, B, chunk, C, lens): M = 4 and more chunks than CUs, so each
    # workgroup owns two chunks; C odd leaves the last workgroup one chunk.
    # lens: full, one token, mid, empty, a workgroup's first chunk full and
    # its second empty, one token in a second chunk, one token in the lone
    # last chunk.
    (2, 4, 8, 1024, 9, [9216, 1, 5000, 0, 1024, 1025, 2049, 8193]),
    (8, 8, 2, 2048, 17, [34816, 2049]),
]


@pytest.mark.parametrize("G,Hkv,B,chunk,C,lens", TWO_CHUNK)
def test_two_chunks_per_workgroup(G, Hkv, B, chunk, C, lens):
    """Chunk records from workgroups that own two chunks each: the plain
    decode (records + merge launch), the records themselves, and the decode
    step (merge in the launch), against the oracle."""
    say(f"two chunks per workgroup G={G} Hkv={Hkv} B={B} chunk={chunk} C={C} lens={lens}")
    _, inp = gen.random_case(3600 + G, batch=B, n_q_heads=G * Hkv, n_kv_heads=Hkv,
                             max_len=chunk * C, n_sub=4, lens=lens)
    t = gpu_inputs(inp)
    desc = pq.attn_desc(t[0], t[1], t[3], chunk=chunk)
    assert pq.pq_attn_num_chunks(desc) == C
    out = pq.pq_attn_decode(*t, desc=desc)
    pm, pl, po = pq.pq_attn_partials(*t, desc=desc)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), oracle_out(inp), "two-chunk decode")
    rm, rl, ro = oracle.chunk_partials(inp["q"], inp["k_codes"], inp["v_codes"], inp["k_cb"],
                                       inp["v_cb"], inp["lens"], chunk=chunk)
    np.testing.assert_allclose(pm.cpu().numpy(), rm, rtol=0, atol=1e-4)
    np.testing.assert_allclose(pl.cpu().numpy(), rl, rtol=2e-4, atol=0)
    assert_attn_close(po.cpu().numpy(), ro, "two-chunk partial o")
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(3700 + G), inp["k_cb"], inp["v_cb"], B)
    lens = np.asarray(lens, np.int32)
    desc2, ws, kc, vc, out2 = run_step(inp, xk, xv, lens, chunk=chunk)
    exp_k, exp_v, ref = step_expected(inp, xk, xv, lens)
    np.testing.assert_array_equal(kc, exp_k)
    np.testing.assert_array_equal(vc, exp_v)
    assert_attn_close(out2, ref, "two-chunk step")
    for b, l in enumerate(lens):
        if l == 0:
            assert (out2[b] == 0).all()
    check_counters_zero(desc2, ws)


def test_step_twice_reuses_workspace():
    """Two consecutive steps through one workspace: the second appends after
    the first and sees both new tokens."""
    say("two steps, one workspace")
    B, Hq, Hkv, L, M = 3, 16, 2, 2048, 8
    _, inp = gen.random_case(3400, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_len=L, n_sub=M,
                             lens=[1000, 2047, 3])
    rng = np.random.default_rng(3401)
    xk1, _, xv1, _ = gen.step_tokens(rng, inp["k_cb"], inp["v_cb"], B)
    xk2, _, xv2, _ = gen.step_tokens(rng, inp["k_cb"], inp["v_cb"], B)
    lens1 = inp["lens"].astype(np.int32)
    lens2 = lens1 + 1
    q, kcb, vcb = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"])
    kc, vc = dev(inp["k_codes"]), dev(inp["v_codes"])
    desc = pq.attn_desc(q, kc, kcb, chunk=512)
    ws = pq.step_workspace(desc, q.device)
    pq.pq_attn_decode_step(q, dev(xk1), dev(xv1), kc, vc, kcb, vcb, dev(lens1), desc=desc, workspace=ws)
    out = pq.pq_attn_decode_step(q, dev(xk2), dev(xv2), kc, vc, kcb, vcb, dev(lens2), desc=desc,
                                 workspace=ws)
    torch.cuda.synchronize()
    exp_k1, exp_v1, _ = step_expected(inp, xk1, xv1, lens1)
    inp2 = dict(inp, k_codes=exp_k1, v_codes=exp_v1)
    exp_k, exp_v, ref = step_expected(inp2, xk2, xv2, lens2)
    np.testing.assert_array_equal(kc.cpu().numpy(), exp_k)
    np.testing.assert_array_equal(vc.cpu().numpy(), exp_v)
    assert_attn_close(out.cpu().numpy(), ref, "second step")
    check_counters_zero(desc, ws)


def test_step_codes_equal_pq_encode_on_unstructured_vectors():
    """The step kernel's in-kernel encode and pq_encode take the same
    decisions even without generated margins: N(0, 1) vectors, whose nearest
    codewords can be close calls, encoded both ways."""
    say("step encode vs pq_encode on N(0,1) vectors (no margins)")
    B, Hq, Hkv, L = 64, 64, 8, 256
    for M in (4, 8):
        _, inp = gen.random_case(3500 + M, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_len=L,
                                 n_sub=M, lens=[L] * B)
        rng = np.random.default_rng(3600 + M)
        xk = rng.standard_normal((B, Hkv, 128), dtype=np.float32).astype(np.float16)
        xv = rng.standard_normal((B, Hkv, 128), dtype=np.float32).astype(np.float16)
        lens = np.full(B, L, np.int32)
        _, _, kc, vc, _ = run_step(inp, xk, xv, lens, chunk=128)
        ek = torch.empty((B, Hkv, M), dtype=torch.uint8, device="cuda")
        ev = torch.empty((B, Hkv, M), dtype=torch.uint8, device="cuda")
        pq.pq_encode(dev(xk), dev(inp["k_cb"]), ek)
        pq.pq_encode(dev(xv), dev(inp["v_cb"]), ev)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(kc[:, :, L - 1], ek.cpu().numpy())
        np.testing.assert_array_equal(vc[:, :, L - 1], ev.cpu().numpy())


def test_step_shape_changes_between_steps():
    """Steps of two shapes interleaved, each with the workspace made for its
    descriptor (the binding refuses the other's): every step matches the
    oracle and leaves its counters at zero."""
    say("steps of two shapes, interleaved, one workspace each")
    cases = []
    for seed, B, L, lens in ((3800, 2, 2048, [2048, 1500]), (3801, 4, 4096, [4096, 1, 3000, 2049])):
        _, inp = gen.random_case(seed, batch=B, n_q_heads=16, n_kv_heads=2, max_len=L, n_sub=8,
                                 lens=lens)
        q, kcb = dev(inp["q"]), dev(inp["k_cb"])
        desc = pq.attn_desc(q, dev(inp["k_codes"]), kcb, chunk=512)
        cases.append((inp, np.asarray(lens, np.int32), desc, pq.step_workspace(desc, q.device)))
    with pytest.raises(ValueError):
        inp, lens, desc, _ = cases[0]
        run_step(inp, *gen.step_tokens(np.random.default_rng(1), inp["k_cb"], inp["v_cb"],
                                       len(lens))[::2], lens, chunk=512, ws=cases[1][3])
    for rnd in range(2):
        for i, (inp, lens, desc, ws) in enumerate(cases):
            xk, _, xv, _ = gen.step_tokens(np.random.default_rng(3900 + 10 * rnd + i), inp["k_cb"],
                                           inp["v_cb"], len(lens))
            d, _, kc, vc, out = run_step(inp, xk, xv, lens, chunk=512, ws=ws)
            exp_k, exp_v, ref = step_expected(inp, xk, xv, lens)
            np.testing.assert_array_equal(kc, exp_k)
            assert_attn_close(out, ref, f"shape {i} round {rnd}")
            check_counters_zero(d, ws)


def test_reduce_polyexp_matches_oracle_merge():
    """The merge with the reduction unit's polynomial exponential (PAM page,
    section 3.2.2 (1)): against the oracle's exact merge, and within ~1e-6
    of the hardware-exponential merge; empty rows and chunks, and statistics
    spread over ~100 nats (weights far below 2^-126 count as zero)."""
    say("reduce with the polynomial exp")
    rng = np.random.default_rng(19)
    rows, C, D = 53, 37, 128
    m = (rng.normal(size=(rows, C)) * 8).astype(np.float32)
    m[7] = np.linspace(0, -100, C).astype(np.float32)
    l = rng.uniform(0.5, 3, size=(rows, C)).astype(np.float32)
    o = rng.normal(size=(rows, C, D)).astype(np.float32)
    m[3, :] = -np.inf
    l[3, :] = 0
    o[3] = 0
    m[5, 2:] = -np.inf
    l[5, 2:] = 0
    o[5, 2:] = 0
    t = (dev(m), dev(l), dev(o))
    got = pq.pq_attn_reduce(*t, polyexp=True)
    hw = pq.pq_attn_reduce(*t)
    torch.cuda.synchronize()
    ref = oracle.merge_partials(m, l, o)
    assert (got[3] == 0).all()
    assert_attn_close(got.cpu().numpy(), ref, "reduce polyexp vs oracle")
    d = np.abs(got.cpu().numpy() - hw.cpu().numpy()).max() / np.abs(ref).max()
    say(f"polyexp vs hardware exp merge: {d:.2e} of max|out|")
    assert d <= 1e-6
