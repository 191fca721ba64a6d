"""GPU parity for the paged code cache: the HIP library through its C ABI
against the CPU oracle's paged attention.

Bars as for the dense cache: codes bit-exact; attention within
max|gpu - oracle| <= 1e-3 * max|oracle| over a call's output.  Pages are
scattered in a seeded random order with spare pages of random codes, and the
table entries past each request's pages hold -1, so a kernel that reads the
wrong page, slot or table entry gives a wrong answer.  The paged kernels do
the dense kernels' arithmetic in the same order, so the paged output also
equals the dense library call on the same logical cache bit for bit.
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
ATTN = ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")


def say(msg):
    print(f"[paged] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pq.load_library()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def assert_attn_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all()
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    if scale == 0:
        assert err == 0, what
        return
    say(f"{what}: max|d| = {err:.3e}, max|ref| = {scale:.3e}, ratio {err / scale:.2e}")
    assert err <= TOL * scale, f"{what}: max|d| {err:.3e} > {TOL} * {scale:.3e}"


def token_slots(table, lens, P):
    """(b, t, slot) of every token below lens, from the table (test side)."""
    b_of = np.repeat(np.arange(len(lens)), lens)
    t_of = np.concatenate([np.arange(l) for l in lens]) if len(lens) else np.zeros(0, int)
    return b_of, t_of, table[b_of, t_of // P].astype(np.int64) * P + t_of % P


PAGED_EDGE = [
    # (G, M, P, Lmax, chunk, lens)
    (1, 4, 16, 64, 0, [0, 1, 63, 64]),
    (2, 4, 16, 272, 16, [15, 16, 17, 0]),          # one page per chunk
    (4, 8, 64, 528 + 48, 256, [255, 256, 257, 576]),  # pages straddle chunks
    (8, 8, 256, 2048, 1024, [1023, 1024, 1025, 1]),
    (8, 4, 1024, 4096, 0, [4096, 3000, 1, 2]),
    (1, 8, 4096, 8192, 2048, [8192, 4097, 4096, 0]),  # a page longer than a chunk
    (2, 4, 512, 17408, 1024, [17408, 1, 1024, 1025, 0, 16385, 2048, 9000]),  # two chunks per workgroup
    (4, 4, 32, 4096, 4096, [4096, 4095, 2049, 33]),   # several token slots per thread
]


@pytest.mark.parametrize("G,M,P,Lmax,chunk,lens", PAGED_EDGE)
def test_paged_edge_shapes(G, M, P, Lmax, chunk, lens):
    say(f"paged edge G={G} M={M} P={P} Lmax={Lmax} chunk={chunk} lens={lens}")
    Hkv = 2
    _, inp = gen.random_case(400 + G * 10 + M, batch=len(lens), n_q_heads=G * Hkv,
                             n_kv_heads=Hkv, max_len=Lmax, n_sub=M, lens=lens)
    kp, vp, table, _ = gen.paged_cache(np.random.default_rng(500 + P), inp["k_codes"],
                                       inp["v_codes"], inp["lens"], P)
    q, kcb, vcb, lens_d = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"]), dev(inp["lens"])
    out = pq.pq_attn_decode_paged(q, dev(kp), dev(vp), kcb, vcb, dev(table), lens_d,
                                  page_tokens=P, chunk=chunk)
    dense = pq.pq_attn_decode(q, dev(inp["k_codes"]), dev(inp["v_codes"]), kcb, vcb, lens_d,
                              chunk=chunk)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = oracle.decode_attention_paged(inp["q"], kp, vp, inp["k_cb"], inp["v_cb"], table,
                                        inp["lens"], P)
    assert_attn_close(out, ref, f"paged edge G={G} M={M} P={P}")
    np.testing.assert_array_equal(out, dense.cpu().numpy())
    for b, l in enumerate(lens):
        if l == 0:
            assert (out[b] == 0).all()


def test_paged_ragged_prefill_then_decode():
    """The ragged workload on a paged cache: the prefill's K and V are encoded
    straight into shuffled 256-token pages through pool slots, then one decode
    over the pages.  The pool holds exactly the generator's source codes at
    the tokens' slots and its earlier random codes everywhere else."""
    P = 256
    say(f"paged ragged: 64 requests (45x512 + 19x4096), H=32, M=4, pages of {P}")
    w = gen.WORKLOADS[5]
    inp = gen.workload_inputs(5)
    B, H, L, M = w.batch, w.n_kv_heads, w.max_len, w.n_sub
    lens = inp["lens"]
    kp, vp, table, n_pages = gen.paged_cache(np.random.default_rng(5256), inp["k_codes"],
                                             inp["v_codes"], lens, P)
    b_of, t_of, slot = token_slots(table, lens, P)
    # the generator's prefill rows are ordered by request, then token: its
    # dense-cache slots b*H*L + t say so
    np.testing.assert_array_equal(inp["slots"], b_of * H * L + t_of)
    N = int(lens.sum())
    kp_d, vp_d = dev(kp), dev(vp)
    desc = pq.paged_encode_desc(N, H, n_pages, P, n_sub=M)
    slots = dev(slot)
    pq.pq_encode(dev(inp["x_k"]), dev(inp["k_cb"]), kp_d, slots=slots, desc=desc)
    pq.pq_encode(dev(inp["x_v"]), dev(inp["v_cb"]), vp_d, slots=slots, desc=desc)
    torch.cuda.synchronize()
    exp_k, exp_v = kp.copy(), vp.copy()
    exp_k[:, slot] = inp["src_k"].transpose(1, 0, 2)
    exp_v[:, slot] = inp["src_v"].transpose(1, 0, 2)
    np.testing.assert_array_equal(kp_d.cpu().numpy(), exp_k)
    np.testing.assert_array_equal(vp_d.cpu().numpy(), exp_v)
    say("paged ragged: decode over the pages")
    out = pq.pq_attn_decode_paged(dev(inp["q"]), kp_d, vp_d, dev(inp["k_cb"]), dev(inp["v_cb"]),
                                  dev(table), dev(lens), page_tokens=P)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_paged(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], table,
                                        lens, P)
    assert_attn_close(out.cpu().numpy(), ref, "paged ragged decode")


def step_paged_expected(inp, kp, vp, table, lens, P, xk, xv):
    """Pools after the new token's codes (oracle encode) land at the slot of
    token lens[b] - 1, and the oracle's paged attention over them."""
    exp_k, exp_v = kp.copy(), vp.copy()
    assert_clear_margins(xk, inp["k_cb"], "new token K")
    assert_clear_margins(xv, inp["v_cb"], "new token V")
    ck, cv = oracle.encode(xk, inp["k_cb"]), oracle.encode(xv, inp["v_cb"])
    for b, l in enumerate(lens):
        if l >= 1:
            s = int(table[b, (l - 1) // P]) * P + (l - 1) % P
            exp_k[:, s] = ck[b]
            exp_v[:, s] = cv[b]
    ref = oracle.decode_attention_paged(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], table,
                                        lens, P)
    return exp_k, exp_v, ref


def run_step_paged(inp, kp, vp, table, lens, P, xk, xv, chunk=0, ws=None):
    q, kcb, vcb = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"])
    kp_d, vp_d, table_d = dev(kp), dev(vp), dev(table)
    desc, _ = pq.paged_desc(q, kp_d, kcb, table_d, P, chunk=chunk)
    if ws is None:
        ws = pq.step_workspace(desc, q.device)
    out = pq.pq_attn_decode_step_paged(q, dev(xk), dev(xv), kp_d, vp_d, kcb, vcb, table_d,
                                       dev(np.asarray(lens, np.int32)), page_tokens=P,
                                       chunk=chunk, workspace=ws)
    torch.cuda.synchronize()
    return desc, ws, kp_d.cpu().numpy(), vp_d.cpu().numpy(), out.cpu().numpy()


STEP_PAGED = [
    # (G, M, P, Lmax, chunk, lens): the new token at a page's first slot, its
    # last slot, a chunk edge, the cache's last slot, and lens 0
    (8, 8, 64, 1024, 256, [65, 64, 256, 1024]),
    (1, 4, 16, 512, 0, [1, 0, 17, 512]),
    (4, 8, 256, 4096, 1024, [257, 1024, 1025, 4096]),
    (2, 4, 4096, 8192, 2048, [4097, 4096, 2048, 1]),
    # more than 8 chunks per (request, KV head): the spread merge
    (8, 4, 64, 2048, 128, [1, 2048, 700, 0]),
    (2, 8, 32, 1536, 64, [1536, 65, 33, 0]),
    # 8 requests x 2 KV heads x 17 chunks of 1024 > 256: two chunks per
    # workgroup, the last workgroup of each (request, KV head) with one
    (4, 4, 256, 17408, 1024, [17408, 1, 1024, 1025, 0, 16385, 2048, 9000]),
]


@pytest.mark.parametrize("G,M,P,Lmax,chunk,lens", STEP_PAGED)
def test_paged_step(G, M, P, Lmax, chunk, lens):
    say(f"paged step G={G} M={M} P={P} Lmax={Lmax} chunk={chunk} lens={lens}")
    Hkv = 2
    B = len(lens)
    _, inp = gen.random_case(600 + G * 10 + M, batch=B, n_q_heads=G * Hkv, n_kv_heads=Hkv,
                             max_len=Lmax, n_sub=M, lens=lens)
    lens = np.asarray(lens, np.int32)
    kp, vp, table, _ = gen.paged_cache(np.random.default_rng(700 + P), inp["k_codes"],
                                       inp["v_codes"], lens, P)
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(800 + G), inp["k_cb"], inp["v_cb"], B)
    desc, ws, kp_g, vp_g, out = run_step_paged(inp, kp, vp, table, lens, P, xk, xv, chunk=chunk)
    exp_k, exp_v, ref = step_paged_expected(inp, kp, vp, table, lens, P, xk, xv)
    np.testing.assert_array_equal(kp_g, exp_k)
    np.testing.assert_array_equal(vp_g, exp_v)
    assert_attn_close(out, ref, f"paged step G={G} M={M} P={P}")
    if ws is not None:
        rec = pq.pq_attn_workspace_bytes(desc)
        assert (ws[rec:rec + desc.batch * desc.n_kv_heads * 4] == 0).all()


@pytest.mark.parametrize("chunk", [0, 2048])
def test_paged_step_gqa_workload(chunk):
    """The benchmarked step shape (B=8, Hq=64, Hkv=8, L=8192, M=8) on 256-token
    pages: codes and output as the oracle's, output equal to the dense step's
    (the library's head split, and four merged chunks)."""
    P = 256
    say(f"paged step on the gqa workload, pages of {P}, chunk {chunk or 'library'}")
    inp = gen.workload_inputs(3, with_encode=False)
    lens = inp["lens"]
    kp, vp, table, _ = gen.paged_cache(np.random.default_rng(3256), inp["k_codes"],
                                       inp["v_codes"], lens, P)
    xk, sk, xv, sv = gen.step_tokens(np.random.default_rng(3001), inp["k_cb"], inp["v_cb"], 8)
    desc, ws, kp_g, vp_g, out = run_step_paged(inp, kp, vp, table, lens, P, xk, xv, chunk=chunk)
    assert pq.pq_attn_num_chunks(desc) == (1 if chunk == 0 else 4)
    exp_k, exp_v, ref = step_paged_expected(inp, kp, vp, table, lens, P, xk, xv)
    np.testing.assert_array_equal(kp_g, exp_k)
    np.testing.assert_array_equal(vp_g, exp_v)
    assert_attn_close(out, ref, "paged gqa step")
    # the dense step on the same logical cache
    q, kcb, vcb = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"])
    kc, vc = dev(inp["k_codes"]), dev(inp["v_codes"])
    dense = pq.pq_attn_decode_step(q, dev(xk), dev(xv), kc, vc, kcb, vcb, dev(lens), chunk=chunk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out, dense.cpu().numpy())


def test_paged_page_range_shards_merge_like_one_call():
    """A page-range split: two calls over tables that each name half of every
    request's pages (the other half's entries point at a spare page whose
    tokens are cut off by lens), records merged with pq_attn_reduce, equal the
    oracle's attention over the whole cache."""
    B, H, L, M, P = 4, 8, 1024, 4, 128
    say("paged page-range shards")
    _, inp = gen.random_case(3000, batch=B, n_q_heads=2 * H, n_kv_heads=H, max_len=L, n_sub=M,
                             lens=[1024, 700, 513, 129])
    kp, vp, table, _ = gen.paged_cache(np.random.default_rng(3001), inp["k_codes"], inp["v_codes"],
                                       inp["lens"], P)
    lens = inp["lens"]
    half = L // 2                                   # shard 0: tokens [0, 512); shard 1: [512, 1024)
    q, kcb, vcb = (dev(inp[k]) for k in ("q", "k_cb", "v_cb"))
    kp_d, vp_d = dev(kp), dev(vp)
    # shard 0: the first half of every table row, lens cut at 512
    t0 = np.ascontiguousarray(table[:, : half // P])
    l0 = np.minimum(lens, half).astype(np.int32)
    # shard 1: the second half, tokens renumbered from 0
    t1 = np.ascontiguousarray(table[:, half // P:])
    l1 = np.maximum(lens - half, 0).astype(np.int32)
    recs = []
    for t, l in ((t0, l0), (t1, l1)):
        recs.append(pq.pq_attn_partials_paged(q, kp_d, vp_d, kcb, vcb, dev(t), dev(l),
                                              page_tokens=P, chunk=256))
    pm = torch.cat([r[0] for r in recs], dim=2).contiguous()
    pl = torch.cat([r[1] for r in recs], dim=2).contiguous()
    po = torch.cat([r[2] for r in recs], dim=2).contiguous()
    out = pq.pq_attn_reduce(pm, pl, po)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_paged(inp["q"], kp, vp, inp["k_cb"], inp["v_cb"], table, lens, P)
    assert_attn_close(out.cpu().numpy(), ref, "paged page-range shards")
