"""GPU parity of the request-batched score kernel (one query head per KV head
and at least 1024 (request, KV head) pairs: four requests of a KV head per
workgroup), through the C ABI against the CPU oracle.  Bar: max|gpu - oracle|
<= 1e-3 * max|oracle| over a call's output.
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
    print(f"[mha] {msg}", flush=True)
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
    say(f"{what}: max|d| = {err:.3e}, max|ref| = {scale:.3e}, ratio {err / scale:.2e}")
    assert err <= TOL * scale, f"{what}: max|d| {err:.3e} > {TOL} * {scale:.3e}"


def ragged(rng, B, L):
    lens = rng.integers(1, L + 1, B).astype(np.int32)
    lens[:6] = [0, 1, L, L - 1, 2, 0]
    return lens


MHA = [
    # (B, H, L, M, chunk): B*H >= 1024
    (66, 16, 512, 4, 0),      # a last group of two requests (second pass empty); T = 512, one chunk
    (69, 16, 1024, 4, 0),     # a last group of five requests (second pass with one)
    (64, 16, 4096, 8, 0),     # T = 2048: two chunks merged
    (64, 32, 1024, 4, 300),   # explicit chunks across thread strides
    (128, 8, 256, 8, 0),      # short caches
]


@pytest.mark.parametrize("B,H,L,M,chunk", MHA)
def test_batched_decode_matches_oracle(B, H, L, M, chunk):
    say(f"batched decode B={B} H={H} L={L} M={M} chunk={chunk}")
    rng = np.random.default_rng(2000 + B + L + M)
    _, inp = gen.random_case(2000 + B + M, batch=B, n_q_heads=H, n_kv_heads=H, max_len=L, n_sub=M,
                             lens=ragged(rng, B, L))
    t = [dev(inp[k]) for k in ATTN]
    desc = pq.attn_desc(t[0], t[1], t[3], chunk=chunk)
    out = pq.pq_attn_decode(*t, desc=desc)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.decode_attention(*(inp[k] for k in ATTN))
    assert_attn_close(got, ref, f"batched B={B} H={H} M={M}")
    assert (got[inp["lens"] == 0] == 0).all()


def test_batched_partials_match_oracle_records():
    """The chunk records themselves (m, l, o), on a sample of rows."""
    B, H, L, M, T = 64, 16, 640, 4, 256
    say(f"batched partials B={B} H={H} L={L} T={T}")
    rng = np.random.default_rng(2100)
    _, inp = gen.random_case(2100, batch=B, n_q_heads=H, n_kv_heads=H, max_len=L, n_sub=M,
                             lens=ragged(rng, B, L))
    t = [dev(inp[k]) for k in ATTN]
    pm, pl, po = pq.pq_attn_partials(*t, chunk=T)
    torch.cuda.synchronize()
    bs = [0, 1, 2, 3, 17, 63]
    sub = {k: (inp[k][bs] if k in ("q", "k_codes", "v_codes", "lens") else inp[k]) for k in ATTN}
    rm, rl, ro = oracle.chunk_partials(*(sub[k] for k in ATTN), chunk=T)
    pm, pl, po = pm.cpu().numpy()[bs], pl.cpu().numpy()[bs], po.cpu().numpy()[bs]
    empty = np.isneginf(rm)
    assert (np.isneginf(pm) == empty).all()
    np.testing.assert_allclose(pm[~empty], rm[~empty], rtol=0, atol=1e-4)
    np.testing.assert_allclose(pl[~empty], rl[~empty], rtol=2e-4, atol=0)
    assert (pl[empty] == 0).all() and (po[empty] == 0).all()
    assert_attn_close(po, ro, "batched partial o")


def test_batched_paged_decode():
    B, H, L, M, P = 64, 16, 1024, 4, 64
    say(f"batched paged decode B={B} H={H} L={L} P={P}")
    rng = np.random.default_rng(2200)
    _, inp = gen.random_case(2200, batch=B, n_q_heads=H, n_kv_heads=H, max_len=L, n_sub=M,
                             lens=ragged(rng, B, L))
    kp, vp, table, _ = gen.paged_cache(np.random.default_rng(2201), inp["k_codes"], inp["v_codes"],
                                       inp["lens"], P)
    q, kcb, vcb, lens = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"]), dev(inp["lens"])
    out = pq.pq_attn_decode_paged(q, dev(kp), dev(vp), kcb, vcb, dev(table), lens, page_tokens=P)
    dense = pq.pq_attn_decode(q, dev(inp["k_codes"]), dev(inp["v_codes"]), kcb, vcb, lens)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_paged(inp["q"], kp, vp, inp["k_cb"], inp["v_cb"], table,
                                        inp["lens"], P)
    got = out.cpu().numpy()
    assert_attn_close(got, ref, "batched paged")
    np.testing.assert_array_equal(got, dense.cpu().numpy())


def test_step_with_many_single_head_pairs():
    """The decode step on a request-batched shape (the encode kernel writes
    the new codes, then the request-batched kernel attends): codes and output
    as the oracle's, and the batched plain decode over the updated cache
    agrees."""
    B, H, L, M = 64, 16, 1024, 4
    say(f"step with many G=1 pairs B={B} H={H} L={L}")
    rng = np.random.default_rng(2300)
    _, inp = gen.random_case(2300, batch=B, n_q_heads=H, n_kv_heads=H, max_len=L, n_sub=M,
                             lens=ragged(rng, B, L))
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(2301), inp["k_cb"], inp["v_cb"], B)
    q, kcb, vcb, lens = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"]), dev(inp["lens"])
    kc, vc = dev(inp["k_codes"]), dev(inp["v_codes"])
    out = pq.pq_attn_decode_step(q, dev(xk), dev(xv), kc, vc, kcb, vcb, lens)
    again = pq.pq_attn_decode(q, kc, vc, kcb, vcb, lens)
    torch.cuda.synchronize()
    exp_k, exp_v = inp["k_codes"].copy(), inp["v_codes"].copy()
    assert_clear_margins(xk, inp["k_cb"], "new token K")
    assert_clear_margins(xv, inp["v_cb"], "new token V")
    ck, cv = oracle.encode(xk, inp["k_cb"]), oracle.encode(xv, inp["v_cb"])
    for b, l in enumerate(inp["lens"]):
        if l >= 1:
            exp_k[b, :, l - 1] = ck[b]
            exp_v[b, :, l - 1] = cv[b]
    np.testing.assert_array_equal(kc.cpu().numpy(), exp_k)
    np.testing.assert_array_equal(vc.cpu().numpy(), exp_v)
    ref = oracle.decode_attention(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], inp["lens"])
    assert_attn_close(out.cpu().numpy(), ref, "step, many G=1 pairs")
    assert_attn_close(again.cpu().numpy(), ref, "batched decode after the step")


def test_paged_step_with_many_single_head_pairs():
    """The paged decode step on a request-batched shape: the new codes land at
    the table's slot of token lens[b] - 1 and the output is the oracle's."""
    B, H, L, M, P = 64, 16, 1024, 8, 64
    say(f"paged step with many G=1 pairs B={B} H={H} L={L} M={M} P={P}")
    rng = np.random.default_rng(2400)
    _, inp = gen.random_case(2400, batch=B, n_q_heads=H, n_kv_heads=H, max_len=L, n_sub=M,
                             lens=ragged(rng, B, L))
    kp, vp, table, _ = gen.paged_cache(np.random.default_rng(2401), inp["k_codes"], inp["v_codes"],
                                       inp["lens"], P)
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(2402), inp["k_cb"], inp["v_cb"], B)
    q, kcb, vcb, lens = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"]), dev(inp["lens"])
    kp_d, vp_d, table_d = dev(kp), dev(vp), dev(table)
    desc, _ = pq.paged_desc(q, kp_d, kcb, table_d, P)
    assert pq.pq_attn_num_chunks(desc) == 1
    out = pq.pq_attn_decode_step_paged(q, dev(xk), dev(xv), kp_d, vp_d, kcb, vcb, table_d, lens,
                                       page_tokens=P)
    torch.cuda.synchronize()
    exp_k, exp_v = kp.copy(), vp.copy()
    assert_clear_margins(xk, inp["k_cb"], "new token K")
    assert_clear_margins(xv, inp["v_cb"], "new token V")
    ck, cv = oracle.encode(xk, inp["k_cb"]), oracle.encode(xv, inp["v_cb"])
    for b, l in enumerate(inp["lens"]):
        if l >= 1:
            slot = int(table[b, (l - 1) // P]) * P + (l - 1) % P
            exp_k[:, slot] = ck[b]
            exp_v[:, slot] = cv[b]
    np.testing.assert_array_equal(kp_d.cpu().numpy(), exp_k)
    np.testing.assert_array_equal(vp_d.cpu().numpy(), exp_v)
    ref = oracle.decode_attention_paged(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], table,
                                        inp["lens"], P)
    assert_attn_close(out.cpu().numpy(), ref, "paged step, many G=1 pairs")


@pytest.mark.parametrize("paged", [False, True])
def test_step_with_many_single_head_pairs_two_chunks(paged):
    """M = 8 and 4096-token caches: the batched chunk is 2048 tokens, so the
    step is the encode kernel, the batched partials and the merge; a
    workspace reused for a second step."""
    B, H, L, M, P = 64, 16, 4096, 8, 256
    say(f"step, many G=1 pairs, two chunks, paged={paged}")
    rng = np.random.default_rng(2500)
    _, inp = gen.random_case(2500, batch=B, n_q_heads=H, n_kv_heads=H, max_len=L, n_sub=M,
                             lens=ragged(rng, B, L))
    lens = inp["lens"]
    lens[6:10] = [2048, 2049, 4096, 2047]            # new tokens at the chunk edge and the end
    q, kcb, vcb, lens_d = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"]), dev(lens)
    if paged:
        kp, vp, table, _ = gen.paged_cache(np.random.default_rng(2501), inp["k_codes"],
                                           inp["v_codes"], lens, P)
        kc_d, vc_d, table_d = dev(kp), dev(vp), dev(table)
        desc, _ = pq.paged_desc(q, kc_d, kcb, table_d, P)
    else:
        kc_d, vc_d = dev(inp["k_codes"]), dev(inp["v_codes"])
        desc = pq.attn_desc(q, kc_d, kcb)
    assert pq.pq_attn_num_chunks(desc) == 2
    ws = pq.step_workspace(desc, q.device)
    exp_k = (kp if paged else inp["k_codes"]).copy()
    exp_v = (vp if paged else inp["v_codes"]).copy()
    for step in range(2):
        xk, _, xv, _ = gen.step_tokens(np.random.default_rng(2502 + step), inp["k_cb"], inp["v_cb"], B)
        if paged:
            out = pq.pq_attn_decode_step_paged(q, dev(xk), dev(xv), kc_d, vc_d, kcb, vcb, table_d,
                                               lens_d, page_tokens=P, workspace=ws)
        else:
            out = pq.pq_attn_decode_step(q, dev(xk), dev(xv), kc_d, vc_d, kcb, vcb, lens_d,
                                         desc=desc, workspace=ws)
        torch.cuda.synchronize()
        assert_clear_margins(xk, inp["k_cb"], "new token K")
        assert_clear_margins(xv, inp["v_cb"], "new token V")
        ck, cv = oracle.encode(xk, inp["k_cb"]), oracle.encode(xv, inp["v_cb"])
        for b, l in enumerate(lens):
            if l >= 1:
                if paged:
                    slot = int(table[b, (l - 1) // P]) * P + (l - 1) % P
                    exp_k[:, slot] = ck[b]
                    exp_v[:, slot] = cv[b]
                else:
                    exp_k[b, :, l - 1] = ck[b]
                    exp_v[b, :, l - 1] = cv[b]
        np.testing.assert_array_equal(kc_d.cpu().numpy(), exp_k)
        np.testing.assert_array_equal(vc_d.cpu().numpy(), exp_v)
        if paged:
            ref = oracle.decode_attention_paged(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"],
                                                table, lens, P)
        else:
            ref = oracle.decode_attention(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], lens)
        assert_attn_close(out.cpu().numpy(), ref, f"two-chunk step {step}, paged={paged}")
    rec = pq.pq_attn_workspace_bytes(desc)
    assert (ws[rec:rec + B * H * 4] == 0).all()
