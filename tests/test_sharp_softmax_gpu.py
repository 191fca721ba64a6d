"""GPU parity on sharp softmax distributions: one "sink" token 12-16 nats
above every other token of its (request, KV head), the others sharing one K
code row so their scores are equal.  The chunked softmax (PAM page, section
2.2.3 (1)) and its rescaling merge (memory-wall chapter, section 1.4.3 (5.1))
must hold for any score distribution; here the chunk's mass is ~1 while the
other tokens' weights are ~1e-6 each, the case a fixed-point histogram scaled
by the chunk's capacity instead of its mass gets wrong.

Cases: the per-request kernel at G = 8 with M = 4 and M = 8 (one chunk of
4096 tokens, and two of 2048 merged), the decode step, the paged cache, and
the request-batched kernel at 4096-token chunks.  Bar: max|gpu - oracle| <=
2e-4 * max|oracle| over the call's output (five times tighter than the
general 1e-3).
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

TOL_SHARP = 2e-4
ATTN = ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")


def say(msg):
    print(f"[sharp] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pq.load_library()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def assert_sharp_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all()
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    say(f"{what}: max|d| = {err:.3e}, max|ref| = {scale:.3e}, ratio {err / scale:.2e}")
    assert err <= TOL_SHARP * scale, f"{what}: max|d| {err:.3e} > {TOL_SHARP} * {scale:.3e}"


def sink_inputs(seed, B, Hq, Hkv, L, M, lens):
    """Random inputs, then per (request, KV head): every valid token's K codes
    set to one row c0, one token (random position) to another row c*, and each
    query head of the group pointed along K*^ - K0^ so that the sink leads by
    12..16 nats (spread over the group's heads).  V codes stay random."""
    _, inp = gen.random_case(seed, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_len=L, n_sub=M,
                             lens=lens)
    rng = np.random.default_rng(seed + 1)
    G = Hq // Hkv
    D = 128
    scale = oracle.default_scale(D)
    kc = inp["k_codes"]
    q = np.zeros((B, Hq, D), np.float16)
    leads = []
    for b in range(B):
        n = int(lens[b])
        for g in range(Hkv):
            c0 = rng.integers(0, 256, M).astype(np.uint8)
            cs = rng.integers(0, 256, M).astype(np.uint8)
            if n > 0:
                kc[b, g, :n] = c0
                kc[b, g, int(rng.integers(0, n))] = cs
            k0 = oracle.reconstruct(c0[None], inp["k_cb"][g])[0]
            ks = oracle.reconstruct(cs[None], inp["k_cb"][g])[0]
            d = ks - k0
            for j in range(G):
                lead = 12.0 + 4.0 * j / max(1, G - 1)
                qv = (lead / (scale * float(d @ d))) * d
                q[b, g * G + j] = qv.astype(np.float16)
                leads.append(scale * float(q[b, g * G + j].astype(np.float64) @ d))
    inp["q"] = q
    inp["k_codes"] = kc
    leads = np.array(leads)
    assert leads.min() > 11.5 and leads.max() < 16.5
    return inp


@pytest.mark.parametrize("M,chunk", [(4, 4096), (8, 4096), (4, 2048), (8, 2048)])
def test_sink_dense_g8(M, chunk):
    B, Hq, Hkv, L = 3, 16, 2, 4096
    lens = np.array([4096, 4000, 2500], np.int32)
    say(f"dense sink G=8 M={M} chunk={chunk} lens={lens.tolist()}")
    inp = sink_inputs(7000 + M + chunk, B, Hq, Hkv, L, M, lens)
    t = [dev(inp[k]) for k in ATTN]
    out = pq.pq_attn_decode(*t, chunk=chunk)
    torch.cuda.synchronize()
    assert_sharp_close(out.cpu().numpy(), oracle.decode_attention(*(inp[k] for k in ATTN)),
                       f"dense M={M} chunk={chunk}")


def test_sink_decode_step_g8():
    B, Hq, Hkv, L, M = 2, 16, 2, 4096, 8
    lens = np.array([4096, 3001], np.int32)
    say("decode step on sink inputs, G=8 M=8, chunk 2048")
    inp = sink_inputs(7100, B, Hq, Hkv, L, M, lens)
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(7101), inp["k_cb"], inp["v_cb"], B)
    assert_clear_margins(xk, inp["k_cb"], "new token K")
    assert_clear_margins(xv, inp["v_cb"], "new token V")
    q, kcb, vcb = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"])
    kc, vc = dev(inp["k_codes"]), dev(inp["v_codes"])
    desc = pq.attn_desc(q, kc, kcb, chunk=2048)
    ws = pq.step_workspace(desc, q.device)
    out = pq.pq_attn_decode_step(q, dev(xk), dev(xv), kc, vc, kcb, vcb, dev(lens), desc=desc,
                                 workspace=ws)
    torch.cuda.synchronize()
    exp_k, exp_v = inp["k_codes"].copy(), inp["v_codes"].copy()
    ck, cv = oracle.encode(xk, inp["k_cb"]), oracle.encode(xv, inp["v_cb"])
    for b, l in enumerate(lens):
        exp_k[b, :, l - 1] = ck[b]
        exp_v[b, :, l - 1] = cv[b]
    np.testing.assert_array_equal(kc.cpu().numpy(), exp_k)
    np.testing.assert_array_equal(vc.cpu().numpy(), exp_v)
    ref = oracle.decode_attention(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], lens)
    assert_sharp_close(out.cpu().numpy(), ref, "step M=8")


def test_sink_paged_g8():
    B, Hq, Hkv, L, M, P = 3, 16, 2, 4096, 8, 256
    lens = np.array([4096, 1000, 3333], np.int32)
    say("paged sink G=8 M=8, 256-token pages, chunk 4096")
    inp = sink_inputs(7200, B, Hq, Hkv, L, M, lens)
    kp, vp, table, n_pages = gen.paged_cache(np.random.default_rng(7201), inp["k_codes"],
                                             inp["v_codes"], lens, P)
    out = pq.pq_attn_decode_paged(dev(inp["q"]), dev(kp), dev(vp), dev(inp["k_cb"]),
                                  dev(inp["v_cb"]), dev(table), dev(lens), page_tokens=P,
                                  chunk=4096)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_paged(inp["q"], kp, vp, inp["k_cb"], inp["v_cb"], table, lens, P)
    assert_sharp_close(out.cpu().numpy(), ref, "paged M=8")


def test_sink_request_batched_t4096():
    """One query head per KV head and 1024 (request, head) pairs: the
    request-batched kernel, whose chunk is 4096 tokens at M = 4."""
    B, H, L, M = 64, 16, 4096, 4
    rng = np.random.default_rng(7300)
    lens = rng.integers(3000, L + 1, B).astype(np.int32)
    lens[:3] = [L, 1, 4095]
    say(f"request-batched sink B={B} H={H} L={L} M={M}")
    inp = sink_inputs(7301, B, H, H, L, M, lens)
    t = [dev(inp[k]) for k in ATTN]
    desc = pq.attn_desc(t[0], t[1], t[3])
    assert pq.pq_attn_num_chunks(desc) == 1
    out = pq.pq_attn_decode(*t, desc=desc)
    torch.cuda.synchronize()
    assert_sharp_close(out.cpu().numpy(), oracle.decode_attention(*(inp[k] for k in ATTN)),
                       "request-batched M=4 T=4096")
