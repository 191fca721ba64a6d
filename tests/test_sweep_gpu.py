"""GPU parity over a seeded sweep of shapes: the dense and paged decode and
decode step, through the C ABI, against the CPU oracle.

The fixed edge-case lists elsewhere pin chosen boundaries with two KV heads;
this sweep draws the rest of the shape space instead: KV head counts that are
not powers of two, every group size, both segment counts, lengths anywhere in
[0, Lmax] (with 0, 1 and Lmax over-represented), library-chosen and explicit
chunks, and page sizes from 16 to 256 tokens.  The library's planner picks
the kernel (head split, chunks per workgroup, the request-batched kernel), so
the sweep also covers its choices.  Bars as in the other parity tests: codes
bit-exact, outputs within 1e-3 * max|oracle|.
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
PATHS = ("decode", "step", "paged", "paged_step")


def say(msg):
    print(f"[sweep] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    pq.load_library()       # raises if the library is missing: no silent fallback


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def draw_case(i):
    """Shape of sweep case i (seeded; the path cycles through PATHS)."""
    rng = np.random.default_rng(9100 + i)
    path = PATHS[i % len(PATHS)]
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 5, 8, 16, 32]))
    M = int(rng.choice([4, 8]))
    B = int(rng.integers(1, 7))
    P = 0
    if path.startswith("paged"):
        P = int(rng.choice([16, 64, 256]))
        Lmax = P * int(rng.integers(1, max(2, 3072 // P) + 1))
    else:
        Lmax = 16 * int(rng.integers(1, 193))
    lens = []
    for _ in range(B):
        kind = rng.integers(0, 6)
        lens.append(0 if kind == 0 else 1 if kind == 1 else Lmax if kind == 2 else int(rng.integers(1, Lmax + 1)))
    chunk = int(rng.choice([0, 0, 64, 256, 1024, 16 * int(rng.integers(1, Lmax // 16 + 1))]))
    return dict(path=path, G=G, Hkv=Hkv, M=M, B=B, Lmax=Lmax, P=P, lens=lens, chunk=chunk, seed=9200 + i)


CASES = [draw_case(i) for i in range(96)]


def build_expected(c):
    """Inputs and the oracle's results for a case: (inp, pools, table, xk, xv,
    expected caches or pools, expected output)."""
    _, inp = gen.random_case(c["seed"], batch=c["B"], n_q_heads=c["G"] * c["Hkv"],
                             n_kv_heads=c["Hkv"], max_len=c["Lmax"], n_sub=c["M"], lens=c["lens"])
    lens = np.asarray(c["lens"], np.int32)
    rng = np.random.default_rng(c["seed"] + 1)
    kp = vp = table = None
    if c["P"]:
        kp, vp, table, _ = gen.paged_cache(rng, inp["k_codes"], inp["v_codes"], lens, c["P"])
    xk = xv = None
    exp_k, exp_v = (kp, vp) if c["P"] else (inp["k_codes"], inp["v_codes"])
    exp_k, exp_v = exp_k.copy(), exp_v.copy()
    if c["path"].endswith("step"):
        xk, _, xv, _ = gen.step_tokens(rng, inp["k_cb"], inp["v_cb"], c["B"])
        assert_clear_margins(xk, inp["k_cb"], "new token K")
        assert_clear_margins(xv, inp["v_cb"], "new token V")
        ck, cv = oracle.encode(xk, inp["k_cb"]), oracle.encode(xv, inp["v_cb"])
        for b, l in enumerate(lens):
            if l < 1:
                continue
            if c["P"]:
                s = int(table[b, (l - 1) // c["P"]]) * c["P"] + (l - 1) % c["P"]
                exp_k[:, s], exp_v[:, s] = ck[b], cv[b]
            else:
                exp_k[b, :, l - 1], exp_v[b, :, l - 1] = ck[b], cv[b]
    if c["P"]:
        ref = oracle.decode_attention_paged(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], table,
                                            lens, c["P"])
    else:
        ref = oracle.decode_attention(inp["q"], exp_k, exp_v, inp["k_cb"], inp["v_cb"], lens)
    return inp, kp, vp, table, xk, xv, exp_k, exp_v, ref


def assert_attn_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all(), what
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    if scale == 0:
        assert err == 0, f"{what}: expected zeros"
        return
    say(f"{what}: max|d| = {err:.3e}, ratio {err / scale:.2e}")
    assert err <= TOL * scale, f"{what}: max|d| {err:.3e} > {TOL} * {scale:.3e}"


@pytest.mark.parametrize("i", range(len(CASES)))
def test_sweep(i):
    c = CASES[i]
    say(f"case {i}: {c}")
    inp, kp, vp, table, xk, xv, exp_k, exp_v, ref = build_expected(c)
    lens = dev(np.asarray(c["lens"], np.int32))
    q, kcb, vcb = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"])
    if c["P"]:
        k_d, v_d, table_d = dev(kp), dev(vp), dev(table)
    else:
        k_d, v_d = dev(inp["k_codes"]), dev(inp["v_codes"])
    if c["path"] == "decode":
        out = pq.pq_attn_decode(q, k_d, v_d, kcb, vcb, lens, chunk=c["chunk"])
    elif c["path"] == "paged":
        out = pq.pq_attn_decode_paged(q, k_d, v_d, kcb, vcb, table_d, lens, page_tokens=c["P"],
                                      chunk=c["chunk"])
    elif c["path"] == "step":
        desc = pq.attn_desc(q, k_d, kcb, chunk=c["chunk"])
        ws = pq.step_workspace(desc, q.device)
        out = pq.pq_attn_decode_step(q, dev(xk), dev(xv), k_d, v_d, kcb, vcb, lens, desc=desc,
                                     workspace=ws)
    else:
        desc, _ = pq.paged_desc(q, k_d, kcb, table_d, c["P"], chunk=c["chunk"])
        ws = pq.step_workspace(desc, q.device)
        out = pq.pq_attn_decode_step_paged(q, dev(xk), dev(xv), k_d, v_d, kcb, vcb, table_d, lens,
                                           page_tokens=c["P"], chunk=c["chunk"], workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(k_d.cpu().numpy(), exp_k)
    np.testing.assert_array_equal(v_d.cpu().numpy(), exp_v)
    assert_attn_close(out.cpu().numpy(), ref, f"case {i} {c['path']}")
    if c["path"].endswith("step") and ws is not None:
        rec = pq.pq_attn_workspace_bytes(desc)
        assert (ws[rec:rec + desc.batch * desc.n_kv_heads * 4] == 0).all(), "arrival counters not reset"


FP8_CASES = [dict(draw_case(1000 + i), path="decode") for i in range(24)]


@pytest.mark.parametrize("i", range(len(FP8_CASES)))
def test_sweep_fp8_codebooks(i):
    """The same sweep of shapes for the dense decode with E4M3 codebooks: the
    oracle on the exactly decoded bytes, and bit for bit the fp16 call on the
    fp16 upcast."""
    c = FP8_CASES[i]
    say(f"fp8 case {i}: {c}")
    _, inp = gen.random_case(c["seed"], batch=c["B"], n_q_heads=c["G"] * c["Hkv"],
                             n_kv_heads=c["Hkv"], max_len=c["Lmax"], n_sub=c["M"], lens=c["lens"])
    rng = np.random.default_rng(c["seed"] + 2)
    k8 = gen.codebooks_fp8(rng, c["Hkv"], c["M"], 256, 128 // c["M"])
    v8 = gen.codebooks_fp8(rng, c["Hkv"], c["M"], 256, 128 // c["M"])
    kf, vf = oracle.fp8_e4m3_to_float64(k8), oracle.fp8_e4m3_to_float64(v8)
    lens = np.asarray(c["lens"], np.int32)
    ref = oracle.decode_attention(inp["q"], inp["k_codes"], inp["v_codes"], kf, vf, lens)
    q, kc, vc, lens_d = dev(inp["q"]), dev(inp["k_codes"]), dev(inp["v_codes"]), dev(lens)
    out8 = pq.pq_attn_decode_fp8cb(q, kc, vc, dev(k8), dev(v8), lens_d, chunk=c["chunk"])
    out16 = pq.pq_attn_decode(q, kc, vc, dev(kf.astype(np.float16)), dev(vf.astype(np.float16)),
                              lens_d, chunk=c["chunk"])
    torch.cuda.synchronize()
    got = out8.cpu().numpy()
    assert_attn_close(got, ref, f"fp8 case {i}")
    np.testing.assert_array_equal(got, out16.cpu().numpy())


def draw_encode_case(i):
    rng = np.random.default_rng(9700 + i)
    return dict(N=int(rng.choice([1, 7, 16, 17, 255, 256, 257, int(rng.integers(1, 1500))])),
                H=int(rng.choice([1, 2, 3, 8, 32, 40])), M=int(rng.choice([4, 8])),
                slots=bool(rng.integers(0, 2)), fp8=bool(rng.integers(0, 3) == 0), seed=9800 + i)


ENC_CASES = [draw_encode_case(i) for i in range(24)]


@pytest.mark.parametrize("i", range(len(ENC_CASES)))
def test_sweep_encode(i):
    """Encode over a sweep of vector counts (one tile, tile edges, many
    tiles), head counts and both segment counts, into a dense code array or
    through a permuted slot map, with fp16 or E4M3 codebooks: bit-exact
    against the oracle and the generating index on margin-checked inputs."""
    c = ENC_CASES[i]
    say(f"encode case {i}: {c}")
    rng = np.random.default_rng(c["seed"])
    N, H, M = c["N"], c["H"], c["M"]
    if c["fp8"]:
        cb8 = gen.codebooks_fp8(rng, H, M, 256, 128 // M)
        cb = oracle.fp8_e4m3_to_float64(cb8).astype(np.float16)
    else:
        cb = gen.codebooks(rng, H, M, 256, 128 // M)
    x, src = gen.noisy_codewords(rng, cb, N, 0.05)
    assert_clear_margins(x, cb, f"encode case {i}")
    exp = oracle.encode(x, cb)
    np.testing.assert_array_equal(exp, src)
    cb_d = dev(cb8) if c["fp8"] else dev(cb)
    enc = pq.pq_encode_fp8cb if c["fp8"] else pq.pq_encode
    if c["slots"]:
        # vector n goes to row perm[n] of a larger code array; other rows untouched
        rows = N + 5
        perm = rng.permutation(rows)[:N].astype(np.int64)
        codes = torch.full((rows, H, M), 77, dtype=torch.uint8, device="cuda")
        desc = pq.PQEncodeDesc(N, H, 128, M, 256, H * 128, 128, H * M, M, codes.numel())
        enc(dev(x), cb_d, codes, slots=dev(perm), desc=desc)
        torch.cuda.synchronize()
        want = np.full((rows, H, M), 77, dtype=np.uint8)
        want[perm] = exp
        np.testing.assert_array_equal(codes.cpu().numpy(), want)
    else:
        codes = torch.empty((N, H, M), dtype=torch.uint8, device="cuda")
        enc(dev(x), cb_d, codes)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes.cpu().numpy(), exp)
