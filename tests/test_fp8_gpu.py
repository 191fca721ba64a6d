"""GPU parity with FP8 (OCP E4M3) codebooks (AQPIM page, section 4.2), through
the C ABI.

The oracle decodes the codebook bytes exactly (fp8_e4m3_to_float64) and runs
its plain attention and encode on those values.  Bars: attention within
1e-3 * max|oracle| over a call's output, encode bit-exact on inputs whose
float64 margins clear 1e-4.  Since every E4M3 value is an fp16 value, the
FP8 calls must also give exactly -- bit for bit -- what the fp16 calls give
on the fp16 upcast of the same codebooks.
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
    print(f"[fp8] {msg}", flush=True)
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
        assert err == 0
        return
    say(f"{what}: max|d| = {err:.3e}, max|ref| = {scale:.3e}, ratio {err / scale:.2e}")
    assert err <= TOL * scale, f"{what}: max|d| {err:.3e} > {TOL} * {scale:.3e}"


def upcast(cb8):
    return oracle.fp8_e4m3_to_float64(cb8).astype(np.float16)


def fp8_case(seed, B, Hq, Hkv, L, M, lens, every_value=False):
    """A random case whose K and V codebooks are E4M3 bytes (N(0, 1) rounded);
    with every_value, KV head 0's K codebook walks through every finite E4M3
    byte (zeros, -0, subnormals, 448) instead."""
    _, inp = gen.random_case(seed, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_len=L, n_sub=M,
                             lens=lens)
    rng = np.random.default_rng(seed + 17)
    k8 = gen.codebooks_fp8(rng, Hkv, M, 256, 128 // M)
    v8 = gen.codebooks_fp8(rng, Hkv, M, 256, 128 // M)
    if every_value:
        walk = (np.arange(256 * (128 // M)).reshape(256, 128 // M) * 7 + 3) % 256
        walk[np.isin(walk, [0x7F, 0xFF])] = 0x38
        k8[0, 0] = walk.astype(np.uint8)
        v8[0, 1] = walk[::-1].astype(np.uint8)
    inp["k_cb8"], inp["v_cb8"] = k8, v8
    inp["k_cb"], inp["v_cb"] = upcast(k8), upcast(v8)        # exact fp16 values
    return inp


def run_fp8(inp, chunk=0):
    t = [dev(inp[k]) for k in ("q", "k_codes", "v_codes", "k_cb8", "v_cb8", "lens")]
    out = pq.pq_attn_decode_fp8cb(*t, chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # (G, M, Hkv, B, L, chunk, lens)
    (8, 8, 2, 3, 4096, 0, [4096, 1, 2049]),
    (8, 4, 2, 2, 2048, 512, [2048, 700]),
    (4, 8, 2, 4, 1024, 1024, [0, 1024, 1023, 17]),
    (2, 4, 4, 2, 512, 128, [512, 129]),
    (1, 8, 4, 3, 256, 0, [256, 0, 100]),
    (1, 4, 8, 2, 4096, 4096, [4096, 3000]),
]


@pytest.mark.parametrize("G,M,Hkv,B,L,chunk,lens", CASES)
def test_fp8_decode_matches_oracle_and_fp16_upcast(G, M, Hkv, B, L, chunk, lens):
    say(f"fp8 decode G={G} M={M} Hkv={Hkv} B={B} L={L} chunk={chunk} lens={lens}")
    inp = fp8_case(8000 + G * 10 + M, B, G * Hkv, Hkv, L, M, np.asarray(lens, np.int32),
                   every_value=(G == 8))
    got = run_fp8(inp, chunk)
    ref = oracle.decode_attention(inp["q"], inp["k_codes"], inp["v_codes"],
                                  oracle.fp8_e4m3_to_float64(inp["k_cb8"]),
                                  oracle.fp8_e4m3_to_float64(inp["v_cb8"]), inp["lens"])
    assert_attn_close(got, ref, f"fp8 G={G} M={M}")
    for b, l in enumerate(lens):
        if l == 0:
            assert (got[b] == 0).all()
    t16 = [dev(inp[k]) for k in ATTN]
    out16 = pq.pq_attn_decode(*t16, chunk=chunk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, out16.cpu().numpy())


def test_fp8_partials_equal_fp16_partials():
    say("fp8 chunk records vs fp16 records on the upcast codebooks")
    inp = fp8_case(8100, 2, 16, 2, 2048, 8, np.array([2048, 1500], np.int32))
    t8 = [dev(inp[k]) for k in ("q", "k_codes", "v_codes", "k_cb8", "v_cb8", "lens")]
    t16 = [dev(inp[k]) for k in ATTN]
    a = pq.pq_attn_partials_fp8cb(*t8, chunk=256)
    b = pq.pq_attn_partials(*t16, chunk=256)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
    rm, rl, ro = oracle.chunk_partials(inp["q"], inp["k_codes"], inp["v_codes"], inp["k_cb"],
                                       inp["v_cb"], inp["lens"], chunk=256)
    assert_attn_close(a[2].cpu().numpy(), ro, "fp8 partial o")


def test_fp8_gqa_workload_shape():
    """The GQA decode shape (B=8, Hq=64, Hkv=8, L=8192, M=8) with FP8
    codebooks drawn for it."""
    say("fp8 decode on the gqa shape")
    w = gen.WORKLOADS[3]
    inp = gen.workload_inputs(3, with_encode=False)
    rng = np.random.default_rng(8200)
    inp["k_cb8"] = gen.codebooks_fp8(rng, w.n_kv_heads, w.n_sub, 256, w.sub_dim)
    inp["v_cb8"] = gen.codebooks_fp8(rng, w.n_kv_heads, w.n_sub, 256, w.sub_dim)
    got = run_fp8(inp)
    ref = oracle.decode_attention(inp["q"], inp["k_codes"], inp["v_codes"],
                                  oracle.fp8_e4m3_to_float64(inp["k_cb8"]),
                                  oracle.fp8_e4m3_to_float64(inp["v_cb8"]), inp["lens"])
    assert_attn_close(got, ref, "fp8 gqa")


@pytest.mark.parametrize("M,N", [(4, 3000), (8, 40)])
def test_fp8_encode_bit_exact(M, N):
    say(f"fp8 encode M={M} N={N}")
    rng = np.random.default_rng(8300 + M)
    H = 8
    cb8 = gen.codebooks_fp8(rng, H, M, 256, 128 // M)
    cb16 = upcast(cb8)
    x, src = gen.noisy_codewords(rng, cb16, N, 0.05)
    assert_clear_margins(x, cb16, "fp8 encode")
    codes = torch.empty((N, H, M), dtype=torch.uint8, device="cuda")
    pq.pq_encode_fp8cb(dev(x), dev(cb8), codes)
    codes16 = torch.empty((N, H, M), dtype=torch.uint8, device="cuda")
    pq.pq_encode(dev(x), dev(cb16), codes16)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    np.testing.assert_array_equal(got, oracle.encode(x, oracle.fp8_e4m3_to_float64(cb8)))
    np.testing.assert_array_equal(got, src)
    np.testing.assert_array_equal(got, codes16.cpu().numpy())
