"""The decode step without allocation (pq_attn_decode_step_noalloc), called
through the C ABI, against pq_attn_decode_step on the same inputs: two calls
in a row, the second on a smaller shape, in the same process (the library's
device scratch is shared between them).  Outputs and the new codes must be
identical: the two entry points run the same kernels on the same chunking,
only the scratch's place differs."""
import ctypes
import sys

import numpy as np
import pytest

from margins import assert_clear_margins
from synth import gen

torch = pytest.importorskip("torch")
pq = pytest.importorskip("decode_attention_product_amd")

pytestmark = pytest.mark.gpu

TOL = 1e-3


def say(msg):
    print(f"[noalloc] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def both_ways(seed, B, Hq, Hkv, L, M, lens, chunk):
    _, inp = gen.random_case(seed, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, max_len=L, n_sub=M,
                             lens=lens)
    xk, _, xv, _ = gen.step_tokens(np.random.default_rng(seed + 1), inp["k_cb"], inp["v_cb"], B)
    assert_clear_margins(xk, inp["k_cb"], "new token K")
    assert_clear_margins(xv, inp["v_cb"], "new token V")
    q, kcb, vcb, l = dev(inp["q"]), dev(inp["k_cb"]), dev(inp["v_cb"]), dev(np.asarray(lens, np.int32))
    xk_d, xv_d = dev(xk), dev(xv)
    desc = pq.attn_desc(q, dev(inp["k_codes"]), kcb, chunk=chunk)
    # the existing entry point, its own workspace
    kc1, vc1 = dev(inp["k_codes"]), dev(inp["v_codes"])
    ref = pq.pq_attn_decode_step(q, xk_d, xv_d, kc1, vc1, kcb, vcb, l, desc=desc,
                                 workspace=pq.step_workspace(desc, q.device))
    # the no-allocation entry point, straight through the C ABI
    kc2, vc2 = dev(inp["k_codes"]), dev(inp["v_codes"])
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    lib = pq.load_library()
    st = lib.pq_attn_decode_step_noalloc(ctypes.byref(desc), q.data_ptr(), xk_d.data_ptr(),
                                         xv_d.data_ptr(), kc2.data_ptr(), vc2.data_ptr(),
                                         kcb.data_ptr(), vcb.data_ptr(), l.data_ptr(), out.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0, pq.status_string(st)
    torch.cuda.synchronize()
    got, want = out.cpu().numpy(), ref.cpu().numpy()
    assert np.isfinite(got).all()
    scale = np.abs(want).max()
    err = np.abs(got.astype(np.float64) - want).max()
    say(f"B={B} Hq={Hq} Hkv={Hkv} L={L} M={M} chunk={chunk} C={pq.pq_attn_num_chunks(desc)}: "
        f"max|d| = {err:.3e} of {scale:.3e}")
    assert err <= TOL * scale
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(kc2.cpu().numpy(), kc1.cpu().numpy())
    np.testing.assert_array_equal(vc2.cpu().numpy(), vc1.cpu().numpy())


def test_noalloc_step_two_calls_second_smaller():
    # the GQA shape (8 KV heads, 8 query heads each, M = 8), four chunks merged
    # in the launch; then a smaller one with another head group and chunking
    both_ways(9100, 8, 64, 8, 8192, 8, [8192, 5000, 1, 8191, 4096, 4097, 2, 8000], 0)
    both_ways(9200, 3, 8, 2, 1024, 4, [1024, 300, 0], 256)


def test_noalloc_step_request_batched_and_one_chunk():
    # one query head per KV head and 1024 pairs: the encode launch, the
    # request-batched kernel and the merge launch, records in the scratch;
    # then a one-chunk shape that needs no scratch at all
    both_ways(9300, 64, 16, 16, 4096, 8, [4096] * 32 + [1000] * 32, 0)
    both_ways(9400, 2, 4, 4, 512, 8, [512, 17], 0)
