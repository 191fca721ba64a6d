"""The seeded generators: reproducible, right shapes, the recipes' structure."""
import numpy as np

from synth import gen


def test_seeded_reproducible():
    a = gen.workload_inputs(1)
    b = gen.workload_inputs(1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    c = gen.workload_inputs(1, replica=3)
    assert not np.array_equal(a["k_codes"], c["k_codes"])


def test_shapes_and_dtypes_every_workload():
    for wid, w in gen.WORKLOADS.items():
        if wid == 4:   # large; its shapes follow the same code path
            continue
        inp = gen.workload_inputs(wid, with_encode=False)
        assert inp["q"].shape == (w.batch, w.n_q_heads, w.head_dim) and inp["q"].dtype == np.float16
        assert inp["k_codes"].shape == (w.batch, w.n_kv_heads, w.max_len, w.n_sub)
        assert inp["k_codes"].dtype == np.uint8 and inp["v_codes"].dtype == np.uint8
        assert inp["k_cb"].shape == (w.n_kv_heads, w.n_sub, w.n_codes, w.sub_dim)
        assert inp["lens"].dtype == np.int32 and inp["lens"].shape == (w.batch,)


def test_distributions():
    inp = gen.workload_inputs(2, with_encode=False)
    cb = inp["k_cb"].astype(np.float64)
    assert abs(cb.mean()) < 0.01 and abs(cb.std() - 1) < 0.01
    codes = inp["k_codes"]
    counts = np.bincount(codes.ravel(), minlength=256)
    assert counts.min() > 0.8 * codes.size / 256 and counts.max() < 1.2 * codes.size / 256


def test_ragged_mix():
    inp = gen.workload_inputs(5, with_encode=False)
    lens = inp["lens"]
    assert sorted(np.unique(lens).tolist()) == [512, 4096]
    assert (lens == 512).sum() == 45 and (lens == 4096).sum() == 19
    assert int(lens.sum()) == 100_864
    # not sorted: a seeded permutation
    assert not (np.diff(lens) >= 0).all()
    # padding past lens holds random codes, not zeros
    b = int(np.argmax(lens == 512))
    assert inp["k_codes"][b, :, 512:].any()


def test_prefill_slots():
    lens = np.array([3, 0, 2], dtype=np.int32)
    s = gen.prefill_slots(lens, n_kv_heads=4, max_len=10)
    np.testing.assert_array_equal(s, [0, 1, 2, 80, 81])


def test_noisy_codewords_recipe():
    rng = np.random.default_rng(0)
    cb = gen.codebooks(rng, 2, 4, 256, 32)
    x, src = gen.noisy_codewords(rng, cb, 5, 0.05)
    assert x.shape == (5, 2, 128) and x.dtype == np.float16 and src.shape == (5, 2, 4)
    for n in range(5):
        for h in range(2):
            for m in range(4):
                d = x[n, h, m * 32:(m + 1) * 32].astype(np.float64) - cb[h, m, src[n, h, m]]
                assert abs(d.std() - 0.05) < 0.03


def test_step_workspace_is_tied_to_its_descriptor():
    """The binding refuses a step workspace made for another shape (its
    arrival counters sit at a shape-dependent offset): host-side check, no
    GPU call."""
    import pytest
    torch = pytest.importorskip("torch")
    import decode_attention_product_amd as pq
    import os
    if not os.path.exists(pq.LIB_PATH):
        pytest.skip("library not built")
    a = pq.PQAttnDesc(2, 16, 2, 128, 8, 256, 4096, 1024, 0.0883883)
    b = pq.PQAttnDesc(4, 16, 2, 128, 8, 256, 4096, 1024, 0.0883883)
    ws = torch.zeros(pq.pq_attn_step_workspace_bytes(a), dtype=torch.uint8)
    ws._pq_step_key = pq._desc_key(a)
    pq._check_step_workspace(a, ws, "same shape")          # accepted
    with pytest.raises(ValueError):
        pq._check_step_workspace(b, ws, "other shape")


def test_step_workspace_key_follows_the_chunk():
    """The workspace key reuses the planner's chunk count per descriptor
    fields; a descriptor that differs only in its chunk gets its own count."""
    import pytest
    pytest.importorskip("torch")
    import decode_attention_product_amd as pq
    import os
    if not os.path.exists(pq.LIB_PATH):
        pytest.skip("library not built")
    a = pq.PQAttnDesc(1, 64, 8, 128, 4, 256, 131072, 2048, 0.0883883)
    b = pq.PQAttnDesc(1, 64, 8, 128, 4, 256, 131072, 4096, 0.0883883)
    for _ in range(2):     # first call fills the memo, second reads it
        assert pq._desc_key(a)[-1] == pq.pq_attn_num_chunks(a) == 64
        assert pq._desc_key(b)[-1] == pq.pq_attn_num_chunks(b) == 32
    b.chunk = 2048         # mutated in place: the key follows
    assert pq._desc_key(b) == pq._desc_key(a)


def test_tensor_checks_fast_path_and_errors():
    """The binding's tensor checks: the fast path accepts what the detailed
    checks accept (a shape given as a list too) and every failure still
    raises with its own message.  CPU tensors, device check off."""
    import pytest
    torch = pytest.importorskip("torch")
    import decode_attention_product_amd as pq
    t = torch.zeros((2, 3, 128), dtype=torch.float16)
    pq._need(t, "t", torch.float16, (2, 3, 128), device=False)
    pq._need(t, "t", torch.float16, [2, 3, 128], device=False)
    pq._need(None, "t", torch.float16, (1,), device=False)
    with pytest.raises(TypeError, match="expected torch.float16"):
        pq._need(t.float(), "t", torch.float16, (2, 3, 128), device=False)
    with pytest.raises(ValueError, match="expected shape"):
        pq._need(t, "t", torch.float16, (2, 3, 64), device=False)
    with pytest.raises(ValueError, match="contiguous"):
        pq._need(t.transpose(0, 1), "t", torch.float16, (3, 2, 128), device=False)
    with pytest.raises(ValueError, match="GPU tensor"):
        pq._need(t, "t", torch.float16, (2, 3, 128))
