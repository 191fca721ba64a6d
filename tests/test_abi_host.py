"""The C ABI on the host: the library loads, exports every function the
header declares, and rejects bad arguments before launching anything.

No case here passes host validation: every call carries at least one bad
field, so nothing reaches the GPU even on a machine that has one.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import decode_attention_product_amd as pq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pqattn.h")
CSRC = os.path.join(ROOT, "decode_attention_product_amd", "csrc")

FAKE = 0x10000      # an aligned, non-null address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(pq_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pq.LIB_PATH):
        pytest.fail("libpqattn.so is not built (python -m decode_attention_product_amd.build)")
    return pq.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(pq.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", pq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pq_\w+)$", out, flags=re.M))
    assert set(names) <= exported
    for n in names:
        assert hasattr(lib, n)


def _desc(**kw):
    d = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_sub=4, n_codes=256,
             max_len=64, chunk=0, scale=0.0883883)
    d.update(kw)
    return pq.PQAttnDesc(**d)


def test_status_strings(lib):
    for s in range(7):
        assert pq.status_string(s) and pq.status_string(s) != "unknown status"
    assert pq.status_string(99) == "unknown status"


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, 2), ("n_q_heads", 0, 2), ("n_kv_heads", 3, 2), ("head_dim", 130, 2),
    ("n_sub", 0, 2), ("max_len", 0, 2), ("chunk", -1, 2), ("scale", 0.0, 2),
    ("scale", float("nan"), 2), ("scale", float("inf"), 2),
    ("head_dim", 64, 3), ("n_codes", 16, 3), ("n_sub", 2, 3), ("n_sub", 16, 3),
    ("max_len", 40, 3), ("n_q_heads", 32, 3),      # group of 16 is not built
])
def test_bad_descriptor(lib, field, value, status):
    d = _desc(**{field: value})
    assert lib.pq_attn_num_chunks(ctypes.byref(d)) == -1
    assert lib.pq_attn_workspace_bytes(ctypes.byref(d)) == 0
    st = lib.pq_attn_decode(ctypes.byref(d), *([FAKE] * 7), FAKE, 1 << 30, None)
    assert st == status
    st = lib.pq_attn_partials(ctypes.byref(d), *([FAKE] * 9), None)
    assert st == status
    st = lib.pq_attn_partials_timed(ctypes.byref(d), *([FAKE] * 9), None, None, None)
    assert st == status


def test_null_descriptor(lib):
    assert lib.pq_attn_decode(None, *([FAKE] * 7), FAKE, 1 << 30, None) == 1
    assert lib.pq_encode(None, FAKE, FAKE, None, FAKE, None) == 1


@pytest.mark.parametrize("which", range(7))
def test_null_pointer(lib, which):
    ptrs = [FAKE] * 7          # q, kc, vc, kcb, vcb, lens, out
    ptrs[which] = None
    assert lib.pq_attn_decode(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None) == 1


def test_misaligned_pointer(lib):
    ptrs = [FAKE] * 7
    ptrs[1] = FAKE + 4
    assert lib.pq_attn_decode(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None) == 6


def test_workspace_checks(lib):
    d = _desc(max_len=4096, chunk=256)
    need = lib.pq_attn_workspace_bytes(ctypes.byref(d))
    assert need > 0
    ptrs = [FAKE] * 7
    assert lib.pq_attn_decode(ctypes.byref(d), *ptrs, None, need, None) == 4
    assert lib.pq_attn_decode(ctypes.byref(d), *ptrs, FAKE, need - 1, None) == 4
    assert lib.pq_attn_decode(ctypes.byref(d), *ptrs, FAKE + 8, need, None) == 4


def test_chunking_and_workspace_sizes(lib):
    # the long-context workload: T = 2048 over 131072 tokens -> 64 chunks
    d = _desc(batch=1, n_q_heads=64, n_kv_heads=8, max_len=131072, chunk=2048)
    assert lib.pq_attn_num_chunks(ctypes.byref(d)) == 64
    rows, C, D = 64, 64, 128
    assert lib.pq_attn_workspace_bytes(ctypes.byref(d)) >= rows * C * (D + 2) * 4
    assert lib.pq_attn_workspace_bytes(ctypes.byref(d)) <= rows * C * (D + 2) * 4 + 3 * 256
    # one chunk needs no workspace
    d1 = _desc(max_len=512, chunk=512)
    assert lib.pq_attn_num_chunks(ctypes.byref(d1)) == 1
    assert lib.pq_attn_workspace_bytes(ctypes.byref(d1)) == 0
    # chunk larger than the cache is clamped to one chunk
    d2 = _desc(max_len=512, chunk=100000)
    assert lib.pq_attn_num_chunks(ctypes.byref(d2)) == 1
    # the library's pick fills the chip.  The GQA shape has too few (request,
    # KV head) pairs, so the 8 query heads of a KV head are split over 4
    # workgroups of two, each over the whole cache: one chunk, no records
    d3 = _desc(batch=8, n_q_heads=64, n_kv_heads=8, n_sub=8, max_len=8192)
    assert lib.pq_attn_num_chunks(ctypes.byref(d3)) == 1
    assert lib.pq_attn_workspace_bytes(ctypes.byref(d3)) == 0
    assert lib.pq_attn_step_workspace_bytes(ctypes.byref(d3)) == 0
    # an explicit chunk keeps the token split
    d4 = _desc(batch=8, n_q_heads=64, n_kv_heads=8, n_sub=8, max_len=8192, chunk=2048)
    assert lib.pq_attn_num_chunks(ctypes.byref(d4)) == 4
    # longer caches than one chunk of 8192 tokens split the tokens: at least
    # 256 workgroups when possible
    d5 = _desc(batch=2, n_q_heads=64, n_kv_heads=8, n_sub=8, max_len=16384)
    C5 = lib.pq_attn_num_chunks(ctypes.byref(d5))
    assert 2 * 8 * C5 >= 256 and 16384 % C5 == 0
    # so do few pairs (the split would leave most CUs idle)
    d6 = _desc(batch=1, n_q_heads=64, n_kv_heads=8, n_sub=8, max_len=8192)
    assert lib.pq_attn_num_chunks(ctypes.byref(d6)) > 1


def test_step_workspace_sizes(lib):
    # records of pq_attn_workspace_bytes plus one 32-bit counter per (b, kv head)
    d = _desc(batch=8, n_q_heads=64, n_kv_heads=8, n_sub=8, max_len=8192, chunk=2048)
    rec = lib.pq_attn_workspace_bytes(ctypes.byref(d))
    step = lib.pq_attn_step_workspace_bytes(ctypes.byref(d))
    assert rec > 0 and step >= rec + 8 * 8 * 4 and step <= rec + 8 * 8 * 4 + 256
    assert step % 256 == 0
    d1 = _desc(max_len=512, chunk=512)          # one chunk: no records, no counters
    assert lib.pq_attn_step_workspace_bytes(ctypes.byref(d1)) == 0
    assert lib.pq_attn_step_workspace_bytes(ctypes.byref(_desc(n_kv_heads=3))) == 0


@pytest.mark.parametrize("which", range(9))
def test_step_null_pointer(lib, which):
    # q, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, out
    ptrs = [FAKE] * 9
    ptrs[which] = None
    assert lib.pq_attn_decode_step(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None) == 1
    assert lib.pq_attn_decode_step_timed(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None,
                                         None, None) == 1


def test_step_alignment_and_workspace(lib):
    ptrs = [FAKE] * 9
    ptrs[1] = FAKE + 8                           # k_new
    assert lib.pq_attn_decode_step(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None) == 6
    ptrs = [FAKE] * 9
    ptrs[2] = FAKE + 2                           # v_new
    assert lib.pq_attn_decode_step(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None) == 6
    d = _desc(max_len=4096, chunk=256)
    need = lib.pq_attn_step_workspace_bytes(ctypes.byref(d))
    ptrs = [FAKE] * 9
    assert lib.pq_attn_decode_step(ctypes.byref(d), *ptrs, None, need, None) == 4
    assert lib.pq_attn_decode_step(ctypes.byref(d), *ptrs, FAKE, need - 1, None) == 4
    # the record-only size is not enough for the step
    rec = lib.pq_attn_workspace_bytes(ctypes.byref(d))
    assert lib.pq_attn_decode_step(ctypes.byref(d), *ptrs, FAKE, rec, None) == 4
    bad = _desc(n_q_heads=7)                     # not a multiple of n_kv_heads
    assert lib.pq_attn_decode_step(ctypes.byref(bad), *ptrs, FAKE, need, None) == 2
    odd = _desc(n_q_heads=6)                     # G = 3: consistent, not built
    assert lib.pq_attn_decode_step(ctypes.byref(odd), *ptrs, FAKE, need, None) == 3


def test_chunk_longer_than_a_workgroup_takes(lib):
    d = _desc(max_len=8192, chunk=4097)
    assert lib.pq_attn_num_chunks(ctypes.byref(d)) == -1
    assert lib.pq_attn_decode(ctypes.byref(d), *([FAKE] * 7), FAKE, 1 << 30, None) == 3
    d = _desc(max_len=8192, chunk=4096)
    assert lib.pq_attn_num_chunks(ctypes.byref(d)) == 2
    d = _desc(max_len=4096, chunk=10000)      # clamped to the capacity first
    assert lib.pq_attn_num_chunks(ctypes.byref(d)) == 1


def test_reduce_checks(lib):
    assert lib.pq_attn_reduce(4, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.pq_attn_reduce(-1, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.pq_attn_reduce(4, 2, 64, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert lib.pq_attn_reduce(4, 2, 128, None, FAKE, FAKE, FAKE, None) == 1


def _edesc(**kw):
    d = dict(n_vec=10, n_heads=2, head_dim=128, n_sub=4, n_codes=256, x_stride_vec=256,
             x_stride_head=128, codes_stride_slot=8, codes_stride_head=4, codes_bytes=80)
    d.update(kw)
    return pq.PQEncodeDesc(**d)


@pytest.mark.parametrize("field,value,status", [
    ("n_vec", -1, 2), ("n_heads", 0, 2), ("head_dim", 102, 2), ("x_stride_vec", -8, 2),
    ("codes_bytes", -1, 2), ("n_codes", 512, 3), ("n_sub", 2, 3), ("head_dim", 64, 3),
    ("x_stride_vec", 250, 6), ("x_stride_head", 4, 6), ("codes_stride_slot", 6, 6),
    ("codes_stride_head", 2, 6), ("codes_bytes", 79, 2),
])
def test_bad_encode_descriptor(lib, field, value, status):
    d = _edesc(**{field: value})
    assert lib.pq_encode(ctypes.byref(d), FAKE, FAKE, None, FAKE, None) == status


def test_encode_many_checks(lib):
    arr = ctypes.c_void_p * 4
    ok = arr(FAKE, FAKE, FAKE, FAKE)
    d = _edesc(codes_bytes=79)                   # invalid: nothing can launch
    assert lib.pq_encode_many(ctypes.byref(d), 2, ok, ok, None, ok, None) == 2
    d = _edesc(n_sub=3)
    for n in (0, 5, -1):
        assert lib.pq_encode_many(ctypes.byref(d), n, ok, ok, None, ok, None) == 2
    d = _edesc()
    assert lib.pq_encode_many(ctypes.byref(d), 0, ok, ok, None, ok, None) == 2
    assert lib.pq_encode_many(ctypes.byref(d), 5, ok, ok, None, ok, None) == 2
    nul = arr(FAKE, None, FAKE, FAKE)
    assert lib.pq_encode_many(ctypes.byref(d), 2, nul, ok, None, ok, None) == 1
    mis = arr(FAKE, FAKE + 4, FAKE, FAKE)
    assert lib.pq_encode_many(ctypes.byref(d), 2, ok, mis, None, ok, None) == 6


def test_encode_pointer_checks(lib):
    d = _edesc(codes_bytes=79)        # also invalid: nothing can launch
    assert lib.pq_encode(ctypes.byref(d), None, FAKE, None, FAKE, None) in (1, 2)
    d = _edesc(n_sub=3)
    assert lib.pq_encode(ctypes.byref(d), FAKE, FAKE, None, FAKE, None) == 2


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_plan_unit_with_sanitizers(tmp_path):
    """The host planning code built with g++, ASan and UBSan, run on edge cases."""
    exe = tmp_path / "plan_test"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "plan_unit.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan_unit: all" in r.stdout


def _pages(**kw):
    t = dict(block_table=FAKE, page_tokens=16, max_pages=4, n_pages=9)
    t.update(kw)
    return pq.PQPageTable(**t)


def test_paged_null_and_shape_checks(lib):
    d = _desc()                                  # max_len 64 = 4 pages of 16
    ptrs = [FAKE] * 8                            # q, k_pool, v_pool, k_cb, v_cb, lens, out, ws
    ok = _pages()
    assert lib.pq_attn_decode_paged(ctypes.byref(d), None, *ptrs[:7], None, 0, None) == 1
    assert lib.pq_attn_decode_paged(ctypes.byref(d), ctypes.byref(_pages(block_table=None)),
                                    *ptrs[:7], None, 0, None) == 1
    for bad in (_pages(page_tokens=24), _pages(page_tokens=8), _pages(page_tokens=1 << 17),
                _pages(max_pages=3), _pages(n_pages=0), _pages(page_tokens=32)):
        assert lib.pq_attn_decode_paged(ctypes.byref(d), ctypes.byref(bad), *ptrs[:7], None, 0,
                                        None) == 2
    for which in range(7):
        p = list(ptrs[:7])
        p[which] = None
        assert lib.pq_attn_decode_paged(ctypes.byref(d), ctypes.byref(ok), *p, FAKE, 1 << 30,
                                        None) == 1
    p = list(ptrs[:7])
    p[1] = FAKE + 4                              # k_pool
    assert lib.pq_attn_decode_paged(ctypes.byref(d), ctypes.byref(ok), *p, FAKE, 1 << 30,
                                    None) == 6
    # four chunks of 16 tokens need records
    d4 = _desc(chunk=16)
    need = lib.pq_attn_workspace_bytes(ctypes.byref(d4))
    assert need > 0
    assert lib.pq_attn_decode_paged(ctypes.byref(d4), ctypes.byref(ok), *ptrs[:7], FAKE, need - 1,
                                    None) == 4


def test_paged_step_checks(lib):
    d = _desc(chunk=16)
    need = lib.pq_attn_step_workspace_bytes(ctypes.byref(d))
    ptrs = [FAKE] * 10       # q, k_new, v_new, k_pool, v_pool, k_cb, v_cb, lens, out
    ok = _pages()
    for which in range(9):
        p = list(ptrs[:9])
        p[which] = None
        assert lib.pq_attn_decode_step_paged(ctypes.byref(d), ctypes.byref(ok), *p, FAKE, need,
                                             None) == 1
        assert lib.pq_attn_decode_step_paged_timed(ctypes.byref(d), ctypes.byref(ok), *p, FAKE,
                                                   need, None, None, None) == 1
    assert lib.pq_attn_decode_step_paged(ctypes.byref(d), ctypes.byref(_pages(max_pages=5)),
                                         *ptrs[:9], FAKE, need, None) == 2
    assert lib.pq_attn_decode_step_paged(ctypes.byref(d), ctypes.byref(ok), *ptrs[:9], FAKE,
                                         need - 1, None) == 4
    p = list(ptrs[:9])
    p[2] = FAKE + 2                              # v_new
    assert lib.pq_attn_decode_step_paged(ctypes.byref(d), ctypes.byref(ok), *p, FAKE, need,
                                         None) == 6


def test_paged_encode_desc_matches_pool_layout():
    d = pq.paged_encode_desc(10, n_kv_heads=3, n_pages=7, page_tokens=16, n_sub=8)
    assert d.codes_stride_slot == 8 and d.codes_stride_head == 7 * 16 * 8
    assert d.codes_bytes == 3 * 7 * 16 * 8


def _enc_desc(**kw):
    d = dict(n_vec=32, n_heads=2, head_dim=128, n_sub=4, n_codes=256, x_stride_vec=256,
             x_stride_head=128, codes_stride_slot=8, codes_stride_head=4, codes_bytes=32 * 8)
    d.update(kw)
    return pq.PQEncodeDesc(**d)


def test_codebook_update_and_kmeans_checks(lib):
    d = _enc_desc()
    for which in range(3):                       # x, codes, codebook
        p = [FAKE] * 3
        p[which] = None
        assert lib.pq_codebook_update(ctypes.byref(d), *p, None, None) == 1
        assert lib.pq_kmeans(ctypes.byref(d), p[0], p[2], 3, p[1], None) == 1
    # identity places past the codes buffer
    short = _enc_desc(codes_bytes=32 * 8 - 1)
    assert lib.pq_codebook_update(ctypes.byref(short), FAKE, FAKE, FAKE, None, None) == 2
    assert lib.pq_kmeans(ctypes.byref(short), FAKE, FAKE, 1, FAKE, None) == 2
    # more vectors than the exact 64-bit sums allow
    big = _enc_desc(n_vec=(1 << 22) + 1, codes_bytes=((1 << 22) + 1) * 8)
    assert lib.pq_codebook_update(ctypes.byref(big), FAKE, FAKE, FAKE, None, None) == 3
    assert lib.pq_kmeans(ctypes.byref(d), FAKE, FAKE, -1, FAKE, None) == 2
    assert lib.pq_codebook_update(ctypes.byref(d), FAKE + 2, FAKE, FAKE, None, None) == 6
    assert lib.pq_codebook_update(ctypes.byref(d), FAKE, FAKE, FAKE + 8, None, None) == 6
    assert lib.pq_codebook_update(ctypes.byref(_enc_desc(n_sub=2)), FAKE, FAKE, FAKE, None,
                                  None) == 3


def test_kmeans_many_checks(lib):
    d = _enc_desc()
    arr = ctypes.c_void_p * 3
    ok = arr(FAKE, FAKE, FAKE)
    for n in (0, 3):
        assert lib.pq_kmeans_many(ctypes.byref(d), n, ok, ok, 2, ok, None) == 2
    assert lib.pq_kmeans_many(ctypes.byref(d), 2, None, ok, 2, ok, None) == 1
    assert lib.pq_kmeans_many(ctypes.byref(d), 2, ok, ok, 2, arr(FAKE, None, FAKE), None) == 1
    assert lib.pq_kmeans_many(ctypes.byref(d), 2, ok, ok, 2, arr(FAKE, FAKE + 2, FAKE), None) == 6


def test_paged_partials_checks(lib):
    d = _desc()
    ptrs = [FAKE] * 9        # q, k_pool, v_pool, k_cb, v_cb, lens, part_m, part_l, part_o
    assert lib.pq_attn_partials_paged(ctypes.byref(d), None, *ptrs, None) == 1
    assert lib.pq_attn_partials_paged(ctypes.byref(d), ctypes.byref(_pages(page_tokens=24)), *ptrs,
                                      None) == 2
    for which in range(9):
        p = list(ptrs)
        p[which] = None
        assert lib.pq_attn_partials_paged(ctypes.byref(d), ctypes.byref(_pages()), *p, None) == 1


# --------------------------------------------------------------------------
# FP8-codebook entry points: the same host checks, nothing launched
# --------------------------------------------------------------------------

@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, 2), ("n_kv_heads", 3, 2), ("scale", 0.0, 2), ("head_dim", 64, 3),
    ("n_sub", 2, 3), ("max_len", 40, 3),
])
def test_fp8_bad_descriptor(lib, field, value, status):
    d = _desc(**{field: value})
    assert lib.pq_attn_decode_fp8cb(ctypes.byref(d), *([FAKE] * 7), FAKE, 1 << 30, None) == status
    assert lib.pq_attn_partials_fp8cb(ctypes.byref(d), *([FAKE] * 9), None) == status


@pytest.mark.parametrize("which", range(7))
def test_fp8_null_pointer(lib, which):
    ptrs = [FAKE] * 7          # q, kc, vc, kcb, vcb, lens, out
    ptrs[which] = None
    assert lib.pq_attn_decode_fp8cb(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None) == 1


def test_fp8_alignment_and_workspace(lib):
    for which in range(5):
        ptrs = [FAKE] * 7
        ptrs[which] = FAKE + 4
        assert lib.pq_attn_decode_fp8cb(ctypes.byref(_desc()), *ptrs, FAKE, 1 << 30, None) == 6
    d = _desc(max_len=4096, chunk=256)
    need = lib.pq_attn_workspace_bytes(ctypes.byref(d))
    ptrs = [FAKE] * 7
    assert lib.pq_attn_decode_fp8cb(ctypes.byref(d), *ptrs, None, need, None) == 4
    assert lib.pq_attn_decode_fp8cb(ctypes.byref(d), *ptrs, FAKE, need - 1, None) == 4


def test_fp8_encode_checks(lib):
    for field, value, status in (("n_vec", -1, 2), ("n_codes", 512, 3), ("codes_bytes", 79, 2),
                                 ("x_stride_head", 4, 6)):
        d = _edesc(**{field: value})
        assert lib.pq_encode_fp8cb(ctypes.byref(d), FAKE, FAKE, None, FAKE, None) == status
    d = _edesc()
    assert lib.pq_encode_fp8cb(ctypes.byref(d), None, FAKE, None, FAKE, None) == 1
    assert lib.pq_encode_fp8cb(ctypes.byref(d), FAKE, None, None, FAKE, None) == 1
    assert lib.pq_encode_fp8cb(ctypes.byref(d), FAKE, FAKE + 4, None, FAKE, None) == 6
    assert lib.pq_encode_fp8cb(ctypes.byref(d), FAKE, FAKE, None, FAKE + 1, None) == 6


def test_bench_library_exports_the_stream_reference():
    path = os.path.join(os.path.dirname(pq.LIB_PATH), "libpqbench.so")
    if not os.path.exists(path):
        pytest.fail("libpqbench.so is not built (python -m decode_attention_product_amd.build)")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    assert re.search(r"\bT pqbench_stream_read$", out, flags=re.M)
    lib = ctypes.CDLL(path)
    lib.pqbench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    # invalid arguments are refused before any launch (hipErrorInvalidValue = 1)
    assert lib.pqbench_stream_read(None, 16, FAKE, 1, 64, None) == 1
    assert lib.pqbench_stream_read(FAKE, 15, FAKE, 1, 64, None) == 1
    assert lib.pqbench_stream_read(FAKE + 8, 16, FAKE, 1, 64, None) == 1
    assert lib.pqbench_stream_read(FAKE, 16, FAKE, 1, 100, None) == 1
    assert lib.pqbench_stream_read(FAKE, 16, FAKE, 0, 64, None) == 1


def test_noalloc_step_rejects_what_its_scratch_cannot_hold(lib):
    """Shapes whose chunk records exceed the built-in 8 MiB (or whose
    counters exceed 65,536) are refused with PQ_ERR_WORKSPACE before any
    device call; null pointers with PQ_ERR_NULL."""
    big = _desc(batch=64, n_q_heads=64, n_kv_heads=8, max_len=131072, chunk=1024)
    assert lib.pq_attn_workspace_bytes(ctypes.byref(big)) > 8 << 20
    assert lib.pq_attn_decode_step_noalloc(ctypes.byref(big), *([FAKE] * 9), None) == 4
    ptrs = [FAKE] * 9
    ptrs[0] = None
    assert lib.pq_attn_decode_step_noalloc(ctypes.byref(_desc()), *ptrs, None) == 1
    bad = _desc(batch=0)
    assert lib.pq_attn_decode_step_noalloc(ctypes.byref(bad), *([FAKE] * 9), None) == 2
