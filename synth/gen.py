"""Seeded synthetic inputs for PQ-KV decode attention and PQ encode.

This module holds the workload recipes and the random draws only.  It does
none of the method's arithmetic (no lookup tables, no scores, no softmax, no
distance search): the CPU oracle and the HIP library both take their inputs
from here and nothing else is shared between them.

Workloads (one layer, one decode step each):

  tiny          B=1,  Hq=Hkv=8,  L=512,    M=4, plus one new token per head
                to encode (a random codeword + N(0, 0.05^2) noise)
  page-sizing   B=4,  Hq=Hkv=32, L=2048,   M=4  -- the batch/sequence/head
                sizes the AQPIM page uses for its KV footprint (section 2.1)
  gqa           B=8,  Hq=64, Hkv=8, L=8192, M=8 -- the Qwen-72B head shape of
                the memory-wall chapter (section 1.1.1, GQA in 1.4.3)
  long-splitk   B=1,  Hq=64, Hkv=8, L=131072, M=4, chunks of 2048 tokens
  ragged        64 requests, 45 of 512 tokens and 19 of 4096 tokens (the
                70/30 mix of the PAM page, section 4.1), H=32, M=4, with raw
                K/V vectors for every prefill token (codeword + N(0, 0.1^2))

Paged caches (``paged_cache``) hold the same codes in fixed-size pages of a
per-head pool, in a seeded random page order, with a block table per
request; unused table entries hold an out-of-range page id.

Draw order per workload: k codebook, v codebook, k codes, v codes, q, then
request order (ragged), then encode data.  Codebooks and q are fp16 drawn
from N(0, 1); codes are uniform over 0..255.  Cache positions at or beyond
a request's length hold random codes too, so that a kernel that reads past
``lens`` gives a wrong answer instead of a lucky zero.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    max_len: int
    head_dim: int = 128
    n_sub: int = 4
    n_codes: int = 256
    chunk: int = 0                      # 0: the library picks
    lens_mix: Optional[tuple] = None    # ((count, length), ...) for ragged batches
    encode_sigma: Optional[float] = None
    prefill_encode: bool = False        # raw K/V for every valid token

    @property
    def sub_dim(self) -> int:
        return self.head_dim // self.n_sub

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    1: Workload("tiny", batch=1, n_q_heads=8, n_kv_heads=8, max_len=512,
                n_sub=4, encode_sigma=0.05),
    2: Workload("page-sizing", batch=4, n_q_heads=32, n_kv_heads=32,
                max_len=2048, n_sub=4),
    3: Workload("gqa", batch=8, n_q_heads=64, n_kv_heads=8, max_len=8192,
                n_sub=8),
    4: Workload("long-splitk", batch=1, n_q_heads=64, n_kv_heads=8,
                max_len=131072, n_sub=4, chunk=2048),
    5: Workload("ragged", batch=64, n_q_heads=32, n_kv_heads=32,
                max_len=4096, n_sub=4, lens_mix=((45, 512), (19, 4096)),
                encode_sigma=0.1, prefill_encode=True),
}


def rng_for(wid: int, replica: int = 0) -> np.random.Generator:
    """Generator for workload ``wid``; replica 0 is the canonical input."""
    if replica == 0:
        return np.random.default_rng(1000 + wid)
    return np.random.default_rng([1000 + wid, replica])


def _normal_f16(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float16)


def codebooks(rng, n_heads, n_sub, n_codes, sub_dim):
    """fp16 [H][M][K][ds] codebook, entries N(0, 1)."""
    return _normal_f16(rng, (n_heads, n_sub, n_codes, sub_dim))


def codebooks_fp8(rng, n_heads, n_sub, n_codes, sub_dim):
    """uint8 [H][M][K][ds]: entries N(0, 1) rounded to the nearest OCP FP8
    E4M3 value (ties to even, by torch's conversion), as bytes."""
    import torch
    x = rng.standard_normal((n_heads, n_sub, n_codes, sub_dim), dtype=np.float32)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def codes(rng, batch, n_heads, max_len, n_sub, n_codes=256):
    """uint8 [B][H][Lmax][M], uniform."""
    return rng.integers(0, n_codes, size=(batch, n_heads, max_len, n_sub), dtype=np.uint8)


def noisy_codewords(rng, cb, n_vec, sigma):
    """Encode inputs: for each of ``n_vec`` tokens and each head, draw one
    codeword index per subspace, lay the chosen codewords side by side and
    add iid N(0, sigma^2) per dimension; round to fp16.

    Returns (x fp16 [n_vec][H][D], src uint8 [n_vec][H][M]).  ``src`` is the
    index the noise was added to, kept to check the encoder with.
    """
    H, M, K, ds = cb.shape
    src = rng.integers(0, K, size=(n_vec, H, M), dtype=np.uint8)
    x = np.empty((n_vec, H, M * ds), dtype=np.float16)
    step = max(1, (1 << 22) // max(1, H * M * ds))
    for lo in range(0, n_vec, step):
        hi = min(n_vec, lo + step)
        s = src[lo:hi].astype(np.intp)
        picked = cb[np.arange(H)[None, :, None], np.arange(M)[None, None, :], s]   # [n,H,M,ds]
        noise = rng.standard_normal((hi - lo, H, M * ds), dtype=np.float32) * np.float32(sigma)
        x[lo:hi] = (picked.reshape(hi - lo, H, M * ds).astype(np.float32) + noise).astype(np.float16)
    return x, src


def ragged_lens(rng, mix):
    """A seeded permutation of the request lengths in ``mix``."""
    lens = np.concatenate([np.full(n, l, dtype=np.int32) for n, l in mix])
    return lens[rng.permutation(lens.size)].astype(np.int32)


def make_inputs(w: Workload, rng: np.random.Generator, *, with_encode=True):
    """All inputs of one decode step of workload ``w`` as numpy arrays."""
    B, Hq, Hkv, L = w.batch, w.n_q_heads, w.n_kv_heads, w.max_len
    M, K, ds, D = w.n_sub, w.n_codes, w.sub_dim, w.head_dim
    out = {}
    out["k_cb"] = codebooks(rng, Hkv, M, K, ds)
    out["v_cb"] = codebooks(rng, Hkv, M, K, ds)
    out["k_codes"] = codes(rng, B, Hkv, L, M, K)
    out["v_codes"] = codes(rng, B, Hkv, L, M, K)
    out["q"] = _normal_f16(rng, (B, Hq, D))
    if w.lens_mix is not None:
        out["lens"] = ragged_lens(rng, w.lens_mix)
    else:
        out["lens"] = np.full(B, L, dtype=np.int32)
    if with_encode and w.encode_sigma is not None:
        if w.prefill_encode:
            n_tok = int(out["lens"].sum())
            out["x_k"], out["src_k"] = noisy_codewords(rng, out["k_cb"], n_tok, w.encode_sigma)
            out["x_v"], out["src_v"] = noisy_codewords(rng, out["v_cb"], n_tok, w.encode_sigma)
            out["slots"] = prefill_slots(out["lens"], Hkv, L)
        else:
            out["x_k"], out["src_k"] = noisy_codewords(rng, out["k_cb"], B, w.encode_sigma)
            out["x_v"], out["src_v"] = noisy_codewords(rng, out["v_cb"], B, w.encode_sigma)
    return out


def step_tokens(rng, k_cb, v_cb, batch, sigma=0.05):
    """The K and V of the next token of every request for one decode step:
    fp16 [B][Hkv][D] each, a random codeword per subspace plus
    N(0, sigma^2) noise (as ``noisy_codewords``).  Returns
    (x_k, src_k, x_v, src_v)."""
    x_k, src_k = noisy_codewords(rng, k_cb, batch, sigma)
    x_v, src_v = noisy_codewords(rng, v_cb, batch, sigma)
    return x_k, src_k, x_v, src_v


def workload_inputs(wid: int, replica: int = 0, *, with_encode=True):
    return make_inputs(WORKLOADS[wid], rng_for(wid, replica), with_encode=with_encode)


def prefill_slots(lens, n_kv_heads, max_len):
    """Token slot of every prefill token in a [B][Hkv][Lmax][M] code cache:
    token t of request b lands at slot b*Hkv*Lmax + t (the head offset is
    added through the head stride).  Tokens are packed request by request."""
    parts = [np.arange(int(l), dtype=np.int64) + np.int64(b) * n_kv_heads * max_len
             for b, l in enumerate(lens)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def random_case(seed, *, batch, n_q_heads, n_kv_heads, max_len, n_sub=4,
                head_dim=128, n_codes=256, lens=None):
    """A small seeded case with arbitrary shape, for parity sweeps."""
    rng = np.random.default_rng(seed)
    w = Workload("random", batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                 max_len=max_len, head_dim=head_dim, n_sub=n_sub, n_codes=n_codes)
    inp = make_inputs(w, rng, with_encode=False)
    if lens is not None:
        inp["lens"] = np.asarray(lens, dtype=np.int32)
    return w, inp


def paged_cache(rng, k_codes, v_codes, lens, page_tokens, *, spare_pages=3, fill=-1):
    """Scatter dense caches [B, Hkv, Lmax, M] into paged pools.

    Request b needs ceil(lens[b] / P) pages.  Those pages are taken in a
    seeded random order from a pool of (pages needed + spare_pages) pages;
    page j of request b (tokens j*P .. j*P + P - 1) is copied into pool slots
    page*P .. page*P + P - 1 of every KV head.  Pages nobody uses hold random
    codes.  Table entries past a request's pages hold ``fill``.

    Returns (k_pool, v_pool, block_table, n_pages) with pools uint8
    [Hkv, n_pages * P, M] and block_table int32 [B, Lmax // P].
    """
    B, Hkv, Lmax, M = k_codes.shape
    P = int(page_tokens)
    assert Lmax % P == 0
    max_pages = Lmax // P
    need = [-(-int(min(max(int(x), 0), Lmax)) // P) for x in lens]
    n_pages = sum(need) + int(spare_pages)
    order = rng.permutation(n_pages)
    k_pool = rng.integers(0, 256, size=(Hkv, n_pages * P, M), dtype=np.uint8)
    v_pool = rng.integers(0, 256, size=(Hkv, n_pages * P, M), dtype=np.uint8)
    table = np.full((B, max_pages), fill, dtype=np.int32)
    nxt = 0
    for b in range(B):
        for j in range(need[b]):
            page = int(order[nxt])
            nxt += 1
            table[b, j] = page
            k_pool[:, page * P:(page + 1) * P] = k_codes[b, :, j * P:(j + 1) * P]
            v_pool[:, page * P:(page + 1) * P] = v_codes[b, :, j * P:(j + 1) * P]
    return k_pool, v_pool, table, n_pages


def kmeans_case(rng, n_vec, n_heads, n_sub, *, n_codes=256, head_dim=128, sigma=0.05,
                init_sigma=0.3, n_used=None):
    """Inputs for codebook learning: a generating codebook (fp16 N(0,1)), a
    sample of ``n_vec`` vectors per head drawn around its codewords (R12's
    "codeword + noise", only the first ``n_used`` codewords of each segment
    when given), and a starting codebook = generating codebook + iid
    N(0, init_sigma^2), rounded to fp16.

    Returns dict(x fp16 [N, H, D], src uint8 [N, H, M], cb_true, cb_init
    fp16 [H, M, K, D/M])."""
    ds = head_dim // n_sub
    cb_true = codebooks(rng, n_heads, n_sub, n_codes, ds)
    x, src = noisy_codewords(rng, cb_true, n_vec, sigma)
    if n_used is not None:
        src = (src.astype(np.int64) % int(n_used)).astype(np.uint8)
        picked = cb_true[np.arange(n_heads)[None, :, None], np.arange(n_sub)[None, None, :],
                         src.astype(np.intp)]
        noise = rng.standard_normal((n_vec, n_heads, head_dim), dtype=np.float32) * np.float32(sigma)
        x = (picked.reshape(n_vec, n_heads, head_dim).astype(np.float32) + noise).astype(np.float16)
    cb_init = (cb_true.astype(np.float32)
               + rng.standard_normal(cb_true.shape, dtype=np.float32) * np.float32(init_sigma)
               ).astype(np.float16)
    return {"x": x, "src": src, "cb_true": cb_true, "cb_init": cb_init}
