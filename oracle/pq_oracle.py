"""CPU oracle for PQ-KV decode attention and PQ encode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it.

It computes the plain definitions, slowly and in float64:

* Product quantization of a cached vector (AQPIM page, section 3.1): the
  D-dimensional vector is cut into M equal contiguous segments; segment m is
  stored as the index of its nearest codeword in codebook m; decoding looks
  the indices up and lays the M codewords side by side.
* Codebooks are kept per layer and per head (AQPIM page, section 3.2 (1));
  under grouped-query attention a KV head's codebooks serve all the query
  heads of its group (memory-wall chapter, section 1.4.3 (1)).  Query head h
  reads KV head h // G with G = Hq / Hkv.
* Decode attention "the long way" (AQPIM page, section 4): rebuild every
  cached K and V from its indices, then textbook attention for one query
  token: s_t = scale * q . K_t over the t < lens[b] cached tokens, a
  numerically stable softmax, out = sum_t p_t V_t.
* Chunked softmax (PAM page, section 2.2.3 (1); memory-wall chapter,
  section 1.4.3 (5.1)): each chunk of tokens keeps its own max m_c, its sum
  l_c = sum exp(s - m_c) and its unnormalised output o_c = sum exp(s - m_c)V;
  a reduction rescales every chunk by exp(m_c - max_c m_c) and divides.
* Encode (AQPIM page, sections 3.1 and 5.2 (2)): per segment, the index of
  the codeword at the smallest squared Euclidean distance; the lowest index
  wins a tie.
* Codebook learning (AQPIM page, section 3.2 (2): codebooks fitted online
  to the first vectors of a sequence; section 5.2 (1): a fast K-means on a
  small sample such as 32 vectors; section 6.1 (3): a few K-means updates
  every so many tokens): Lloyd's algorithm per head and segment.  Each
  iteration assigns every vector's segment to its nearest codeword (the
  encode above), then moves every codeword that received vectors to their
  mean -- the exact sum divided by the count in float64, rounded to the fp16
  codebook; a codeword that received none keeps its value.
* FP8 codebooks (AQPIM page, section 4.2: codebooks kept as a low-precision
  float such as FP8): bytes of the OCP FP8 E4M3 format are decoded exactly
  to float64, and attention and encode then run on those codeword values.
* Paged code cache (AQPIM page, section 5.1 (4): the index cache managed in
  pages as in vLLM; PAM page, section 2.2.2 (2): paged KV management with a
  global block table of where each token lives): token t of request b sits
  in page block_table[b][t // P] at offset t % P.  Attention over it is the
  same definition as above with the codes read through the table.

Readings where the pages are silent (the scale 1/sqrt(D), lens = 0 gives a
zero output, the head -> KV head map) are listed with the rest of the design
notes of this repository.

Parity pins: every function here is checked against facts that do not come
from this file -- the pages' printed sizes, algebraic identities, closed
forms on tiny inputs, torch's CPU scaled-dot-product attention and scipy's
distance routine -- in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np


def default_scale(head_dim: int) -> float:
    """Softmax temperature 1/sqrt(D) (the pages do not state one)."""
    return 1.0 / math.sqrt(head_dim)


def fp8_e4m3_to_float64(b) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 bytes (AQPIM page, section 4.2: codebooks
    stored as FP8), from the format's definition: bit 7 the sign s, bits 6..3
    the exponent e (bias 7), bits 2..0 the mantissa f;
      e > 0:  (-1)^s (1 + f/8) 2^(e - 7)
      e = 0:  (-1)^s (f/8) 2^(1 - 7)          (subnormal; f = 0 is a signed zero)
      e = 15 and f = 7: NaN (the format has no infinities).
    b: uint8 array of any shape; returns float64 of the same shape."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 0xF
    f = b & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * (1.0 + f / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (f / 8.0) * 2.0 ** (1 - 7)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (f == 7), np.nan, out)


def reconstruct(codes: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """Rebuild vectors from their PQ indices (AQPIM page, section 3.1).

    codes: uint8 [..., M]  (indices of one KV head)
    cb:    [M, K, ds]      (that head's codebook)
    returns float64 [..., M*ds]: the M looked-up codewords side by side.
    """
    M = cb.shape[0]
    cb64 = cb.astype(np.float64)
    segments = [cb64[m][codes[..., m].astype(np.intp)] for m in range(M)]
    return np.concatenate(segments, axis=-1)


def _valid_len(lens, b, max_len):
    return int(min(max(int(lens[b]), 0), max_len))


def attention_weights(q_row: np.ndarray, k_hat: np.ndarray, scale: float) -> np.ndarray:
    """Softmax over t of scale * q . K_t, computed stably (max subtracted)."""
    s = scale * (k_hat @ q_row.astype(np.float64))
    s = s - s.max()
    e = np.exp(s)
    return e / e.sum()


def decode_attention(q, k_codes, v_codes, k_cb, v_cb, lens, scale=None):
    """Single-token decode attention over a PQ-coded KV cache, the plain way.

    q        fp16 [B, Hq, D]
    k_codes  uint8 [B, Hkv, Lmax, M]     v_codes the same
    k_cb     fp16 [Hkv, M, K, D/M]       v_cb the same
    lens     int [B]; tokens t < lens[b] are attended (clamped to [0, Lmax])
    returns  float64 [B, Hq, D]; a request with no tokens gives zeros.
    """
    B, Hq, D = q.shape
    Hkv, Lmax = k_codes.shape[1], k_codes.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(D)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = _valid_len(lens, b, Lmax)
        if L == 0:
            continue
        for g in range(Hkv):
            k_hat = reconstruct(k_codes[b, g, :L], k_cb[g])
            v_hat = reconstruct(v_codes[b, g, :L], v_cb[g])
            for h in range(g * G, (g + 1) * G):
                p = attention_weights(q[b, h], k_hat, scale)
                out[b, h] = p @ v_hat
    return out


def chunk_partials(q, k_codes, v_codes, k_cb, v_cb, lens, chunk, scale=None, n_chunks=None):
    """Per-chunk softmax statistics (PAM page, section 2.2.3 (1)).

    Chunk c covers tokens [c*chunk, (c+1)*chunk) intersected with
    [0, lens[b]).  Returns float64 arrays
      m [B, Hq, C]    max scaled score in the chunk (-inf if empty)
      l [B, Hq, C]    sum_t exp(s_t - m)            (0 if empty)
      o [B, Hq, C, D] sum_t exp(s_t - m) V_t        (0 if empty)
    with C = ceil(Lmax / chunk) unless given.
    """
    B, Hq, D = q.shape
    Hkv, Lmax = k_codes.shape[1], k_codes.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(D)
    C = n_chunks if n_chunks is not None else max(1, -(-Lmax // chunk))
    m = np.full((B, Hq, C), -np.inf)
    l = np.zeros((B, Hq, C))
    o = np.zeros((B, Hq, C, D))
    for b in range(B):
        L = _valid_len(lens, b, Lmax)
        for g in range(Hkv):
            for c in range(C):
                lo, hi = c * chunk, min((c + 1) * chunk, L)
                if lo >= hi:
                    continue
                k_hat = reconstruct(k_codes[b, g, lo:hi], k_cb[g])
                v_hat = reconstruct(v_codes[b, g, lo:hi], v_cb[g])
                for h in range(g * G, (g + 1) * G):
                    s = scale * (k_hat @ q[b, h].astype(np.float64))
                    mc = s.max()
                    e = np.exp(s - mc)
                    m[b, h, c] = mc
                    l[b, h, c] = e.sum()
                    o[b, h, c] = e @ v_hat
    return m, l, o


def merge_partials(m, l, o):
    """Merge chunk statistics into the final output (PAM page, section
    2.2.3 (1) and (3); the rescaling of the memory-wall chapter's online
    softmax, section 1.4.3 (5.1)).

    m, l: [..., C];  o: [..., C, D].  Empty chunks carry m = -inf, l = 0.
    out = sum_c w_c o_c / sum_c w_c l_c  with  w_c = exp(m_c - max_c m_c);
    zeros where every chunk is empty.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    m_star = m.max(axis=-1, keepdims=True)
    finite = np.isfinite(m_star)
    safe = np.where(finite, m_star, 0.0)
    w = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
    num = (w[..., None] * o).sum(axis=-2)
    den = (w * l).sum(axis=-1)
    out = np.zeros(num.shape)
    ok = den > 0
    out[ok] = num[ok] / den[ok][..., None]
    return out


def encode(x, cb, block=1024):
    """Nearest-codeword encode (AQPIM page, sections 3.1 and 5.2 (2)).

    x   fp16 [N, H, D]
    cb  fp16 [H, M, K, ds]
    returns uint8 [N, H, M]: per (vector, head, segment) the index k that
    minimises the squared Euclidean distance sum_j (x_j - C[k]_j)^2, taken in
    float64 from the exact fp16 values; the lowest index wins a tie (numpy
    argmin).
    """
    N, H, D = x.shape
    _, M, K, ds = cb.shape
    codes = np.empty((N, H, M), dtype=np.uint8)
    cb64 = cb.astype(np.float64)
    for lo in range(0, N, block):
        hi = min(N, lo + block)
        xs = x[lo:hi].astype(np.float64).reshape(hi - lo, H, M, ds)
        for h in range(H):
            for m in range(M):
                diff = xs[:, h, m, None, :] - cb64[h, m][None, :, :]     # [n, K, ds]
                d2 = (diff * diff).sum(axis=-1)
                codes[lo:hi, h, m] = np.argmin(d2, axis=1).astype(np.uint8)
    return codes


def paged_slots(block_table, lens, b, page_tokens, max_len):
    """Pool slots of tokens t < lens[b] of request b (PAM page, section
    2.2.2 (2): a block table records where each token lives).

    block_table int [B, max_pages]; page_tokens P.  Token t lives in page
    block_table[b, t // P] at offset t % P, i.e. pool slot
    block_table[b, t // P] * P + t % P.  Table entries past the request's
    last token are never read.
    """
    L = _valid_len(lens, b, max_len)
    t = np.arange(L)
    pages = np.asarray(block_table[b], dtype=np.int64)[t // page_tokens]
    return pages * page_tokens + t % page_tokens


def decode_attention_paged(q, k_pool, v_pool, k_cb, v_cb, block_table, lens, page_tokens,
                           scale=None):
    """Single-token decode attention over a paged PQ code cache (AQPIM page,
    sections 4 and 5.1 (4); PAM page, section 2.2.2 (2)).

    q            fp16 [B, Hq, D]
    k_pool       uint8 [Hkv, n_pages * P, M]: KV head g's pages side by side,
                 page p holding slots p*P .. p*P + P - 1      (v_pool the same)
    k_cb, v_cb   fp16 [Hkv, M, K, D/M]
    block_table  int [B, max_pages]: page of each P-token block of request b
    lens         int [B], clamped to [0, max_pages * P]
    returns float64 [B, Hq, D]: softmax_t(scale q . K_t) V_t over t < lens[b],
    K_t and V_t rebuilt from the codes at token t's slot; zeros for lens 0.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[0]
    G = Hq // Hkv
    max_len = block_table.shape[1] * page_tokens
    if scale is None:
        scale = default_scale(D)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        slots = paged_slots(block_table, lens, b, page_tokens, max_len)
        if slots.size == 0:
            continue
        for g in range(Hkv):
            k_hat = reconstruct(k_pool[g, slots], k_cb[g])
            v_hat = reconstruct(v_pool[g, slots], v_cb[g])
            for h in range(g * G, (g + 1) * G):
                p = attention_weights(q[b, h], k_hat, scale)
                out[b, h] = p @ v_hat
    return out


def codebook_update(x, codes, cb):
    """The update step of one Lloyd iteration for every head and segment
    (AQPIM page, sections 3.2 (2), 5.2 (1) and 6.1 (3)).

    x      fp16 [N, H, D]    the sample vectors
    codes  uint8 [N, H, M]   their current assignment (nearest codewords)
    cb     fp16 [H, M, K, ds]
    returns (new codebook fp16 [H, M, K, ds], counts int64 [H, M, K]):
    codeword k of (h, m) becomes the mean of the segments assigned to it,
    math.fsum (the exactly rounded sum) divided by the count in float64 and
    rounded to fp16; a codeword with no segment keeps its value.
    """
    N, H, D = x.shape
    _, M, K, ds = cb.shape
    new = cb.copy()
    counts = np.zeros((H, M, K), dtype=np.int64)
    x64 = x.astype(np.float64)
    for h in range(H):
        for m in range(M):
            seg = x64[:, h, m * ds:(m + 1) * ds]
            c = codes[:, h, m].astype(np.intp)
            for k in np.unique(c):
                members = seg[c == k]
                n = members.shape[0]
                counts[h, m, k] = n
                mean = np.array([math.fsum(members[:, j]) / n for j in range(ds)])
                new[h, m, k] = mean.astype(np.float16)
    return new, counts


def kmeans(x, cb_init, n_iter):
    """n_iter Lloyd iterations from cb_init (assign with encode, then
    codebook_update), then the assignment to the final codebook.

    Returns (codebook fp16 [H, M, K, ds], codes uint8 [N, H, M])."""
    cb = cb_init.copy()
    for _ in range(int(n_iter)):
        cb, _ = codebook_update(x, encode(x, cb), cb)
    return cb, encode(x, cb)
