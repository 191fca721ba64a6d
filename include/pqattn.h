/*
 * pqattn.h -- C ABI of the PQ-KV decode-attention library for AMD MI355X
 * (gfx950).
 *
 * What it computes.  A KV cache whose every cached K and V vector of
 * dimension D is stored as M one-byte indices, one per contiguous segment of
 * D/M dimensions, into per-head codebooks of K = 256 codewords (product
 * quantization: AQPIM page, section 3.1; per-layer and per-head codebooks,
 * section 3.2 (1)).  Attention for one new query token is scored by looking
 * the query's partial dot products with the codewords up instead of
 * rebuilding K (AQPIM page, section 4.1; the fused kernel of section
 * 5.1 (3)), the softmax runs in token chunks whose (max, sum, partial output)
 * a reduction merges (PAM page, section 2.2.3 (1) and (3)), and new vectors
 * are encoded by nearest codeword (AQPIM page, section 5.2 (2)).
 *
 * Conventions for every call:
 *  - Array pointers are DEVICE pointers owned by the caller; descriptors are
 *    host pointers read during the call only.  The library keeps no pointer
 *    after a call returns and allocates no device memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream) and never synchronise.  Results are ready when the stream is.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    non-zero pq_status means nothing was launched.  A launch the HIP runtime
 *    refuses returns PQ_ERR_HIP.  Values inside device arrays cannot be
 *    checked without a sync: lens[] is clamped to [0, max_len] on the
 *    device, and every uint8 code is a valid index when K = 256.
 *  - Two calls that run at the same time need their own workspaces.
 *  - Supported shapes: head_dim = 128, n_codes = 256, n_sub in {4, 8} (so
 *    segments of 32 or 16 dims), n_q_heads / n_kv_heads in {1, 2, 4, 8},
 *    max_len a multiple of 16, batch and the chunk count C each at most
 *    65535; q, code and codebook pointers 16-byte aligned.  Other valid
 *    shapes return PQ_ERR_UNSUPPORTED.
 */
#ifndef PQATTN_H
#define PQATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pq_status {
  PQ_OK = 0,
  PQ_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PQ_ERR_SHAPE = 2,       /* descriptor fields inconsistent or out of range     */
  PQ_ERR_UNSUPPORTED = 3, /* consistent, but a shape this library does not build */
  PQ_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned         */
  PQ_ERR_HIP = 5,         /* the HIP runtime refused a launch                   */
  PQ_ERR_ALIGN = 6        /* an array pointer is not 16-byte aligned            */
} pq_status;

/* Shape of one decode step of one layer. */
typedef struct pq_attn_desc {
  int32_t batch;       /* B, >= 1                                                */
  int32_t n_q_heads;   /* Hq; query head h reads KV head h / (Hq / Hkv)          */
  int32_t n_kv_heads;  /* Hkv; Hq % Hkv == 0                                     */
  int32_t head_dim;    /* D                                                      */
  int32_t n_sub;       /* M segments per vector, D % M == 0                      */
  int32_t n_codes;     /* K codewords per segment codebook                       */
  int32_t max_len;     /* Lmax: cache capacity in tokens per (b, kv head)        */
  int32_t chunk;       /* T tokens per softmax chunk; 0 lets the library pick    */
  float   scale;       /* score scale, normally 1/sqrt(D); must be finite, > 0   */
} pq_attn_desc;

/* Number of chunks C = ceil(max_len / T) the call will use (T resolved when
 * desc->chunk is 0), or -1 if the descriptor is invalid or unsupported. */
int32_t pq_attn_num_chunks(const pq_attn_desc* desc);

/* Workspace pq_attn_decode needs: 0 when C == 1, else room for the chunk
 * statistics of every (b, query head), B*Hq*C*(D+2)*4 bytes rounded up to
 * 256-byte blocks.  Returns 0 for an invalid descriptor as well. */
size_t pq_attn_workspace_bytes(const pq_attn_desc* desc);

/* One decode step: out[b][h] = softmax_t(scale * q[b][h] . K_t) V_t over the
 * tokens t < lens[b] of KV head h / G, K_t and V_t being the codewords the
 * cache's indices name, laid side by side (AQPIM page, sections 3.1 and 4.1;
 * chunked softmax and merge per PAM page, section 2.2.3).
 *
 *  q        fp16  [B][Hq][D]
 *  k_codes  uint8 [B][Hkv][max_len][M]  token-major, M bytes per token
 *  v_codes  uint8 [B][Hkv][max_len][M]
 *  k_cb     fp16  [Hkv][M][K][D/M]      K codebooks
 *  v_cb     fp16  [Hkv][M][K][D/M]      V codebooks
 *  lens     int32 [B]                   tokens attended per request
 *  out      fp32  [B][Hq][D]            written; a request with lens 0 gets 0
 *  workspace, workspace_bytes           at least pq_attn_workspace_bytes();
 *                                       16-byte aligned; may be NULL when
 *                                       that is 0.  Contents on entry do
 *                                       not matter.
 * Launches the score kernel and, when C > 1, the merge kernel. */
pq_status pq_attn_decode(const pq_attn_desc* desc, const void* q,
                         const uint8_t* k_codes, const uint8_t* v_codes,
                         const void* k_cb, const void* v_cb, const int32_t* lens,
                         float* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* The score kernel alone: per (b, query head, chunk c) the statistics of
 * tokens [c*T, (c+1)*T) intersected with [0, lens[b]) (PAM page, section
 * 2.2.3 (1)):
 *  part_m  fp32 [B][Hq][C]     max_t s_t (natural-log units), -inf if empty
 *  part_l  fp32 [B][Hq][C]     sum_t exp(s_t - m), 0 if empty
 *  part_o  fp32 [B][Hq][C][D]  sum_t exp(s_t - m) V_t, unnormalised, 0 if empty
 * with s_t = scale * q . K_t.  Other arguments as for pq_attn_decode. */
pq_status pq_attn_partials(const pq_attn_desc* desc, const void* q,
                           const uint8_t* k_codes, const uint8_t* v_codes,
                           const void* k_cb, const void* v_cb, const int32_t* lens,
                           float* part_m, float* part_l, float* part_o, void* stream);

/* pq_attn_partials for kernel timing: start_event and stop_event (hipEvent_t
 * handles created by the caller, either may be NULL) are stamped by the
 * runtime at the score kernel's own start and end (hipExtLaunchKernel), so
 * hipEventElapsedTime between them is the kernel's execution time.
 * Everything else is exactly pq_attn_partials. */
pq_status pq_attn_partials_timed(const pq_attn_desc* desc, const void* q,
                                 const uint8_t* k_codes, const uint8_t* v_codes,
                                 const void* k_cb, const void* v_cb, const int32_t* lens,
                                 float* part_m, float* part_l, float* part_o, void* stream,
                                 void* start_event, void* stop_event);

/* Workspace pq_attn_decode_step needs: 0 when C == 1, else the chunk
 * records of pq_attn_workspace_bytes() followed by one 32-bit arrival counter
 * per (b, KV head), rounded up to 256-byte blocks.  0 for an invalid
 * descriptor as well. */
size_t pq_attn_step_workspace_bytes(const pq_attn_desc* desc);

/* One decode step with the new token appended, normally in one kernel
 * launch (see the exception below).  For
 * every request b with lens[b] >= 1 and every KV head g, the new token's K
 * and V (k_new[b][g], v_new[b][g]) are encoded by nearest codeword -- the
 * same decisions pq_encode takes (AQPIM page, sections 3.1 and 5.2 (2)) --
 * and written at slot t = lens[b] - 1 of k_codes and v_codes; out[b][h] is
 * then what pq_attn_decode gives over the cache that now holds the token
 * (scores from the lookup table, AQPIM page, section 4.1; chunked softmax
 * and merge, PAM page, section 2.2.3).
 *
 *  k_new, v_new      fp16  [B][Hkv][D], 16-byte aligned
 *  k_codes, v_codes  uint8 [B][Hkv][max_len][M]; only the new token's slots
 *                    are written
 *  lens              int32 [B]; counts the new token.  lens[b] = 0: nothing
 *                    is written for b and its output is 0.  Clamped to
 *                    [0, max_len] like pq_attn_decode's.
 *  workspace         at least pq_attn_step_workspace_bytes(); may be NULL
 *                    when that is 0.  When it is not 0 the buffer must be
 *                    zero-filled before its first use (e.g. hipMemsetAsync);
 *                    every call leaves it ready for the next call with
 *                    the SAME descriptor (its counters back at zero), and
 *                    a call that returns a non-zero status does not touch
 *                    it.  A step workspace is tied to one descriptor: the
 *                    counters sit after the chunk records, at an offset
 *                    that depends on B, Hq and C, so a step of another
 *                    shape would read old record bytes as counters and
 *                    never merge.  Zero it again (or take a fresh one)
 *                    before using it with another descriptor.  Two calls
 *                    that may run at the same time need their own
 *                    workspaces.
 * Other arguments as for pq_attn_decode.  The workgroup whose chunk holds
 * the new token encodes it; with C > 1 the last workgroup of each (b, KV
 * head) to finish merges the chunk records into out.  Exception: with one
 * query head per KV head and at least 1024 (request, KV head) pairs, the
 * encode kernel writes the new codes first and the request-batched score
 * kernel (then, with C > 1, the merge kernel) follows -- 2 or 3 launches,
 * same results, the counters untouched. */
pq_status pq_attn_decode_step(const pq_attn_desc* desc, const void* q, const void* k_new,
                              const void* v_new, uint8_t* k_codes, uint8_t* v_codes,
                              const void* k_cb, const void* v_cb, const int32_t* lens, float* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* pq_attn_decode_step for kernel timing: start_event and stop_event
 * (hipEvent_t, either may be NULL) are stamped at the kernel's own start and
 * end, as in pq_attn_partials_timed. */
pq_status pq_attn_decode_step_timed(const pq_attn_desc* desc, const void* q, const void* k_new,
                                    const void* v_new, uint8_t* k_codes, uint8_t* v_codes,
                                    const void* k_cb, const void* v_cb, const int32_t* lens,
                                    float* out, void* workspace, size_t workspace_bytes,
                                    void* stream, void* start_event, void* stop_event);

/* A paged code cache (AQPIM page, section 5.1 (4): the index cache kept in
 * pages that grow and are reclaimed as in vLLM; PAM page, section 2.2.2 (2):
 * a global block table records where every token lives).  Each of the K and
 * V caches is a pool of pages per KV head:
 *    pool  uint8 [Hkv][n_pages][page_tokens][M]
 * and token t of request b lives in page block_table[b][t / page_tokens] at
 * offset t % page_tokens.  Pages are shared by all KV heads of a request (one
 * table row per request) and may be shared between requests (a common
 * prefix).  In the pool of KV head g, token t's codes sit at slot
 *    s = block_table[b][t / page_tokens] * page_tokens + t % page_tokens,
 * so pq_encode with those slots, codes_stride_slot = M and codes_stride_head
 * = n_pages * page_tokens * M writes a prefill straight into the pages. */
typedef struct pq_page_table {
  const int32_t* block_table; /* DEVICE int32 [B][max_pages]; entries for the
                                 blocks below lens[b] must name pages in
                                 [0, n_pages); later entries are never used.
                                 An out-of-range entry is clamped into the
                                 pool: no memory outside it is touched, but
                                 the result is unspecified.                   */
  int32_t page_tokens;        /* P: a power of two in [16, 65536]            */
  int32_t max_pages;          /* table row length; the attention descriptor's
                                 max_len must equal max_pages * page_tokens  */
  int32_t n_pages;            /* pages per KV head in each pool, >= 1; one
                                 KV head's pool, n_pages * P * M bytes, must
                                 stay under 2 GiB (PQ_ERR_UNSUPPORTED)       */
} pq_page_table;

/* pq_attn_decode over a paged cache: out[b][h] is exactly what pq_attn_decode
 * gives for a dense cache holding, at token t of (b, g), the codes the table
 * names.  k_pool and v_pool are uint8 [Hkv][n_pages][P][M], 16-byte aligned;
 * pages is a host pointer read during the call.  Workspace as for
 * pq_attn_decode with the same descriptor.  A NULL pages or block_table is
 * PQ_ERR_NULL; a page size or table shape outside the rules above is
 * PQ_ERR_SHAPE. */
pq_status pq_attn_decode_paged(const pq_attn_desc* desc, const pq_page_table* pages,
                               const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                               const void* k_cb, const void* v_cb, const int32_t* lens, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* pq_attn_partials over a paged cache: the chunk records of pq_attn_partials
 * for the cache the table describes (arguments as for pq_attn_decode_paged
 * and pq_attn_partials).  With a table that names only some of a request's
 * pages and lens counting past them, records of different calls merge with
 * pq_attn_reduce like token shards (PAM page, section 2.2.3 (2)). */
pq_status pq_attn_partials_paged(const pq_attn_desc* desc, const pq_page_table* pages,
                                 const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                                 const void* k_cb, const void* v_cb, const int32_t* lens,
                                 float* part_m, float* part_l, float* part_o, void* stream);

/* pq_attn_decode_step over a paged cache: the new token's K and V codes go to
 * the slot of token lens[b] - 1 (its page must already be in the table), and
 * out is pq_attn_decode_paged's over the cache that now holds the token.
 * Workspace (zero-filled before first use) as for pq_attn_decode_step. */
pq_status pq_attn_decode_step_paged(const pq_attn_desc* desc, const pq_page_table* pages,
                                    const void* q, const void* k_new, const void* v_new,
                                    uint8_t* k_pool, uint8_t* v_pool, const void* k_cb,
                                    const void* v_cb, const int32_t* lens, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* pq_attn_decode_step_paged with kernel-stamped events, as in
 * pq_attn_partials_timed. */
pq_status pq_attn_decode_step_paged_timed(const pq_attn_desc* desc, const pq_page_table* pages,
                                          const void* q, const void* k_new, const void* v_new,
                                          uint8_t* k_pool, uint8_t* v_pool, const void* k_cb,
                                          const void* v_cb, const int32_t* lens, float* out,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* start_event, void* stop_event);

/* Merge chunk statistics (PAM page, section 2.2.3 (3); the rescaling of the
 * memory-wall chapter's online softmax, section 1.4.3 (5.1)):
 *   out[r] = sum_c w_c o[r][c] / sum_c w_c l[r][c],  w_c = exp(m[r][c] - max_c m[r][c])
 * for n_rows rows (a row is one (b, query head)), 0 where every chunk is
 * empty (m = -inf, l = 0).  Partials may come from several pq_attn_partials
 * calls over disjoint token ranges, laid side by side along the chunk axis.
 *  part_m, part_l  fp32 [n_rows][n_chunks]
 *  part_o          fp32 [n_rows][n_chunks][head_dim]
 *  out             fp32 [n_rows][head_dim]
 * head_dim must be 128; n_chunks >= 1. */
pq_status pq_attn_reduce(int64_t n_rows, int32_t n_chunks, int32_t head_dim,
                         const float* part_m, const float* part_l, const float* part_o,
                         float* out, void* stream);

/* pq_attn_reduce with the rescaling weights exp(m_c - m*) taken the way the
 * PAM page's reduction units take them (section 3.2.2 (1): a 6th-order
 * polynomial instead of an exponential unit): 2^x = 2^n * P6(f), x = n + f,
 * n = floor(x), P6 a degree-6 minimax fit of 2^f on [0, 1) (relative error
 * at most 8.4e-8 in fp32; exp2_poly_fit.py derives it); weights below
 * 2^-126 count as 0.  Arguments, checks and layouts as for pq_attn_reduce;
 * results agree with it to about 1e-7 relative. */
pq_status pq_attn_reduce_polyexp(int64_t n_rows, int32_t n_chunks, int32_t head_dim,
                                 const float* part_m, const float* part_l, const float* part_o,
                                 float* out, void* stream);

/* Shape and strides of one encode call. */
typedef struct pq_encode_desc {
  int64_t n_vec;              /* N vectors per head (tokens), >= 0                  */
  int32_t n_heads;            /* H                                                  */
  int32_t head_dim;           /* D                                                  */
  int32_t n_sub;              /* M                                                  */
  int32_t n_codes;            /* K                                                  */
  int64_t x_stride_vec;       /* x element (n, h, d) at x[n*x_stride_vec +          */
  int64_t x_stride_head;      /*   h*x_stride_head + d], in fp16 elements           */
  int64_t codes_stride_slot;  /* code (n, h, m) at codes[s*codes_stride_slot +      */
  int64_t codes_stride_head;  /*   h*codes_stride_head + m], bytes; s = slots[n],   */
                              /*   or s = n when slots is NULL                      */
  int64_t codes_bytes;        /* size of the codes buffer: the M codes of a (vector,*/
                              /*   head) whose place falls outside it are skipped,  */
                              /*   not written (a bad slot cannot fault the GPU);   */
                              /*   without slots, every place must fit              */
} pq_encode_desc;

/* Nearest-codeword encode (AQPIM page, sections 3.1 and 5.2 (2)): for every
 * vector n, head h and segment m, the index k minimising the squared
 * Euclidean distance between segment m of x[n][h] and codebook[h][m][k]; the
 * lowest index wins a tie.  Distances are decided in fp32.  Up to
 * 65535 * 256 = 16,776,960 vectors per call (more: PQ_ERR_UNSUPPORTED).
 *  x         fp16  strided as above; rows 16-byte aligned
 *  codebook  fp16  [H][M][K][D/M]
 *  slots     int64 [N] destination token slot per vector, or NULL
 *  codes     uint8 written at the strided places above
 * With the code cache of pq_attn_decode, slot = b*Hkv*max_len + t,
 * codes_stride_slot = M and codes_stride_head = max_len*M put token t of
 * request b straight into the cache. */
pq_status pq_encode(const pq_encode_desc* desc, const void* x, const void* codebook,
                    const int64_t* slots, uint8_t* codes, void* stream);

/* pq_encode for n (1..4) tensors of the same shape and strides in one launch
 * -- typically a new token's K and V, each with its own codebook and code
 * array.  x, codebook and codes are host arrays of n device pointers; slots
 * is shared.  Each plane i gives exactly what pq_encode(desc, x[i],
 * codebook[i], slots, codes[i]) gives.  n outside 1..4 is PQ_ERR_SHAPE. */
pq_status pq_encode_many(const pq_encode_desc* desc, int32_t n, const void* const* x,
                         const void* const* codebook, const int64_t* slots,
                         uint8_t* const* codes, void* stream);

/* The update step of one Lloyd (K-means) iteration of codebook learning
 * (AQPIM page, section 3.2 (2): codebooks fitted online to the first vectors
 * of a sequence; section 5.2 (1): a fast K-means on a small sample;
 * section 6.1 (3): a few K-means updates every so many tokens).  For every
 * head h, segment m and codeword k with at least one vector n whose code
 * (n, h, m) is k, codebook[h][m][k] becomes the mean of segment m of those
 * x[n][h]: the exact sum, divided by the count in double precision and
 * rounded to the nearest fp16 (ties to even).  Codewords no vector names keep
 * their value.  The result does not depend on the order of the vectors.
 *  desc      shape and strides as for pq_encode; the codes are read at their
 *            identity places (slot n for vector n), which must fit
 *            codes_bytes.  At most 4,194,304 vectors (PQ_ERR_UNSUPPORTED).
 *  x         fp16, as for pq_encode
 *  codes     uint8, e.g. what pq_encode wrote for the same x and codebook
 *  codebook  fp16 [H][M][K][D/M], updated in place, 16-byte aligned
 *  counts    uint32 [H][M][K] vectors per codeword, written; may be NULL */
pq_status pq_codebook_update(const pq_encode_desc* desc, const void* x, const uint8_t* codes,
                             void* codebook, uint32_t* counts, void* stream);

/* n_iter Lloyd iterations of codebook learning on the sample x, starting from
 * the codebook passed in (AQPIM page, sections 3.2 (2), 5.2 (1), 6.1 (3)):
 * each iteration is pq_encode of x into codes followed by
 * pq_codebook_update; then x is encoded once more, so on return codebook
 * holds the learned codewords and codes the sample's codes under them.
 * n_iter >= 0 (0: encode only).  Arguments as for pq_codebook_update, plus
 * codes aligned to M bytes; codes receives the final assignment.  Samples of
 * up to 8192 vectors run in one launch (the whole run on chip); larger ones
 * as 2 * n_iter + 1 launches.  Either way the result is the same and the
 * call does not synchronise. */
pq_status pq_kmeans(const pq_encode_desc* desc, const void* x, void* codebook, int32_t n_iter,
                    uint8_t* codes, void* stream);

/* pq_kmeans for n (1 or 2) samples of the same shape and strides in one call
 * -- typically the K and the V vectors of a layer, each with its own
 * codebook and codes.  x, codebook and codes are host arrays of n device
 * pointers; plane i gets exactly what pq_kmeans(desc, x[i], codebook[i],
 * n_iter, codes[i]) gives.  n outside 1..2 is PQ_ERR_SHAPE. */
pq_status pq_kmeans_many(const pq_encode_desc* desc, int32_t n, const void* const* x,
                         void* const* codebook, int32_t n_iter, uint8_t* const* codes,
                         void* stream);

/* pq_attn_decode_step for callers that cannot allocate device memory or pass
 * a workspace -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and results as
 * pq_attn_decode_step on a dense cache, without workspace: the chunk records
 * and arrival counters live in a device array inside the library, 8 MiB of
 * records and 65,536 counters, held on each GPU the library runs on until
 * the process ends.  Shapes whose step needs more (pq_attn_workspace_bytes
 * above 8 MiB, or B * n_kv_heads above 65,536) return PQ_ERR_WORKSPACE
 * with nothing launched.  The call allocates nothing; its first call on a
 * device also enqueues one small kernel that zeroes the counters.  Every
 * call on one GPU shares that GPU's array (each call leaves the counters at
 * zero, the records are rewritten by every call), so calls that overlap in
 * time on one GPU race: serialise them (one stream, or events). */
pq_status pq_attn_decode_step_noalloc(const pq_attn_desc* desc, const void* q, const void* k_new,
                                      const void* v_new, uint8_t* k_codes, uint8_t* v_codes,
                                      const void* k_cb, const void* v_cb, const int32_t* lens,
                                      float* out, void* stream);

/* ---- FP8 codebooks ------------------------------------------------------
 * The AQPIM page, section 4.2, stores the codebooks as a low-precision float
 * such as FP8.  These calls take K and V codebooks (and the encode's
 * codebook) as uint8 [Hkv][M][K][D/M] (resp. [H][M][K][D/M]) arrays of OCP
 * FP8 E4M3 values: bit 7 the sign, bits 6..3 the exponent e (bias 7), bits
 * 2..0 the mantissa f; the value is (-1)^s (1 + f/8) 2^(e-7), or
 * (-1)^s f 2^-9 for e = 0; bytes 0x7F and 0xFF (NaN) are not valid entries
 * and give unspecified results.  A codebook is half the bytes of the fp16
 * one (32 KB per KV head and tensor at M = 4, K = 256, D = 128).  Every E4M3
 * value is an fp16 value and the kernels convert on load, so each call
 * gives exactly (bit for bit) what its fp16 counterpart gives on the fp16
 * upcast of the codebooks.  Every other argument, check and layout is the
 * fp16 call's; the per-request score kernel runs for every shape (the
 * request-batched one is fp16 only), with the chunking -- and so the
 * workspace size -- of the fp16 call on the same descriptor. */

/* pq_attn_decode with FP8 E4M3 codebooks. */
pq_status pq_attn_decode_fp8cb(const pq_attn_desc* desc, const void* q,
                               const uint8_t* k_codes, const uint8_t* v_codes,
                               const uint8_t* k_cb, const uint8_t* v_cb, const int32_t* lens,
                               float* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* pq_attn_partials with FP8 E4M3 codebooks. */
pq_status pq_attn_partials_fp8cb(const pq_attn_desc* desc, const void* q,
                                 const uint8_t* k_codes, const uint8_t* v_codes,
                                 const uint8_t* k_cb, const uint8_t* v_cb, const int32_t* lens,
                                 float* part_m, float* part_l, float* part_o, void* stream);

/* pq_encode against an FP8 E4M3 codebook: the nearest of the codewords'
 * exact values (the decision of pq_encode on the fp16 upcast). */
pq_status pq_encode_fp8cb(const pq_encode_desc* desc, const void* x, const uint8_t* codebook,
                          const int64_t* slots, uint8_t* codes, void* stream);

/* A static, human-readable name for a status code. */
const char* pq_status_string(pq_status status);

#ifdef __cplusplus
}
#endif

#endif /* PQATTN_H */
