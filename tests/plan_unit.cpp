// Host-only unit test of the argument checking and launch planning, built
// with g++ and the address/undefined-behaviour sanitizers by
// tests/test_abi_host.py.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "plan.h"

using namespace pqattn;

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static pq_attn_desc base() {
  pq_attn_desc d;
  d.batch = 8; d.n_q_heads = 64; d.n_kv_heads = 8; d.head_dim = 128; d.n_sub = 8;
  d.n_codes = 256; d.max_len = 8192; d.chunk = 0; d.scale = 0.08838835f;
  return d;
}

int main() {
  AttnPlan p;
  pq_attn_desc d = base();
  EXPECT(plan_attn(&d, &p) == PQ_OK);
  EXPECT(p.G == 8 && p.DS == 16 && p.rows == 512);
  // 64 (request, KV head) pairs and 8192 tokens: the query heads split in
  // four parts of two, one chunk each
  EXPECT(p.HS == 4 && p.GW == 2 && p.C == 1 && p.T == 8192 && p.ws_bytes == 0);
  EXPECT(p.blocks == int64_t(p.B) * p.Hkv * p.HS * p.C);
  EXPECT(p.T * (p.C - 1) < p.Lmax && p.T * p.C >= p.Lmax);
  EXPECT(p.blocks >= 256);
  {   // few pairs, or a cache longer than one chunk: the token split
    pq_attn_desc e = base();
    e.batch = 1;        // 8 pairs: split both, 2 heads x 1024 tokens per workgroup
    EXPECT(plan_attn(&e, &p) == PQ_OK && p.HS == 4 && p.C == 8 && p.blocks == 256);
    e = base();
    e.max_len = 16384;
    EXPECT(plan_attn(&e, &p) == PQ_OK && p.HS == 1 && p.GW == 8 && p.C > 1);
    e = base();
    e.n_q_heads = 32;   // G = 4 and 64 pairs: two parts give only 128 workgroups
    EXPECT(plan_attn(&e, &p) == PQ_OK && p.HS == 1);
    e.batch = 16;       // 128 pairs: two parts of two, 256 workgroups
    EXPECT(plan_attn(&e, &p) == PQ_OK && p.HS == 2 && p.GW == 2 && p.C == 1);
    e = base();
    e.batch = 64;       // enough pairs for the token split
    EXPECT(plan_attn(&e, &p) == PQ_OK && p.HS == 1);
  }

  // explicit chunks
  d.chunk = 2048;
  EXPECT(plan_attn(&d, &p) == PQ_OK && p.C == 4 && p.T == 2048);
  EXPECT(p.ws_bytes >= size_t(512) * 4 * 130 * 4);
  EXPECT(p.ws_l_off % 256 == 0 && p.ws_o_off % 256 == 0 && p.ws_bytes % 256 == 0);
  d.chunk = 7;
  EXPECT(plan_attn(&d, &p) == PQ_OK && p.C == (8192 + 6) / 7);
  d.chunk = 4096;
  EXPECT(plan_attn(&d, &p) == PQ_OK && p.C == 2);
  d.chunk = 8192;                                   // longer than one workgroup takes
  EXPECT(plan_attn(&d, &p) == PQ_ERR_UNSUPPORTED);
  d.max_len = 4096; d.chunk = 1 << 30;              // clamped to the capacity
  EXPECT(plan_attn(&d, &p) == PQ_OK && p.C == 1 && p.ws_bytes == 0);
  d.max_len = 8192;

  // bad and unsupported
  d = base(); d.n_kv_heads = 7;                 EXPECT(plan_attn(&d, &p) == PQ_ERR_SHAPE);
  d = base(); d.scale = std::nanf("");          EXPECT(plan_attn(&d, &p) == PQ_ERR_SHAPE);
  d = base(); d.scale = -1.0f;                  EXPECT(plan_attn(&d, &p) == PQ_ERR_SHAPE);
  d = base(); d.max_len = 8190;                 EXPECT(plan_attn(&d, &p) == PQ_ERR_UNSUPPORTED);
  d = base(); d.n_q_heads = 8 * 16;             EXPECT(plan_attn(&d, &p) == PQ_ERR_UNSUPPORTED);
  d = base(); d.batch = std::numeric_limits<int32_t>::max(); d.chunk = 1;
  EXPECT(plan_attn(&d, &p) == PQ_ERR_UNSUPPORTED);        // too many workgroups
  d = base(); d.batch = 65535; d.n_q_heads = 8; d.n_kv_heads = 1;
  EXPECT(plan_attn(&d, &p) == PQ_OK);                     // largest grid z extent
  d.batch = 65536;                              EXPECT(plan_attn(&d, &p) == PQ_ERR_UNSUPPORTED);
  d = base(); d.batch = 1; d.max_len = 16 * 65535; d.chunk = 16;
  EXPECT(plan_attn(&d, &p) == PQ_OK && p.C == 65535);     // largest grid y extent
  d.max_len = 16 * 65536;                       EXPECT(plan_attn(&d, &p) == PQ_ERR_UNSUPPORTED);
  EXPECT(plan_attn(nullptr, &p) == PQ_ERR_NULL);

  // chunk pick: small problems still get one chunk per 256 tokens at most
  EXPECT(pick_chunk(1, 8, 512, 512, 256) == 256);
  EXPECT(pick_chunk(64, 32, 4096, 512, 256) == 4096);
  EXPECT(pick_chunk(1, 8, 131072, 512, 256) == 2048);
  EXPECT(pick_chunk(1, 1, 16, 512, 256) == 16);
  EXPECT(pick_chunk(1, 1, 1 << 20, 256, 512) == kMaxChunk);
  d = base(); d.chunk = 0;
  EXPECT(plan_attn(&d, &p) == PQ_OK && p.T <= kMaxChunkSmall && p.T % 512 == 0);

  // encode
  pq_encode_desc e;
  e.n_vec = 100; e.n_heads = 32; e.head_dim = 128; e.n_sub = 4; e.n_codes = 256;
  e.x_stride_vec = 32 * 128; e.x_stride_head = 128; e.codes_stride_slot = 4;
  e.codes_stride_head = 4096 * 4; e.codes_bytes = 1 << 20;
  EncodePlan ep;
  EXPECT(plan_encode(&e, 128, &ep) == PQ_OK && ep.blocks_x == 1 && ep.DS == 32);
  e.n_vec = 0;        EXPECT(plan_encode(&e, 128, &ep) == PQ_OK && ep.blocks_x == 0);
  e.n_vec = 100; e.x_stride_head = 12;  EXPECT(plan_encode(&e, 128, &ep) == PQ_ERR_ALIGN);
  e.x_stride_head = 128; e.codes_stride_slot = 6; EXPECT(plan_encode(&e, 128, &ep) == PQ_ERR_ALIGN);
  e.codes_stride_slot = 4; e.n_codes = 128; EXPECT(plan_encode(&e, 128, &ep) == PQ_ERR_UNSUPPORTED);
  e.n_codes = 256; e.n_vec = int64_t(65535) * 256; EXPECT(plan_encode(&e, 256, &ep) == PQ_OK && ep.blocks_x == 65535);
  e.n_vec += 1;       EXPECT(plan_encode(&e, 256, &ep) == PQ_ERR_UNSUPPORTED);

  // request batching: one query head per KV head and many pairs
  {
    pq_attn_desc md = base();
    md.batch = 64; md.n_q_heads = 32; md.n_kv_heads = 32; md.n_sub = 4; md.max_len = 4096;
    AttnPlan mp;
    EXPECT(plan_attn(&md, &mp) == PQ_OK && mp.R == kMhaRequests && mp.T == 4096 && mp.C == 1);
    md.n_sub = 8;
    EXPECT(plan_attn(&md, &mp) == PQ_OK && mp.R == kMhaRequests && mp.T == 2048 && mp.C == 2);
    md.n_sub = 4; md.max_len = 512;
    EXPECT(plan_attn(&md, &mp) == PQ_OK && mp.R == kMhaRequests && mp.T == 512 && mp.C == 1);
    md.chunk = 300;
    EXPECT(plan_attn(&md, &mp) == PQ_OK && mp.R == kMhaRequests && mp.T == 300 && mp.C == 2);
    md.chunk = 0; md.batch = 4;                     // 128 pairs: one request per workgroup
    EXPECT(plan_attn(&md, &mp) == PQ_OK && mp.R == 1);
    md.batch = 64; md.n_q_heads = 64;               // two query heads per KV head
    EXPECT(plan_attn(&md, &mp) == PQ_OK && mp.R == 1);
    md.n_q_heads = 32; md.max_len = 8192; md.chunk = 8192;   // longer than the batched kernel's
    EXPECT(plan_attn(&md, &mp) == PQ_OK && mp.R == 1 && mp.T == 8192 && mp.C == 1);
    md.max_len = 16384; md.chunk = 16384;                    // longer than any kernel's chunk
    EXPECT(plan_attn(&md, &mp) == PQ_ERR_UNSUPPORTED);
  }

  // two chunks per workgroup: M = 4, chunks of 1024 or 2048 tokens, more
  // (request, KV head, chunk) triples than CUs
  {
    pq_attn_desc ld = base();
    ld.batch = 1; ld.n_q_heads = 64; ld.n_kv_heads = 8; ld.n_sub = 4; ld.max_len = 131072;
    AttnPlan lp;
    ld.chunk = 2048;   // the long-context workload: 8 x 64 = 512 chunks
    EXPECT(plan_attn(&ld, &lp) == PQ_OK && lp.C == 64 && lp.CPW == 2);
    ld.chunk = 1024;
    EXPECT(plan_attn(&ld, &lp) == PQ_OK && lp.C == 128 && lp.CPW == 2);
    ld.chunk = 0;      // the library's chunk (4096): 256 workgroups already
    EXPECT(plan_attn(&ld, &lp) == PQ_OK && lp.T == 4096 && lp.CPW == 1);
    ld.chunk = 1536;   // not a whole number of token slots per thread
    EXPECT(plan_attn(&ld, &lp) == PQ_OK && lp.CPW == 1);
    ld.chunk = 2048; ld.n_sub = 8;   // two M = 8 histograms do not fit in LDS
    EXPECT(plan_attn(&ld, &lp) == PQ_OK && lp.CPW == 1);
    ld.n_sub = 4; ld.max_len = 65536;   // 8 x 32 = 256 chunks: one per CU already
    EXPECT(plan_attn(&ld, &lp) == PQ_OK && lp.C == 32 && lp.CPW == 1);
    ld.max_len = 67584;                 // 8 x 33 = 264 > 256
    EXPECT(plan_attn(&ld, &lp) == PQ_OK && lp.C == 33 && lp.CPW == 2);
  }

  // paged cache
  {
    pq_attn_desc pd = base();              // max_len 8192
    AttnPlan pp;
    EXPECT(plan_attn(&pd, &pp) == PQ_OK);
    int32_t dummy = 0;
    pq_page_table t{&dummy, 256, 32, 1000};
    PagePlan pg;
    EXPECT(plan_pages(pp, &t, &pg) == PQ_OK && pg.shift == 8 && pg.P == 256);
    EXPECT(pg.pool_head_bytes == int64_t(1000) * 256 * 8);
    t.page_tokens = 16; t.max_pages = 512;
    EXPECT(plan_pages(pp, &t, &pg) == PQ_OK && pg.shift == 4);
    t.page_tokens = 65536; t.max_pages = 1;   // one page longer than the cache: shape
    EXPECT(plan_pages(pp, &t, &pg) == PQ_ERR_SHAPE);
    t.page_tokens = 8192; t.max_pages = 1;
    EXPECT(plan_pages(pp, &t, &pg) == PQ_OK && pg.shift == 13);
    t.page_tokens = 96; t.max_pages = 85;     // not a power of two
    EXPECT(plan_pages(pp, &t, &pg) == PQ_ERR_SHAPE);
    t.page_tokens = 8; t.max_pages = 1024;    // below the minimum
    EXPECT(plan_pages(pp, &t, &pg) == PQ_ERR_SHAPE);
    t.page_tokens = 256; t.max_pages = 32; t.n_pages = 0;
    EXPECT(plan_pages(pp, &t, &pg) == PQ_ERR_SHAPE);
    t.n_pages = (1 << 20) - 1;                 // a KV head's pool just under 2 GiB
    EXPECT(plan_pages(pp, &t, &pg) == PQ_OK && pg.pool_head_bytes == int64_t(t.n_pages) * 256 * 8);
    t.n_pages = 1 << 20;                       // 2 GiB: past the kernels' 32-bit offsets
    EXPECT(plan_pages(pp, &t, &pg) == PQ_ERR_UNSUPPORTED);
    t.block_table = nullptr;
    EXPECT(plan_pages(pp, &t, &pg) == PQ_ERR_NULL);
    EXPECT(plan_pages(pp, nullptr, &pg) == PQ_ERR_NULL);
  }

  // reduce
  EXPECT(check_reduce(10, 1, 128) == PQ_OK);
  EXPECT(check_reduce(10, 0, 128) == PQ_ERR_SHAPE);
  EXPECT(check_reduce(10, 4, 96) == PQ_ERR_UNSUPPORTED);

  if (failures) {
    std::printf("plan_unit: %d failures\n", failures);
    return 1;
  }
  std::printf("plan_unit: all checks passed\n");
  return 0;
}
