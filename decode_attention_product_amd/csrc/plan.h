// Host-side argument checking and launch planning for the PQ-KV attention
// library.  Pure C++ (no HIP): the same file is compiled into the shared
// library and into a host-only unit test.
#pragma once

#include <cstddef>
#include <cstdint>

#include "pqattn.h"

namespace pqattn {

constexpr int kHeadDim = 128;   // D supported by the kernels
constexpr int kCodes = 256;     // K codewords per segment codebook
constexpr int kLenAlign = 16;   // cache capacity granularity, tokens
constexpr int kMaxChunk = 4096; // longest chunk a score workgroup of 4 or 8 query heads takes
constexpr int kMaxChunkSmall = 8192;  // ... of 1 or 2 query heads (8 token slots per thread)
// Request batching for one query head per KV head: kMhaRequests requests of
// a KV head per score workgroup (in passes of kMhaPassRequests) once there
// are at least kMhaMinPairs (request, KV head) pairs; chunks of up to
// kMhaMaxChunkM4 / M8 tokens.
constexpr int kMhaRequests = 8;
constexpr int kMhaPassRequests = 4;
constexpr int64_t kMhaMinPairs = 1024;
constexpr int kMhaMaxChunkM4 = 4096;
constexpr int kMhaMaxChunkM8 = 2048;
// A per-request score workgroup takes two chunks when one chunk each would
// give more workgroups than the chip has CUs (a second round of workgroups,
// each with its own prologue and table build) and two histograms fit in LDS:
// M = 4 and chunks of exactly 1024 or 2048 tokens.
constexpr int64_t kCpwCUs = 256;
// When the library chooses the chunk (desc->chunk == 0) it also chooses
// whether to split the query heads of a KV head over G / 2 workgroups of
// two (G >= 4): among chunk lengths of 1024 * 2^k tokens (or the whole
// cache) and the two head splits, the one split_cost_ns estimates fastest.

// A checked decode-attention shape with the chunking resolved.
struct AttnPlan {
  int32_t B, Hq, Hkv, G, D, M, DS, K, Lmax, T, C;
  int32_t R;            // requests per score workgroup of the plain decode (1, or
                        // kMhaRequests for the request-batched kernel)
  int32_t CPW;          // chunks per workgroup of the per-request score kernel
                        // (1, or 2: see kCpwCUs)
  int32_t HS;           // head split: workgroups per (b, KV head, chunk), each with
                        // GW = G / HS query heads (see kSplitMinBlocks)
  int32_t GW;
  float scale;
  int64_t rows;         // B * Hq
  int64_t blocks;       // score-kernel workgroups, B * Hkv * C
  size_t ws_m_off, ws_l_off, ws_o_off, ws_bytes;   // workspace carve-up (C > 1)
  size_t ws_cnt_off, ws_step_bytes;                // decode step: + arrival counters (C > 1)
};

// Checks *d and fills *p.  Returns PQ_OK, PQ_ERR_NULL, PQ_ERR_SHAPE or
// PQ_ERR_UNSUPPORTED.  Never touches the GPU.
pq_status plan_attn(const pq_attn_desc* d, AttnPlan* p);

// The chunk length the library picks when the caller passes chunk = 0: enough
// chunks that the score kernel has about `target_blocks` workgroups, each
// chunk a multiple of `granule` tokens.
int32_t pick_chunk(int32_t B, int32_t Hkv, int32_t Lmax, int32_t target_blocks, int32_t granule);

// The time model behind the library's choice (ns, see plan.cpp) and the
// choice itself: chunk length *T and head split *HS for the per-request
// score kernel.
double split_cost_ns(int64_t blocks, int64_t tokens, int GW, int M, int C, int HS);
void choose_split(int32_t B, int32_t Hkv, int32_t G, int32_t M, int32_t Lmax, int32_t* T,
                  int32_t* HS);

struct EncodePlan {
  int64_t N;
  int32_t H, D, M, DS, K;
  int64_t blocks_x;     // vector tiles (grid y extent, at most 65535)
};

pq_status plan_encode(const pq_encode_desc* d, int32_t vec_per_block, EncodePlan* p);

pq_status check_reduce(int64_t n_rows, int32_t n_chunks, int32_t head_dim);

// A checked paged-cache description for an attention plan.
struct PagePlan {
  const int32_t* block_table;
  int32_t P, shift, max_pages, n_pages;
  int64_t pool_head_bytes;   // n_pages * P * M: one KV head's pool
};

// Checks *t against the plan (max_len == max_pages * page_tokens, page_tokens
// a power of two in [kMinPageTokens, kMaxPageTokens]) and fills *out.
// Returns PQ_OK, PQ_ERR_NULL or PQ_ERR_SHAPE.  Never touches the GPU.
constexpr int kMinPageTokens = 16;
constexpr int kMaxPageTokens = 65536;
pq_status plan_pages(const AttnPlan& p, const pq_page_table* t, PagePlan* out);

inline bool aligned16(const void* ptr) {
  return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

const char* status_string(pq_status s);

}  // namespace pqattn
