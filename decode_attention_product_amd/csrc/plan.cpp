// Host-side argument checking and launch planning (no HIP calls).
#include "plan.h"

#include <cmath>
#include <limits>

namespace pqattn {

namespace {

constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxGridYZ = 65535;
constexpr int kTargetBlocks = 256;     // one score workgroup per CU (256 CUs)
constexpr int kChunkGranule = 1024;    // one token per thread of a 1024-thread workgroup

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

}  // namespace

// Estimated time (ns) of the per-request score kernel (and its merge) for
// one split of the work: `blocks` workgroups of `tokens` tokens and GW query
// heads each, over the 256 CUs in rounds of one workgroup per CU; fitted to
// in-kernel clock stamps on MI355X (prologue and table build plus
// contraction ~6 us per workgroup; table gathers and histogram atomics
// ~0.067 ns per token per LDS instruction; chunk records, arrival and merge
// ~4.5 us, ~1 us more past 8 chunks; a head split reads each code row
// HS times through L2: ~2 us for 8192 tokens at M = 8, in proportion).
double split_cost_ns(int64_t blocks, int64_t tokens, int GW, int M, int C, int HS) {
  const int64_t rounds = (blocks + kTargetBlocks - 1) / kTargetBlocks;
  const double lds_per_token = M * 0.067 * ((GW + 3) / 4 + (GW >= 2 ? GW / 2 : 1));
  double t = double(rounds) * (6000.0 + lds_per_token * double(tokens));
  if (C > 1) t += C > 8 ? 5500.0 : 4500.0;
  if (HS > 1) t += double(rounds) * 2000.0 * double(tokens) * M / (8192.0 * 8.0);
  return t;
}

void choose_split(int32_t B, int32_t Hkv, int32_t G, int32_t M, int32_t Lmax, int32_t* T_out,
                  int32_t* HS_out) {
  double best = 0.0;
  int32_t bestT = 0, bestHS = 1;
  const int32_t hs_options[2] = {1, G >= 4 ? G / 2 : 1};
  for (int32_t hs : hs_options) {
    if (hs == 1 && bestT != 0 && hs_options[1] == 1) break;
    const int GW = G / hs;
    const int32_t tmax = GW <= 2 ? kMaxChunkSmall : kMaxChunk;
    for (int32_t t = kChunkGranule; t <= 2 * tmax; t *= 2) {
      const int32_t T = t <= tmax ? (t < Lmax ? t : Lmax) : (Lmax <= tmax ? Lmax : 0);
      if (T == 0) continue;
      const int64_t C = (int64_t(Lmax) + T - 1) / T;
      if (C > kMaxGridYZ) continue;
      int64_t blocks = int64_t(B) * Hkv * hs * C;
      int64_t tokens = T;
      if (hs == 1 && M == 4 && C >= 2 && (T == 1024 || T == 2048) && blocks > kCpwCUs) {
        blocks = (int64_t(B) * Hkv) * ((C + 1) / 2);   // two chunks per workgroup
        tokens = 2 * T;
      }
      const double c = split_cost_ns(blocks, tokens, GW, M, int(C), hs);
      // ties: fewer chunks, then no head split
      if (bestT == 0 || c < best - 1.0 ||
          (c <= best + 1.0 && (C < (int64_t(Lmax) + bestT - 1) / bestT))) {
        best = c;
        bestT = T;
        bestHS = hs;
      }
    }
  }
  *T_out = bestT;
  *HS_out = bestHS;
}

int32_t pick_chunk(int32_t B, int32_t Hkv, int32_t Lmax, int32_t target_blocks, int32_t granule) {
  const int64_t pairs = int64_t(B) * Hkv;
  int64_t want_chunks = (target_blocks + pairs - 1) / pairs;
  if (want_chunks < 1) want_chunks = 1;
  int64_t t = (Lmax + want_chunks - 1) / want_chunks;
  t = (t + granule - 1) / granule * granule;
  if (t < granule) t = granule;
  if (t > kMaxChunk) t = kMaxChunk;
  if (t > Lmax) t = Lmax;
  return int32_t(t);
}

pq_status plan_attn(const pq_attn_desc* d, AttnPlan* p) {
  if (d == nullptr || p == nullptr) return PQ_ERR_NULL;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->n_sub < 1 || d->n_codes < 1 || d->max_len < 1 || d->chunk < 0)
    return PQ_ERR_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0) return PQ_ERR_SHAPE;
  if (d->head_dim % d->n_sub != 0) return PQ_ERR_SHAPE;
  if (!std::isfinite(d->scale) || !(d->scale > 0.0f)) return PQ_ERR_SHAPE;

  const int G = d->n_q_heads / d->n_kv_heads;
  if (d->head_dim != kHeadDim || d->n_codes != kCodes) return PQ_ERR_UNSUPPORTED;
  if (d->n_sub != 4 && d->n_sub != 8) return PQ_ERR_UNSUPPORTED;
  if (!supported_group(G)) return PQ_ERR_UNSUPPORTED;
  if (d->max_len % kLenAlign != 0) return PQ_ERR_UNSUPPORTED;

  p->B = d->batch;
  p->Hq = d->n_q_heads;
  p->Hkv = d->n_kv_heads;
  p->G = G;
  p->D = d->head_dim;
  p->M = d->n_sub;
  p->DS = d->head_dim / d->n_sub;
  p->K = d->n_codes;
  p->Lmax = d->max_len;
  int32_t hs_pick = 1;
  if (d->chunk > 0) {
    p->T = d->chunk < d->max_len ? d->chunk : d->max_len;
  } else {
    choose_split(d->batch, d->n_kv_heads, G, d->n_sub, d->max_len, &p->T, &hs_pick);
  }
  // one query head per KV head and many (request, KV head) pairs: the
  // request-batched score kernel, with chunks as long as it takes
  p->R = 1;
  if (G == 1 && int64_t(p->B) * p->Hkv >= kMhaMinPairs) {
    const int tmax = p->M == 4 ? kMhaMaxChunkM4 : kMhaMaxChunkM8;
    const int32_t tb = d->chunk > 0 ? p->T : (p->Lmax < tmax ? p->Lmax : tmax);
    if (tb <= tmax) {
      p->R = kMhaRequests;
      p->T = tb;
    }
  }
  p->HS = p->R == 1 ? hs_pick : 1;
  p->GW = G / p->HS;
  if (p->T > (p->GW <= 2 ? kMaxChunkSmall : kMaxChunk)) return PQ_ERR_UNSUPPORTED;
  p->C = int32_t((int64_t(p->Lmax) + p->T - 1) / p->T);
  p->scale = d->scale;
  p->rows = int64_t(p->B) * p->Hq;
  p->CPW = (p->R == 1 && p->M == 4 && p->C >= 2 && (p->T == 1024 || p->T == 2048) &&
            int64_t(p->B) * p->Hkv * p->C > kCpwCUs) ? 2 : 1;
  p->blocks = int64_t(p->B) * p->Hkv * p->HS * p->C;
  if (p->blocks > kMaxBlocks || p->rows > kMaxBlocks) return PQ_ERR_UNSUPPORTED;
  // score-kernel grids (Hkv, C, B) and (Hkv, C, B / R): the y and z extents are 16-bit
  if (p->C > kMaxGridYZ || p->B > kMaxGridYZ) return PQ_ERR_UNSUPPORTED;

  // workspace: m and l [rows][C], o [rows][C][D], each 256-byte aligned
  const size_t n_stat = size_t(p->rows) * size_t(p->C);
  if (n_stat > std::numeric_limits<size_t>::max() / (size_t(p->D) * 4 + 8)) return PQ_ERR_SHAPE;
  if (p->C == 1) {
    p->ws_m_off = p->ws_l_off = p->ws_o_off = 0;
    p->ws_bytes = 0;
  } else {
    p->ws_m_off = 0;
    p->ws_l_off = round_up(n_stat * 4, 256);
    p->ws_o_off = p->ws_l_off + round_up(n_stat * 4, 256);
    p->ws_bytes = p->ws_o_off + round_up(n_stat * size_t(p->D) * 4, 256);
  }
  // decode step: the chunk records plus one arrival counter per (b, kv head,
  // head part)
  if (p->C == 1) {
    p->ws_cnt_off = 0;
    p->ws_step_bytes = 0;
  } else {
    p->ws_cnt_off = p->ws_bytes;
    p->ws_step_bytes = p->ws_cnt_off + round_up(size_t(p->B) * size_t(p->Hkv) * p->HS * 4, 256);
  }
  return PQ_OK;
}

pq_status plan_encode(const pq_encode_desc* d, int32_t vec_per_block, EncodePlan* p) {
  if (d == nullptr || p == nullptr) return PQ_ERR_NULL;
  if (d->n_vec < 0 || d->n_heads < 1 || d->head_dim < 1 || d->n_sub < 1 || d->n_codes < 1)
    return PQ_ERR_SHAPE;
  if (d->head_dim % d->n_sub != 0) return PQ_ERR_SHAPE;
  if (d->x_stride_vec < 0 || d->x_stride_head < 0 || d->codes_stride_slot < 0 ||
      d->codes_stride_head < 0 || d->codes_bytes < 0)
    return PQ_ERR_SHAPE;
  if (d->head_dim != kHeadDim || d->n_codes != kCodes) return PQ_ERR_UNSUPPORTED;
  if (d->n_sub != 4 && d->n_sub != 8) return PQ_ERR_UNSUPPORTED;
  // 16-byte rows of x; codes of one (vector, head) written as one M-byte word
  if (d->x_stride_vec % 8 != 0 || d->x_stride_head % 8 != 0) return PQ_ERR_ALIGN;
  if (d->codes_stride_slot % d->n_sub != 0 || d->codes_stride_head % d->n_sub != 0)
    return PQ_ERR_ALIGN;
  p->N = d->n_vec;
  p->H = d->n_heads;
  p->D = d->head_dim;
  p->M = d->n_sub;
  p->DS = d->head_dim / d->n_sub;
  p->K = d->n_codes;
  p->blocks_x = (d->n_vec + vec_per_block - 1) / vec_per_block;
  // encode grid (H, tiles, planes): the tile count is a 16-bit y extent
  if (p->blocks_x > kMaxGridYZ || d->n_heads > 65535) return PQ_ERR_UNSUPPORTED;
  return PQ_OK;
}

pq_status plan_pages(const AttnPlan& p, const pq_page_table* t, PagePlan* out) {
  if (t == nullptr || out == nullptr || t->block_table == nullptr) return PQ_ERR_NULL;
  const int32_t P = t->page_tokens;
  if (P < kMinPageTokens || P > kMaxPageTokens || (P & (P - 1)) != 0) return PQ_ERR_SHAPE;
  if (t->max_pages < 1 || t->n_pages < 1) return PQ_ERR_SHAPE;
  if (int64_t(t->max_pages) * P != p.Lmax) return PQ_ERR_SHAPE;
  // every pool offset (and Hkv pools side by side) must fit in 62 bits
  const int64_t head_bytes = int64_t(t->n_pages) * P * p.M;
  if (head_bytes > (int64_t(1) << 62) / p.Hkv) return PQ_ERR_SHAPE;
  // the score kernels address a KV head's pool with 32-bit buffer offsets
  if (head_bytes >= (int64_t(1) << 31)) return PQ_ERR_UNSUPPORTED;
  out->block_table = t->block_table;
  out->P = P;
  int shift = 0;
  while ((1 << shift) < P) ++shift;
  out->shift = shift;
  out->max_pages = t->max_pages;
  out->n_pages = t->n_pages;
  out->pool_head_bytes = head_bytes;
  return PQ_OK;
}

pq_status check_reduce(int64_t n_rows, int32_t n_chunks, int32_t head_dim) {
  if (n_rows < 0 || n_chunks < 1 || head_dim < 1) return PQ_ERR_SHAPE;
  if (head_dim != kHeadDim) return PQ_ERR_UNSUPPORTED;
  if (n_rows > kMaxBlocks) return PQ_ERR_UNSUPPORTED;
  return PQ_OK;
}

const char* status_string(pq_status s) {
  switch (s) {
    case PQ_OK: return "ok";
    case PQ_ERR_NULL: return "a required pointer is NULL";
    case PQ_ERR_SHAPE: return "descriptor fields are inconsistent or out of range";
    case PQ_ERR_UNSUPPORTED: return "shape not supported by this library";
    case PQ_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PQ_ERR_HIP: return "the HIP runtime refused a launch";
    case PQ_ERR_ALIGN: return "an array pointer or stride is not suitably aligned";
  }
  return "unknown status";
}

}  // namespace pqattn
