// C entry points of the PQ-KV decode-attention library (declared in
// include/pqattn.h).  Each call checks its arguments on the host, picks the
// kernel instance for the shape and enqueues it on the caller's stream.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <mutex>

#include "decode_kernel.hpp"
#include "decode_mha_kernel.hpp"
#include "encode_kernel.hpp"
#include "kmeans_kernel.hpp"
#include "plan.h"
#include "pqattn.h"

namespace pqattn {
namespace {

static_assert(kMaxChunk == 4 * kDecodeThreads && kMaxChunkSmall == 8 * kDecodeThreads,
              "a chunk is at most 4 token slots per thread (8 with one or two query heads)");

constexpr int kReduceThreads = 128;
constexpr int kEncodeVectors = 256;   // vectors per encode workgroup (one wave per segment)
constexpr int kEncodeVectorsSmall = 16;   // one tile: for launches with fewer workgroups than CUs
constexpr int64_t kEncodeCUs = 256;

// Vectors per encode workgroup: 256, or one 16-vector tile when 256-vector
// tiles would leave CUs idle (e.g. a decode step's new tokens): every
// workgroup loads its codebook half and computes its norms either way, so
// more, shorter workgroups finish sooner.
int encode_vectors(int64_t n_vec, int64_t heads, int64_t planes) {
  const int64_t big = (n_vec + kEncodeVectors - 1) / kEncodeVectors;
  return big * heads * planes < kEncodeCUs ? kEncodeVectorsSmall : kEncodeVectors;
}

// A one-tile launch whose workgroups, split one segment each, still fit on
// the CUs in one round runs them split (128 threads, grid z = plane * M +
// segment): each loads 1/M of the codebook, so the launch's latency drops.
// Measured: the GQA workload's three-launch step (16 workgroups of 8
// segments) 22.96 -> 21.31 us; the ragged step's encode (256 workgroups of 4
// segments, already a full round) was 0.2-0.4 us slower split.
bool encode_split(int64_t n_vec, int nv, int64_t heads, int64_t planes, int M) {
  const int64_t tiles = (n_vec + nv - 1) / nv;
  return nv == kEncodeVectorsSmall && tiles * heads * planes * M <= kEncodeCUs;
}

const void* encode_fn(int M, int nv, bool split) {
  if (split)
    return M == 4 ? reinterpret_cast<const void*>(&encode_kernel<4, kEncodeVectorsSmall, CbFmt::F16, true>)
                  : reinterpret_cast<const void*>(&encode_kernel<8, kEncodeVectorsSmall, CbFmt::F16, true>);
  if (nv == kEncodeVectorsSmall)
    return M == 4 ? reinterpret_cast<const void*>(&encode_kernel<4, kEncodeVectorsSmall>)
                  : reinterpret_cast<const void*>(&encode_kernel<8, kEncodeVectorsSmall>);
  return M == 4 ? reinterpret_cast<const void*>(&encode_kernel<4, kEncodeVectors>)
                : reinterpret_cast<const void*>(&encode_kernel<8, kEncodeVectors>);
}

using DecodeFn = void (*)(DecodeArgs);

template <int G, int M, int NT, bool STEP, bool PAGED, int CPW = 1>
DecodeFn kernel_for() {
  if constexpr (PAGED) return &decode_paged_kernel<G, M, NT, STEP, CPW>;
  else return &decode_partials_kernel<G, M, NT, STEP, CPW>;
}

template <int G, int M, bool STEP, bool PAGED>
DecodeFn pick_nt(int T, int cpw) {
  if constexpr (M == 4) {   // two chunks of exactly 1024 or 2048 tokens per workgroup
    if (cpw == 2) {
      if (T == kDecodeThreads) return kernel_for<G, M, 2, STEP, PAGED, 2>();
      if (T == 2 * kDecodeThreads) return kernel_for<G, M, 4, STEP, PAGED, 2>();
      return nullptr;
    }
  }
  if (cpw != 1) return nullptr;
  if (T <= kDecodeThreads) return kernel_for<G, M, 1, STEP, PAGED>();
  if (T <= 2 * kDecodeThreads) return kernel_for<G, M, 2, STEP, PAGED>();
  if (T <= 4 * kDecodeThreads) return kernel_for<G, M, 4, STEP, PAGED>();
  if constexpr (G <= 2) {
    if (T <= 8 * kDecodeThreads) return kernel_for<G, M, 8, STEP, PAGED>();
  }
  return nullptr;
}

template <bool STEP, bool PAGED>
DecodeFn pick_gm(int G, int M, int T, int cpw) {
  switch (M * 16 + G) {
    case 4 * 16 + 1: return pick_nt<1, 4, STEP, PAGED>(T, cpw);
    case 4 * 16 + 2: return pick_nt<2, 4, STEP, PAGED>(T, cpw);
    case 4 * 16 + 4: return pick_nt<4, 4, STEP, PAGED>(T, cpw);
    case 4 * 16 + 8: return pick_nt<8, 4, STEP, PAGED>(T, cpw);
    case 8 * 16 + 1: return pick_nt<1, 8, STEP, PAGED>(T, cpw);
    case 8 * 16 + 2: return pick_nt<2, 8, STEP, PAGED>(T, cpw);
    case 8 * 16 + 4: return pick_nt<4, 8, STEP, PAGED>(T, cpw);
    case 8 * 16 + 8: return pick_nt<8, 8, STEP, PAGED>(T, cpw);
  }
  return nullptr;
}

// The kernel instance for (G, M) (query heads per workgroup), the chunk length T, the
// chunks per workgroup, the plain or decode-step variant and the dense or
// paged cache.
DecodeFn pick_decode(int G, int M, int T, int cpw, bool step, bool paged) {
  if (paged) return step ? pick_gm<true, true>(G, M, T, cpw) : pick_gm<false, true>(G, M, T, cpw);
  return step ? pick_gm<true, false>(G, M, T, cpw) : pick_gm<false, false>(G, M, T, cpw);
}


// The request-batched kernel (one query head per KV head) whose NT token
// slots per thread cover a chunk of T tokens.
template <int M, bool PAGED>
DecodeFn pick_mha_nt(int T) {
  constexpr int TPR = kDecodeThreads / kMhaPassRequests;   // threads per request in a pass
  if (T <= TPR) return &decode_mha_kernel<M, kMhaRequests, 1, PAGED>;
  if (T <= 2 * TPR) return &decode_mha_kernel<M, kMhaRequests, 2, PAGED>;
  if (T <= 4 * TPR) return &decode_mha_kernel<M, kMhaRequests, 4, PAGED>;
  if (T <= 8 * TPR) return &decode_mha_kernel<M, kMhaRequests, 8, PAGED>;
  if constexpr (M == 4) {
    if (T <= 16 * TPR) return &decode_mha_kernel<M, kMhaRequests, 16, PAGED>;
  }
  return nullptr;
}

DecodeFn pick_mha(int M, int T, bool paged) {
  if (M == 4) return paged ? pick_mha_nt<4, true>(T) : pick_mha_nt<4, false>(T);
  return paged ? pick_mha_nt<8, true>(T) : pick_mha_nt<8, false>(T);
}

// Launch; with events, the runtime stamps them at the kernel's own start and
// end (hipExtLaunchKernel), which is what a kernel timer should see.
pq_status launch(const void* fn, dim3 grid, dim3 block, void* arg, hipStream_t stream,
                 hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
  void* args[] = {arg};
  const hipError_t e = (start || stop)
      ? hipExtLaunchKernel(fn, grid, block, args, 0, stream, start, stop, 0)
      : hipLaunchKernel(fn, grid, block, args, 0, stream);
  return e == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

pq_status check_attn_pointers(const void* q, const void* kc, const void* vc, const void* kcb,
                              const void* vcb, const void* lens) {
  if (!q || !kc || !vc || !kcb || !vcb || !lens) return PQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(kcb) || !aligned16(vcb))
    return PQ_ERR_ALIGN;
  return PQ_OK;
}

// What one score-kernel launch reads and writes: the chunk records (pm, pl,
// po) or, with C == 1, the normalised output (out); for the decode step the
// new token's K and V and, for the fused merge (C > 1), the arrival
// counters; for a paged cache its checked plan.
struct ScoreIO {
  const void* q = nullptr;
  const uint8_t* kc = nullptr;
  const uint8_t* vc = nullptr;
  const void* kcb = nullptr;
  const void* vcb = nullptr;
  const int32_t* lens = nullptr;
  const PagePlan* pages = nullptr;
  float* pm = nullptr;
  float* pl = nullptr;
  float* po = nullptr;
  float* out = nullptr;
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  uint32_t* counters = nullptr;
};

ScoreIO score_inputs(const void* q, const uint8_t* kc, const uint8_t* vc, const void* kcb,
                     const void* vcb, const int32_t* lens, const PagePlan* pages) {
  ScoreIO io;
  io.q = q;
  io.kc = kc;
  io.vc = vc;
  io.kcb = kcb;
  io.vcb = vcb;
  io.lens = lens;
  io.pages = pages;
  return io;
}

// The records of a C > 1 call inside the caller's workspace.
void carve_records(const AttnPlan& p, void* workspace, ScoreIO& io) {
  char* ws = static_cast<char*>(workspace);
  io.pm = reinterpret_cast<float*>(ws + p.ws_m_off);
  io.pl = reinterpret_cast<float*>(ws + p.ws_l_off);
  io.po = reinterpret_cast<float*>(ws + p.ws_o_off);
}

// One score-kernel launch (the step variant when io.k_new is set).
pq_status launch_score(const AttnPlan& p, const ScoreIO& io, hipStream_t stream,
                       hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
  const bool step = io.k_new != nullptr;
  const PagePlan* pages = io.pages;
  DecodeArgs a{};
  a.q = static_cast<const __half*>(io.q);
  // only the step kernel writes the code arrays (the new token's slot)
  a.k_codes = const_cast<uint8_t*>(io.kc);
  a.v_codes = const_cast<uint8_t*>(io.vc);
  a.k_cb = static_cast<const __half*>(io.kcb);
  a.v_cb = static_cast<const __half*>(io.vcb);
  a.lens = io.lens;
  a.part_m = io.pm;
  a.part_l = io.pl;
  a.part_o = io.po;
  a.out = io.out;
  a.k_new = static_cast<const __half*>(io.k_new);
  a.v_new = static_cast<const __half*>(io.v_new);
  a.counters = io.counters;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Lmax = p.Lmax;
  a.T = p.T;
  a.C = p.C;
  a.hs = p.HS;
  a.qscale = p.scale * kLog2e;
  if (pages != nullptr) {
    a.block_table = pages->block_table;
    a.pool_head_bytes = pages->pool_head_bytes;
    a.page_shift = pages->shift;
    a.max_pages = pages->max_pages;
    a.n_pages = uint32_t(pages->n_pages);
  }
  if (p.R > 1 && !step) {   // request-batched: grid (Hkv, C, request groups)
    DecodeFn fn = pick_mha(p.M, p.T, pages != nullptr);
    if (!fn) return PQ_ERR_UNSUPPORTED;
    return launch(reinterpret_cast<const void*>(fn),
                  dim3(unsigned(p.Hkv), unsigned(p.C), unsigned((p.B + p.R - 1) / p.R)),
                  dim3(kDecodeThreads), &a, stream, start, stop);
  }
  const int cpw = p.CPW;   // the chunk records are the same either way
  DecodeFn fn = pick_decode(p.GW, p.M, p.T, cpw, step, pages != nullptr);
  if (!fn) return PQ_ERR_UNSUPPORTED;
  return launch(reinterpret_cast<const void*>(fn),
                dim3(unsigned(p.Hkv * p.HS), unsigned((p.C + cpw - 1) / cpw), unsigned(p.B)),
                dim3(kDecodeThreads), &a, stream, start, stop);
}

// The new token's K and V codes of a decode step, written by the encode
// kernel at the slot of token lens[b] - 1 (dense or paged cache).
pq_status launch_step_encode(const AttnPlan& p, const PagePlan* pages, const void* k_new,
                             const void* v_new, uint8_t* kc, uint8_t* vc, const void* kcb,
                             const void* vcb, const int32_t* lens, hipStream_t stream,
                             hipEvent_t start) {
  EncodeArgs e{};
  e.x[0] = static_cast<const __half*>(k_new);
  e.x[1] = static_cast<const __half*>(v_new);
  e.cb[0] = static_cast<const __half*>(kcb);
  e.cb[1] = static_cast<const __half*>(vcb);
  e.codes[0] = kc;
  e.codes[1] = vc;
  e.N = p.B;
  e.sxv = int64_t(p.Hkv) * p.D;
  e.sxh = p.D;
  e.scs = p.M;
  e.lens = lens;
  e.Lmax = p.Lmax;
  e.Hkv = p.Hkv;
  if (pages != nullptr) {
    e.sch = pages->pool_head_bytes;
    e.codes_bytes = int64_t(p.Hkv) * pages->pool_head_bytes;
    e.table = pages->block_table;
    e.max_pages = pages->max_pages;
    e.page_shift = pages->shift;
    e.n_pages = uint32_t(pages->n_pages);
  } else {
    e.sch = int64_t(p.Lmax) * p.M;
    e.codes_bytes = int64_t(p.B) * p.Hkv * p.Lmax * p.M;
  }
  const int nv = encode_vectors(p.B, p.Hkv, 2);
  const unsigned tiles = unsigned((p.B + nv - 1) / nv);
  const bool seg = encode_split(p.B, nv, p.Hkv, 2, p.M);
  return launch(encode_fn(p.M, nv, seg), dim3(unsigned(p.Hkv), tiles, seg ? 2u * unsigned(p.M) : 2u),
                dim3(seg ? 128 : 128 * p.M), &e, stream, start, nullptr);
}

pq_status launch_reduce(int64_t rows, int32_t C, const float* pm, const float* pl, const float* po,
                        float* out, hipStream_t stream, hipEvent_t stop = nullptr, bool poly = false) {
  if (rows == 0) return PQ_OK;
  ReduceArgs a{pm, pl, po, out, C};
  const void* fn = poly ? reinterpret_cast<const void*>(&reduce_kernel<kHeadDim, true>)
                        : reinterpret_cast<const void*>(&reduce_kernel<kHeadDim, false>);
  return launch(fn, dim3(unsigned(rows)),
                dim3(kReduceThreads), &a, stream, nullptr, stop);
}

}  // namespace
}  // namespace pqattn

namespace pqattn {
namespace {

// Where a decode step keeps its scratch: the chunk records (carved as in a
// workspace of pq_attn_workspace_bytes from `records`) and the arrival
// counters, B*Hkv 32-bit words that are zero on entry and left zero.
struct StepScratch {
  void* records = nullptr;
  uint32_t* counters = nullptr;
};

// The checks every decode-step entry point makes before anything is
// enqueued (the scratch aside).
pq_status check_step(const pq_attn_desc* desc, const pq_page_table* pages, bool paged,
                     const void* q, const void* k_new, const void* v_new, const uint8_t* k_codes,
                     const uint8_t* v_codes, const void* k_cb, const void* v_cb,
                     const int32_t* lens, const float* out, AttnPlan* p, PagePlan* pg) {
  pq_status st = plan_attn(desc, p);
  if (st != PQ_OK) return st;
  if (paged && (st = plan_pages(*p, pages, pg)) != PQ_OK) return st;
  st = check_attn_pointers(q, k_codes, v_codes, k_cb, v_cb, lens);
  if (st != PQ_OK) return st;
  if (!out || !k_new || !v_new) return PQ_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return PQ_ERR_ALIGN;
  return PQ_OK;
}

// The decode step once checked, with its scratch placed.
pq_status run_step(const AttnPlan& p, const PagePlan* pgp, const void* q, const void* k_new,
                   const void* v_new, uint8_t* k_codes, uint8_t* v_codes, const void* k_cb,
                   const void* v_cb, const int32_t* lens, float* out, const StepScratch& ss,
                   hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  pq_status st;
  ScoreIO io = score_inputs(q, k_codes, v_codes, k_cb, v_cb, lens, pgp);
  if (p.C > 1) carve_records(p, ss.records, io);
  if (p.R > 1) {
    // one query head per KV head and many pairs: the encode kernel writes the
    // new codes, then the request-batched score kernel (and the merge) reads
    // the cache that holds them
    st = launch_step_encode(p, pgp, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, s, e0);
    if (st != PQ_OK) return st;
    if (p.C == 1) {
      io.out = out;
      return launch_score(p, io, s, nullptr, e1);
    }
    st = launch_score(p, io, s);
    if (st != PQ_OK) return st;
    return launch_reduce(p.rows, p.C, io.pm, io.pl, io.po, out, s, e1);
  }
  // one launch: encode, attend and (C > 1) the fused merge
  io.out = out;
  io.k_new = k_new;
  io.v_new = v_new;
  if (p.C > 1) io.counters = ss.counters;
  return launch_score(p, io, s, e0, e1);
}

}  // namespace
}  // namespace pqattn

using namespace pqattn;

extern "C" {

int32_t pq_attn_num_chunks(const pq_attn_desc* desc) {
  AttnPlan p;
  return plan_attn(desc, &p) == PQ_OK ? p.C : -1;
}

size_t pq_attn_workspace_bytes(const pq_attn_desc* desc) {
  AttnPlan p;
  return plan_attn(desc, &p) == PQ_OK ? p.ws_bytes : 0;
}

// pq_attn_decode over a dense cache (pages NULL) or a paged one.
static pq_status attn_decode(const pq_attn_desc* desc, const pq_page_table* pages, const void* q,
                             const uint8_t* k_codes, const uint8_t* v_codes, const void* k_cb,
                             const void* v_cb, const int32_t* lens, float* out, void* workspace,
                             size_t workspace_bytes, void* stream, bool paged) {
  AttnPlan p;
  pq_status st = plan_attn(desc, &p);
  if (st != PQ_OK) return st;
  PagePlan pg;
  if (paged && (st = plan_pages(p, pages, &pg)) != PQ_OK) return st;
  const PagePlan* pgp = paged ? &pg : nullptr;
  st = check_attn_pointers(q, k_codes, v_codes, k_cb, v_cb, lens);
  if (st != PQ_OK) return st;
  if (!out) return PQ_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ScoreIO io = score_inputs(q, k_codes, v_codes, k_cb, v_cb, lens, pgp);
  if (p.C == 1) {
    io.out = out;
    return launch_score(p, io, s);
  }
  if (!workspace || workspace_bytes < p.ws_bytes || !aligned16(workspace)) return PQ_ERR_WORKSPACE;
  carve_records(p, workspace, io);
  st = launch_score(p, io, s);
  if (st != PQ_OK) return st;
  return launch_reduce(p.rows, p.C, io.pm, io.pl, io.po, out, s);
}

pq_status pq_attn_decode(const pq_attn_desc* desc, const void* q, const uint8_t* k_codes,
                         const uint8_t* v_codes, const void* k_cb, const void* v_cb,
                         const int32_t* lens, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return attn_decode(desc, nullptr, q, k_codes, v_codes, k_cb, v_cb, lens, out, workspace,
                     workspace_bytes, stream, false);
}

pq_status pq_attn_decode_paged(const pq_attn_desc* desc, const pq_page_table* pages,
                               const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                               const void* k_cb, const void* v_cb, const int32_t* lens, float* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return attn_decode(desc, pages, q, k_pool, v_pool, k_cb, v_cb, lens, out, workspace,
                     workspace_bytes, stream, true);
}

pq_status pq_attn_partials(const pq_attn_desc* desc, const void* q, const uint8_t* k_codes,
                           const uint8_t* v_codes, const void* k_cb, const void* v_cb,
                           const int32_t* lens, float* part_m, float* part_l, float* part_o,
                           void* stream) {
  AttnPlan p;
  pq_status st = plan_attn(desc, &p);
  if (st != PQ_OK) return st;
  st = check_attn_pointers(q, k_codes, v_codes, k_cb, v_cb, lens);
  if (st != PQ_OK) return st;
  if (!part_m || !part_l || !part_o) return PQ_ERR_NULL;
  ScoreIO io = score_inputs(q, k_codes, v_codes, k_cb, v_cb, lens, nullptr);
  io.pm = part_m;
  io.pl = part_l;
  io.po = part_o;
  return launch_score(p, io, static_cast<hipStream_t>(stream));
}

pq_status pq_attn_partials_paged(const pq_attn_desc* desc, const pq_page_table* pages,
                                 const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                                 const void* k_cb, const void* v_cb, const int32_t* lens,
                                 float* part_m, float* part_l, float* part_o, void* stream) {
  AttnPlan p;
  pq_status st = plan_attn(desc, &p);
  if (st != PQ_OK) return st;
  PagePlan pg;
  if ((st = plan_pages(p, pages, &pg)) != PQ_OK) return st;
  st = check_attn_pointers(q, k_pool, v_pool, k_cb, v_cb, lens);
  if (st != PQ_OK) return st;
  if (!part_m || !part_l || !part_o) return PQ_ERR_NULL;
  ScoreIO io = score_inputs(q, k_pool, v_pool, k_cb, v_cb, lens, &pg);
  io.pm = part_m;
  io.pl = part_l;
  io.po = part_o;
  return launch_score(p, io, static_cast<hipStream_t>(stream));
}

pq_status pq_attn_partials_timed(const pq_attn_desc* desc, const void* q, const uint8_t* k_codes,
                                 const uint8_t* v_codes, const void* k_cb, const void* v_cb,
                                 const int32_t* lens, float* part_m, float* part_l, float* part_o,
                                 void* stream, void* start_event, void* stop_event) {
  AttnPlan p;
  pq_status st = plan_attn(desc, &p);
  if (st != PQ_OK) return st;
  st = check_attn_pointers(q, k_codes, v_codes, k_cb, v_cb, lens);
  if (st != PQ_OK) return st;
  if (!part_m || !part_l || !part_o) return PQ_ERR_NULL;
  ScoreIO io = score_inputs(q, k_codes, v_codes, k_cb, v_cb, lens, nullptr);
  io.pm = part_m;
  io.pl = part_l;
  io.po = part_o;
  return launch_score(p, io, static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                      static_cast<hipEvent_t>(stop_event));
}

size_t pq_attn_step_workspace_bytes(const pq_attn_desc* desc) {
  AttnPlan p;
  return plan_attn(desc, &p) == PQ_OK ? p.ws_step_bytes : 0;
}

// The decode step over a dense cache (pages NULL, paged false) or a paged one,
// its scratch in the caller's workspace.
static pq_status decode_step(const pq_attn_desc* desc, const void* q, const void* k_new,
                             const void* v_new, uint8_t* k_codes, uint8_t* v_codes,
                             const void* k_cb, const void* v_cb, const int32_t* lens, float* out,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* start_event, void* stop_event,
                             const pq_page_table* pages = nullptr, bool paged = false) {
  AttnPlan p;
  PagePlan pg;
  pq_status st = check_step(desc, pages, paged, q, k_new, v_new, k_codes, v_codes, k_cb, v_cb,
                            lens, out, &p, &pg);
  if (st != PQ_OK) return st;
  if (p.C > 1 && (!workspace || workspace_bytes < p.ws_step_bytes || !aligned16(workspace)))
    return PQ_ERR_WORKSPACE;
  StepScratch ss;
  ss.records = workspace;
  if (p.C > 1) ss.counters = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + p.ws_cnt_off);
  return run_step(p, paged ? &pg : nullptr, q, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, out,
                  ss, static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                  static_cast<hipEvent_t>(stop_event));
}

pq_status pq_attn_decode_step(const pq_attn_desc* desc, const void* q, const void* k_new,
                              const void* v_new, uint8_t* k_codes, uint8_t* v_codes,
                              const void* k_cb, const void* v_cb, const int32_t* lens, float* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_step(desc, q, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, out, workspace,
                     workspace_bytes, stream, nullptr, nullptr);
}

pq_status pq_attn_decode_step_timed(const pq_attn_desc* desc, const void* q, const void* k_new,
                                    const void* v_new, uint8_t* k_codes, uint8_t* v_codes,
                                    const void* k_cb, const void* v_cb, const int32_t* lens,
                                    float* out, void* workspace, size_t workspace_bytes,
                                    void* stream, void* start_event, void* stop_event) {
  return decode_step(desc, q, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, out, workspace,
                     workspace_bytes, stream, start_event, stop_event);
}

pq_status pq_attn_decode_step_paged(const pq_attn_desc* desc, const pq_page_table* pages,
                                    const void* q, const void* k_new, const void* v_new,
                                    uint8_t* k_pool, uint8_t* v_pool, const void* k_cb,
                                    const void* v_cb, const int32_t* lens, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_step(desc, q, k_new, v_new, k_pool, v_pool, k_cb, v_cb, lens, out, workspace,
                     workspace_bytes, stream, nullptr, nullptr, pages, true);
}

pq_status pq_attn_decode_step_paged_timed(const pq_attn_desc* desc, const pq_page_table* pages,
                                          const void* q, const void* k_new, const void* v_new,
                                          uint8_t* k_pool, uint8_t* v_pool, const void* k_cb,
                                          const void* v_cb, const int32_t* lens, float* out,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* start_event, void* stop_event) {
  return decode_step(desc, q, k_new, v_new, k_pool, v_pool, k_cb, v_cb, lens, out, workspace,
                     workspace_bytes, stream, start_event, stop_event, pages, true);
}

pq_status pq_attn_reduce(int64_t n_rows, int32_t n_chunks, int32_t head_dim, const float* part_m,
                         const float* part_l, const float* part_o, float* out, void* stream) {
  pq_status st = check_reduce(n_rows, n_chunks, head_dim);
  if (st != PQ_OK) return st;
  if (!part_m || !part_l || !part_o || !out) return PQ_ERR_NULL;
  return launch_reduce(n_rows, n_chunks, part_m, part_l, part_o, out,
                       static_cast<hipStream_t>(stream));
}

pq_status pq_attn_reduce_polyexp(int64_t n_rows, int32_t n_chunks, int32_t head_dim,
                                 const float* part_m, const float* part_l, const float* part_o,
                                 float* out, void* stream) {
  pq_status st = check_reduce(n_rows, n_chunks, head_dim);
  if (st != PQ_OK) return st;
  if (!part_m || !part_l || !part_o || !out) return PQ_ERR_NULL;
  return launch_reduce(n_rows, n_chunks, part_m, part_l, part_o, out,
                       static_cast<hipStream_t>(stream), nullptr, true);
}

}  // extern "C"

namespace pqattn {
namespace {

// The codes' identity places (slot n for vector n) must fit the buffer.
bool identity_places_fit(const pq_encode_desc* d, const EncodePlan& p) {
  if (p.N == 0) return true;
  const double last = double(p.N - 1) * double(d->codes_stride_slot) +
                      double(p.H - 1) * double(d->codes_stride_head) + p.M;
  return last <= double(d->codes_bytes);
}

pq_status encode_planes(const pq_encode_desc* desc, int32_t n, const void* const* x,
                        const void* const* codebook, const int64_t* slots, uint8_t* const* codes,
                        hipStream_t stream) {
  EncodePlan p;
  pq_status st = plan_encode(desc, kEncodeVectors, &p);
  if (st != PQ_OK) return st;
  if (n < 1 || n > kMaxEncodePlanes) return PQ_ERR_SHAPE;
  if (!x || !codebook || !codes) return PQ_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    if (!x[i] || !codebook[i] || !codes[i]) return PQ_ERR_NULL;
    if (!aligned16(x[i]) || !aligned16(codebook[i])) return PQ_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(codes[i]) % p.M) != 0) return PQ_ERR_ALIGN;
  }
  if (p.N == 0) return PQ_OK;
  if (!slots && !identity_places_fit(desc, p)) return PQ_ERR_SHAPE;
  EncodeArgs a{};
  for (int i = 0; i < n; ++i) {
    a.x[i] = static_cast<const __half*>(x[i]);
    a.cb[i] = static_cast<const __half*>(codebook[i]);
    a.codes[i] = codes[i];
  }
  a.slots = slots;
  a.N = p.N;
  a.codes_bytes = desc->codes_bytes;
  a.sxv = desc->x_stride_vec;
  a.sxh = desc->x_stride_head;
  a.scs = desc->codes_stride_slot;
  a.sch = desc->codes_stride_head;
  const int nv = encode_vectors(p.N, p.H, n);
  const unsigned tiles = unsigned((p.N + nv - 1) / nv);   // one-vector-tile launches have < 4,096 tiles
  const bool seg = encode_split(p.N, nv, p.H, n, p.M);
  return launch(encode_fn(p.M, nv, seg), dim3(unsigned(p.H), tiles, seg ? unsigned(n * p.M) : unsigned(n)),
                dim3(seg ? 128 : 128 * p.M), &a, stream);
}

// Checks for the update step: the encode's shape rules, identity places
// that fit the codes buffer, and at most kMaxUpdateVectors vectors.
pq_status check_update(const pq_encode_desc* desc, const void* x, const void* codes,
                       const void* codebook, EncodePlan* p) {
  pq_status st = plan_encode(desc, kEncodeVectors, p);
  if (st != PQ_OK) return st;
  if (p->N > kMaxUpdateVectors) return PQ_ERR_UNSUPPORTED;
  if (!x || !codes || !codebook) return PQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codebook)) return PQ_ERR_ALIGN;
  if (!identity_places_fit(desc, *p)) return PQ_ERR_SHAPE;
  return PQ_OK;
}

pq_status launch_update(const pq_encode_desc* desc, const EncodePlan& p, const void* x,
                        const uint8_t* codes, void* codebook, uint32_t* counts, hipStream_t stream) {
  UpdateArgs a{};
  a.x = static_cast<const __half*>(x);
  a.codes = codes;
  a.cb = static_cast<__half*>(codebook);
  a.counts = counts;
  a.N = p.N;
  a.sxv = desc->x_stride_vec;
  a.sxh = desc->x_stride_head;
  a.scs = desc->codes_stride_slot;
  a.sch = desc->codes_stride_head;
  const void* fn = p.M == 4 ? reinterpret_cast<const void*>(&codebook_update_kernel<4>)
                            : reinterpret_cast<const void*>(&codebook_update_kernel<8>);
  return launch(fn, dim3(unsigned(p.M), unsigned(p.H)), dim3(kUpdateThreads), &a, stream);
}

// Lloyd runs for n (1..kMaxKmeansPlanes) samples of one shape: one launch
// when the sample fits the fused kernel, else encode and update launches per
// iteration and plane.
pq_status kmeans_planes(const pq_encode_desc* desc, int32_t n, const void* const* x,
                        void* const* codebook, int32_t n_iter, uint8_t* const* codes,
                        hipStream_t stream) {
  if (n < 1 || n > kMaxKmeansPlanes) return PQ_ERR_SHAPE;
  if (!x || !codebook || !codes) return PQ_ERR_NULL;
  EncodePlan p;
  for (int i = 0; i < n; ++i) {
    pq_status st = check_update(desc, x[i], codes[i], codebook[i], &p);
    if (st != PQ_OK) return st;
    if ((reinterpret_cast<uintptr_t>(codes[i]) % p.M) != 0) return PQ_ERR_ALIGN;
  }
  if (n_iter < 0) return PQ_ERR_SHAPE;
  if (p.N == 0) return PQ_OK;
  if (p.N <= kMaxFusedVectors) {
    KmeansArgs a{};
    for (int i = 0; i < n; ++i) {
      a.x[i] = static_cast<const __half*>(x[i]);
      a.cb[i] = static_cast<__half*>(codebook[i]);
      a.codes[i] = codes[i];
    }
    a.N = p.N;
    a.sxv = desc->x_stride_vec;
    a.sxh = desc->x_stride_head;
    a.scs = desc->codes_stride_slot;
    a.sch = desc->codes_stride_head;
    a.codes_bytes = desc->codes_bytes;
    a.n_iter = n_iter;
    const void* fn = p.M == 4 ? reinterpret_cast<const void*>(&kmeans_kernel<4>)
                              : reinterpret_cast<const void*>(&kmeans_kernel<8>);
    return launch(fn, dim3(unsigned(p.M), unsigned(p.H), unsigned(n)), dim3(kKmeansThreads), &a,
                  stream);
  }
  for (int i = 0; i < n; ++i) {
    const void* cb = codebook[i];
    for (int32_t it = 0; it <= n_iter; ++it) {
      pq_status st = encode_planes(desc, 1, &x[i], &cb, nullptr, &codes[i], stream);
      if (st != PQ_OK) return st;
      if (it == n_iter) break;
      st = launch_update(desc, p, x[i], codes[i], codebook[i], nullptr, stream);
      if (st != PQ_OK) return st;
    }
  }
  return PQ_OK;
}

}  // namespace
}  // namespace pqattn

extern "C" {

pq_status pq_codebook_update(const pq_encode_desc* desc, const void* x, const uint8_t* codes,
                             void* codebook, uint32_t* counts, void* stream) {
  EncodePlan p;
  pq_status st = check_update(desc, x, codes, codebook, &p);
  if (st != PQ_OK) return st;
  return launch_update(desc, p, x, codes, codebook, counts, static_cast<hipStream_t>(stream));
}

pq_status pq_kmeans(const pq_encode_desc* desc, const void* x, void* codebook, int32_t n_iter,
                    uint8_t* codes, void* stream) {
  return kmeans_planes(desc, 1, &x, &codebook, n_iter, &codes, static_cast<hipStream_t>(stream));
}

pq_status pq_kmeans_many(const pq_encode_desc* desc, int32_t n, const void* const* x,
                         void* const* codebook, int32_t n_iter, uint8_t* const* codes,
                         void* stream) {
  return kmeans_planes(desc, n, x, codebook, n_iter, codes, static_cast<hipStream_t>(stream));
}

pq_status pq_encode(const pq_encode_desc* desc, const void* x, const void* codebook,
                    const int64_t* slots, uint8_t* codes, void* stream) {
  return encode_planes(desc, 1, &x, &codebook, slots, &codes, static_cast<hipStream_t>(stream));
}

pq_status pq_encode_many(const pq_encode_desc* desc, int32_t n, const void* const* x,
                         const void* const* codebook, const int64_t* slots,
                         uint8_t* const* codes, void* stream) {
  return encode_planes(desc, n, x, codebook, slots, codes, static_cast<hipStream_t>(stream));
}

const char* pq_status_string(pq_status status) { return status_string(status); }

}  // extern "C"

// ---- The decode step for callers that cannot allocate ----------------------
// Its scratch (arrival counters, then chunk records) is a file-scope device
// array of fixed size instead of a caller's workspace.  In host code the
// array's name stands for a host-side shadow, not a device address: the
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever handed to a kernel.
namespace pqattn {
namespace {

constexpr size_t kNoAllocCounters = 65536;                    // B * Hkv at most
constexpr size_t kNoAllocCounterBytes = kNoAllocCounters * 4;  // 256 KiB
constexpr size_t kNoAllocRecordBytes = size_t(8) << 20;       // chunk records, 8 MiB at most
constexpr int kNoAllocMaxDevices = 64;

}  // namespace
}  // namespace pqattn

static __device__ __align__(256) unsigned char scratch[pqattn::kNoAllocCounterBytes +
                                                       pqattn::kNoAllocRecordBytes];

namespace pqattn {
namespace {

__global__ void zero_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

std::mutex g_scratch_mu;
void* g_scratch[kNoAllocMaxDevices];   // device address of `scratch` per device, once set up

// The current device's scratch address.  The first call on a device takes
// the address with hipGetSymbolAddress and zeroes the counters with a fill
// kernel on `stream` (no memset node, so the call can be captured); every
// later step leaves them at zero again.
pq_status device_scratch(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PQ_ERR_HIP;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return PQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return PQ_ERR_HIP;
    uint32_t* counters = static_cast<uint32_t*>(ptr);
    uint32_t n = uint32_t(kNoAllocCounters);
    void* args[] = {&counters, &n};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&zero_words_kernel), dim3(64), dim3(256), args,
                        0, stream) != hipSuccess)
      return PQ_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch[dev]);
  return PQ_OK;
}

}  // namespace
}  // namespace pqattn

extern "C" {

pq_status pq_attn_decode_step_noalloc(const pq_attn_desc* desc, const void* q, const void* k_new,
                                      const void* v_new, uint8_t* k_codes, uint8_t* v_codes,
                                      const void* k_cb, const void* v_cb, const int32_t* lens,
                                      float* out, void* stream) {
  AttnPlan p;
  PagePlan pg;
  pq_status st = check_step(desc, nullptr, false, q, k_new, v_new, k_codes, v_codes, k_cb, v_cb,
                            lens, out, &p, &pg);
  if (st != PQ_OK) return st;
  if (size_t(p.B) * size_t(p.Hkv) * size_t(p.HS) > kNoAllocCounters || p.ws_bytes > kNoAllocRecordBytes)
    return PQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = nullptr;
  if ((st = device_scratch(s, &base)) != PQ_OK) return st;
  StepScratch ss;
  ss.counters = reinterpret_cast<uint32_t*>(base);
  ss.records = base + kNoAllocCounterBytes;
  return run_step(p, nullptr, q, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, out, ss, s,
                  nullptr, nullptr);
}

}  // extern "C"
