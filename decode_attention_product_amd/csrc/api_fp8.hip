// C entry points for FP8 (OCP E4M3) codebooks (declared in include/pqattn.h):
// the AQPIM page, section 4.2, keeps the codebooks in a low-precision float
// such as FP8.  The kernels are the fp16 ones with the codebook operands
// converted on load (every E4M3 value is an fp16 value), instantiated here
// in a translation unit of their own so the two builds compile in parallel.
#include <hip/hip_runtime.h>

#include "decode_kernel.hpp"
#include "encode_kernel.hpp"
#include "plan.h"
#include "pqattn.h"

namespace pqattn {
namespace {

constexpr CbFmt kF8 = CbFmt::E4M3;
constexpr int kEncodeVectorsF8 = 256;
constexpr int kEncodeVectorsF8Small = 16;
constexpr int64_t kEncodeCUsF8 = 256;

using DecodeFn = void (*)(DecodeArgs);

template <int G, int M>
DecodeFn pick_nt_f8(int T) {
  if (T <= kDecodeThreads) return &decode_partials_kernel<G, M, 1, false, 1, kF8>;
  if (T <= 2 * kDecodeThreads) return &decode_partials_kernel<G, M, 2, false, 1, kF8>;
  if (T <= 4 * kDecodeThreads) return &decode_partials_kernel<G, M, 4, false, 1, kF8>;
  if constexpr (G <= 2) {
    if (T <= 8 * kDecodeThreads) return &decode_partials_kernel<G, M, 8, false, 1, kF8>;
  }
  return nullptr;
}

DecodeFn pick_decode_f8(int G, int M, int T) {
  switch (M * 16 + G) {
    case 4 * 16 + 1: return pick_nt_f8<1, 4>(T);
    case 4 * 16 + 2: return pick_nt_f8<2, 4>(T);
    case 4 * 16 + 4: return pick_nt_f8<4, 4>(T);
    case 4 * 16 + 8: return pick_nt_f8<8, 4>(T);
    case 8 * 16 + 1: return pick_nt_f8<1, 8>(T);
    case 8 * 16 + 2: return pick_nt_f8<2, 8>(T);
    case 8 * 16 + 4: return pick_nt_f8<4, 8>(T);
    case 8 * 16 + 8: return pick_nt_f8<8, 8>(T);
  }
  return nullptr;
}

pq_status launch_f8(const void* fn, dim3 grid, dim3 block, void* arg, hipStream_t stream) {
  void* args[] = {arg};
  return hipLaunchKernel(fn, grid, block, args, 0, stream) == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

// The checked plan of an FP8-codebook call: the per-request score kernel
// with one chunk per workgroup (the request-batched kernel and two-chunk
// workgroups are built for fp16 codebooks only); the chunking and the head
// split, and so the workspace size, are those of the fp16 call with the
// same descriptor.
pq_status plan_f8(const pq_attn_desc* desc, const void* q, const uint8_t* kc, const uint8_t* vc,
                  const uint8_t* kcb, const uint8_t* vcb, const int32_t* lens, AttnPlan* p) {
  pq_status st = plan_attn(desc, p);
  if (st != PQ_OK) return st;
  if (!q || !kc || !vc || !kcb || !vcb || !lens) return PQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(kcb) || !aligned16(vcb))
    return PQ_ERR_ALIGN;
  p->R = 1;
  p->CPW = 1;
  return PQ_OK;
}

pq_status launch_score_f8(const AttnPlan& p, const void* q, const uint8_t* kc, const uint8_t* vc,
                          const uint8_t* kcb, const uint8_t* vcb, const int32_t* lens, float* pm,
                          float* pl, float* po, float* out, hipStream_t stream) {
  DecodeFn fn = pick_decode_f8(p.GW, p.M, p.T);
  if (!fn) return PQ_ERR_UNSUPPORTED;
  DecodeArgs a{};
  a.q = static_cast<const __half*>(q);
  a.k_codes = const_cast<uint8_t*>(kc);   // read only: the plain decode writes no codes
  a.v_codes = const_cast<uint8_t*>(vc);
  a.k_cb = kcb;
  a.v_cb = vcb;
  a.lens = lens;
  a.part_m = pm;
  a.part_l = pl;
  a.part_o = po;
  a.out = out;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Lmax = p.Lmax;
  a.T = p.T;
  a.C = p.C;
  a.hs = p.HS;
  a.qscale = p.scale * kLog2e;
  return launch_f8(reinterpret_cast<const void*>(fn), dim3(unsigned(p.Hkv * p.HS), unsigned(p.C), unsigned(p.B)),
                   dim3(kDecodeThreads), &a, stream);
}

}  // namespace
}  // namespace pqattn

using namespace pqattn;

extern "C" {

pq_status pq_attn_decode_fp8cb(const pq_attn_desc* desc, const void* q, const uint8_t* k_codes,
                               const uint8_t* v_codes, const uint8_t* k_cb, const uint8_t* v_cb,
                               const int32_t* lens, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  AttnPlan p;
  pq_status st = plan_f8(desc, q, k_codes, v_codes, k_cb, v_cb, lens, &p);
  if (st != PQ_OK) return st;
  if (!out) return PQ_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.C == 1)
    return launch_score_f8(p, q, k_codes, v_codes, k_cb, v_cb, lens, nullptr, nullptr, nullptr, out, s);
  if (!workspace || workspace_bytes < p.ws_bytes || !aligned16(workspace)) return PQ_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* pm = reinterpret_cast<float*>(ws + p.ws_m_off);
  float* pl = reinterpret_cast<float*>(ws + p.ws_l_off);
  float* po = reinterpret_cast<float*>(ws + p.ws_o_off);
  st = launch_score_f8(p, q, k_codes, v_codes, k_cb, v_cb, lens, pm, pl, po, nullptr, s);
  if (st != PQ_OK) return st;
  return pq_attn_reduce(p.rows, p.C, p.D, pm, pl, po, out, stream);
}

pq_status pq_attn_partials_fp8cb(const pq_attn_desc* desc, const void* q, const uint8_t* k_codes,
                                 const uint8_t* v_codes, const uint8_t* k_cb, const uint8_t* v_cb,
                                 const int32_t* lens, float* part_m, float* part_l, float* part_o,
                                 void* stream) {
  AttnPlan p;
  pq_status st = plan_f8(desc, q, k_codes, v_codes, k_cb, v_cb, lens, &p);
  if (st != PQ_OK) return st;
  if (!part_m || !part_l || !part_o) return PQ_ERR_NULL;
  return launch_score_f8(p, q, k_codes, v_codes, k_cb, v_cb, lens, part_m, part_l, part_o, nullptr,
                         static_cast<hipStream_t>(stream));
}

pq_status pq_encode_fp8cb(const pq_encode_desc* desc, const void* x, const uint8_t* codebook,
                          const int64_t* slots, uint8_t* codes, void* stream) {
  EncodePlan p;
  pq_status st = plan_encode(desc, kEncodeVectorsF8, &p);
  if (st != PQ_OK) return st;
  if (!x || !codebook || !codes) return PQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codebook)) return PQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(codes) % p.M) != 0) return PQ_ERR_ALIGN;
  if (p.N == 0) return PQ_OK;
  if (!slots) {   // identity places (slot n for vector n) must fit the buffer
    const double last = double(p.N - 1) * double(desc->codes_stride_slot) +
                        double(p.H - 1) * double(desc->codes_stride_head) + p.M;
    if (last > double(desc->codes_bytes)) return PQ_ERR_SHAPE;
  }
  EncodeArgs a{};
  a.x[0] = static_cast<const __half*>(x);
  a.cb[0] = codebook;
  a.codes[0] = codes;
  a.slots = slots;
  a.N = p.N;
  a.codes_bytes = desc->codes_bytes;
  a.sxv = desc->x_stride_vec;
  a.sxh = desc->x_stride_head;
  a.scs = desc->codes_stride_slot;
  a.sch = desc->codes_stride_head;
  // 256-vector workgroups, or one 16-vector tile each when those would
  // leave CUs idle (as for fp16 codebooks)
  const int64_t big = (p.N + kEncodeVectorsF8 - 1) / kEncodeVectorsF8;
  const int nv = big * p.H < kEncodeCUsF8 ? kEncodeVectorsF8Small : kEncodeVectorsF8;
  const void* fn;
  const unsigned tiles = unsigned((p.N + nv - 1) / nv);
  // one segment per workgroup when that still fits the CUs in one round (as
  // for fp16 codebooks)
  const bool seg = nv == kEncodeVectorsF8Small && int64_t(tiles) * p.H * p.M <= kEncodeCUsF8;
  if (seg)
    fn = p.M == 4 ? reinterpret_cast<const void*>(&encode_kernel<4, kEncodeVectorsF8Small, kF8, true>)
                  : reinterpret_cast<const void*>(&encode_kernel<8, kEncodeVectorsF8Small, kF8, true>);
  else if (nv == kEncodeVectorsF8Small)
    fn = p.M == 4 ? reinterpret_cast<const void*>(&encode_kernel<4, kEncodeVectorsF8Small, kF8>)
                  : reinterpret_cast<const void*>(&encode_kernel<8, kEncodeVectorsF8Small, kF8>);
  else
    fn = p.M == 4 ? reinterpret_cast<const void*>(&encode_kernel<4, kEncodeVectorsF8, kF8>)
                  : reinterpret_cast<const void*>(&encode_kernel<8, kEncodeVectorsF8, kF8>);
  return launch_f8(fn, dim3(unsigned(p.H), tiles, seg ? unsigned(p.M) : 1u), dim3(seg ? 128 : 128 * p.M), &a,
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
