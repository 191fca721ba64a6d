// Fused PQ decode-attention score kernel and chunk-merge kernel (gfx950).
//
// One workgroup of 1024 threads owns one (request b, KV head g, chunk c) and
// the G query heads that share g (grouped-query attention, memory-wall
// chapter section 1.4.3 (1)).  The codes come from a dense cache
// [B][Hkv][Lmax][M] or from a paged one (decode_paged_kernel): per-head
// pools of P-token pages and a block table naming the page of every P
// tokens of a request (AQPIM page, section 5.1 (4); PAM page, section
// 2.2.2 (2)).  Steps:
//
//   0. The operands are requested in the order they are used: q and the K
//      codebook (table build) before lens[b] is even waited for, then the
//      chunk's K codes (with several token slots per thread, once the
//      codebook is in); once the table is built, the V codes; and inside the
//      histogram, the V codebook operands of the contraction.
//   1. Lookup table LUT[m][k][h] = q_h[m] . Ck_g[m][k] -- the query's partial
//      dot product with every K codeword (AQPIM page, section 4.1; kept on
//      chip as the page's GPU note suggests) -- computed as M small
//      [G x DS] x [DS x 256] products on the matrix cores (fp16 inputs,
//      exact products, fp32 sums), scaled by scale*log2(e) and stored in LDS.
//   2. Scores: per token and head, the sum over m of LUT[m][code_m][h]; the
//      K vectors are never rebuilt.
//   3. Chunk max m_c and p_t = 2^(s_t - m_c) <= 1 (PAM page, section
//      2.2.3 (1)).
//   4. V histogram Hist[m][k][h] = sum of p_t over the chunk's tokens whose
//      segment-m V code is k.  LDS float atomics are slow on gfx950, so p is
//      added as a 32-bit fixed-point integer, two heads per 64-bit
//      ds_add_u64.  The scale 2^S of a (chunk, head) comes from the chunk's
//      mass: an upper estimate of l_c = sum_t p_t (one reduction) sets
//      S = 30 - ceil(log2 l_c), so the bins of a segment, which add up to
//      about l_c * 2^S, stay below 2^31 whatever the score distribution, and
//      a chunk dominated by one token keeps ~29 bits for the rest.  Every
//      token lands in exactly one bin of segment 0, so the l_c of the record
//      is the integer sum of those bins: exact, and the same quantised p
//      that the contraction weights.
//   5. Contraction o[h][m*DS + j] = sum_k Hist[m][k][h] * Cv_g[m][k][j] on
//      the matrix cores.  This equals sum_t p_t V_t because every V_t is
//      made of codewords.  The histogram enters as fp16 hi + lo parts, so
//      the product keeps about 22 bits of the fp32 bin value.
//   6. (m_c, l_c, o_c) is written for the merge, or o_c / l_c when the whole
//      cache is one chunk.
// Scores are in base-2 units (q . C times scale*log2(e)) so exponentials are
// single v_exp_f32 instructions; m is written back in natural-log units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace pqattn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDecodeThreads = 1024;

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Codebook element formats: fp16, or the 8-bit OCP FP8 E4M3 format (sign,
// 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities;
// bytes 0x7F and 0xFF are NaN and are not valid codebook entries) for the
// low-precision codebooks of the AQPIM page, section 4.2.  Every E4M3 value
// is an fp16 value, so the kernels convert on load and from there on run
// the fp16 arithmetic unchanged: an FP8 codebook gives exactly the results
// of its fp16 upcast.
enum class CbFmt { F16, E4M3 };

// Two E4M3 bytes (bits 0-7 and 8-15 of w) as two fp16 values, by gfx950's
// packed FP8 conversion with a scale of 1 (every E4M3 value, subnormals
// included, is an fp16 value, so the conversion is exact).
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
// Four E4M3 bytes (little-endian in w) as four fp16 values.
__device__ __forceinline__ f16x4 e4m3x4_to_f16x4(uint32_t w) {
  const uint32_t lo = e4m3x2_to_f16x2(w);
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  return __builtin_bit_cast(f16x4, make_uint2(lo, hi));
}
// Codebook elements e .. e+3 (e a multiple of 4) as fp16.
template <CbFmt F>
__device__ __forceinline__ f16x4 cb_load4(const void* base, int64_t e) {
  if constexpr (F == CbFmt::F16) return *reinterpret_cast<const f16x4*>(static_cast<const _Float16*>(base) + e);
  else return e4m3x4_to_f16x4(*reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(base) + e));
}
// Codebook element e as fp16.
template <CbFmt F>
__device__ __forceinline__ _Float16 cb_load1(const void* base, int64_t e) {
  if constexpr (F == CbFmt::F16) return static_cast<const _Float16*>(base)[e];
  else return __builtin_bit_cast(f16x2, e4m3x2_to_f16x2(static_cast<const uint8_t*>(base)[e]))[0];
}

struct DecodeArgs {
  const __half* q;           // [B][Hq][D]
  uint8_t* k_codes;          // [B][Hkv][Lmax][M]; written only by the step
  uint8_t* v_codes;          //   kernel, at the new token's slot
  const void* k_cb;          // [Hkv][M][K][DS], fp16 or E4M3 (the kernel's CbFmt)
  const void* v_cb;
  const int32_t* lens;       // [B]
  float* part_m;             // [B*Hq][C]     chunk records; all three null:
  float* part_l;             // [B*Hq][C]     the normalised output is written
  float* part_o;             // [B*Hq][C][D]  directly (C == 1)
  float* out;                // [B*Hq][D]
  const __half* k_new;       // [B][Hkv][D] the new token's K and V (step kernel)
  const __half* v_new;
  uint32_t* counters;        // [B*Hkv] chunk arrivals (step kernel with C > 1):
                             // zero on entry, zero again on exit
  int32_t B, Hq, Hkv, Lmax, T, C;
  int32_t hs;                // head split: workgroups sharing one (b, KV head, chunk),
                             // each taking G of its Hq / Hkv query heads (grid x
                             // = hs * Hkv; counters [B*Hkv*hs])
  float qscale;              // scale * log2(e)
  // Paged cache only: k_codes and v_codes are pools [Hkv][n_pages][P][M] and
  // token t of request b lives at slot block_table[b][t >> page_shift] * P +
  // (t & (P - 1)) of its KV head's pool.  Lmax = max_pages * P.
  const int32_t* block_table;  // [B][max_pages]
  int64_t pool_head_bytes;     // n_pages * P * M
  int32_t page_shift;          // log2(P)
  int32_t max_pages;
  uint32_t n_pages;            // page ids are clamped to [0, n_pages)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x by the reduction unit's method of the PAM page, section 3.2.2 (1): a
// 6th-order polynomial in place of an exponential unit.  x = n + f with
// n = floor(x), f in [0, 1); 2^f from a degree-6 minimax polynomial (Horner,
// fp32; coefficients from exp2_poly_fit.py, Remez exchange on relative
// error: 8.4e-8 at most in fp32), then 2^n through the exponent field.
// x below -126 (a merge weight under 2^-126) gives 0; -inf gives 0.
__device__ __forceinline__ float poly_exp2(float x) {
  constexpr float c0 = 1.000000000e+00f, c1 = 6.931470037e-01f, c2 = 2.402298301e-01f,
                  c3 = 5.548334122e-02f, c4 = 9.678840637e-03f, c5 = 1.243968727e-03f,
                  c6 = 2.170225489e-04f;
  if (!(x >= -126.0f)) return 0.0f;
  const float n = __builtin_floorf(x);
  const float f = x - n;
  float p = fmaf(c6, f, c5);
  p = fmaf(p, f, c4);
  p = fmaf(p, f, c3);
  p = fmaf(p, f, c2);
  p = fmaf(p, f, c1);
  p = fmaf(p, f, c0);
  return __builtin_ldexpf(p, int(n));
}

// The merge's exponential: the hardware's, or the polynomial above.
template <bool POLY>
__device__ __forceinline__ float merge_exp2(float x) {
  if constexpr (POLY) return poly_exp2(x);
  else return fast_exp2(x);
}

// log2 of a power of two (compile time)
constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// IEEE-754 maximum (v_maximum_f32 / v_maximum3_f32).  fmaxf lowers to maxnum,
// which first quiets both operands with two extra v_max instructions; the
// values here are never NaN, and maximum is exact on them and on +-inf.
__device__ __forceinline__ float max_f(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// DPP lane moves inside a row of 16 lanes (no LDS traffic).  Every source
// lane of the patterns used is valid, so bound_ctrl changes no value; it
// lets the compiler fold the move into the VALU instruction that uses it.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;   // quad_perm(2,3,0,1)
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

// v[l] + v[l ^ 16] and v[l] + v[l ^ 32] in every lane l: the lane-swap
// instructions return the pair (v[l & ~m], v[l | m]) in their two outputs,
// and their sum is the same float in both lanes of the pair (VALU only, no
// LDS traffic).
__device__ __forceinline__ float pair_sum16(float v) {
  const int b = __builtin_bit_cast(int, v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return __builtin_bit_cast(float, int(r[0])) + __builtin_bit_cast(float, int(r[1]));
}
__device__ __forceinline__ float pair_sum32(float v) {
  const int b = __builtin_bit_cast(int, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, int(r[0])) + __builtin_bit_cast(float, int(r[1]));
}

// Max of N values over each row of 16 lanes (every lane of the row receives
// its row's results): DPP only, no cross-row steps.
template <int N>
__device__ __forceinline__ void row_max_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float x = v[i];
    x = max_f(x, dpp_f<kDppXor1>(x));
    x = max_f(x, dpp_f<kDppXor2>(x));
    x = max_f(x, dpp_f<kDppRor4>(x));
    x = max_f(x, dpp_f<kDppRor8>(x));
    v[i] = x;
  }
}

// Sum of N values over each row of 16 lanes (every lane of the row receives
// its row's sums), as row_max_n.
template <int N>
__device__ __forceinline__ void row_sum_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float x = v[i];
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppRor4>(x);
    x += dpp_f<kDppRor8>(x);
    v[i] = x;
  }
}

// Fixed point of the V histogram.  A (chunk, head) adds u_t = round(p_t 2^S)
// per token, p_t = 2^(s_t - m_c) <= 1, into 32-bit bins.  S comes from an
// upper estimate of the chunk's mass l_c = sum_t p_t, accumulated as
// kMassBits fixed-point integers rounded up (lest = ceil-sums of l_c 2^16):
// S = 30 - ceil(log2 l_c), clamped to [14, 30].  Then the u_t of a segment
// sum to at most l_c 2^S + T/2 <= 2^30 + 2^11 < 2^31, so no bin and no
// integer sum of bins overflows; a chunk whose mass is one dominant token
// gets S = 29 or 30.  l_c >= 1 always (the maximum token has p = 1).
constexpr int kMassBits = 16;
__device__ __forceinline__ int fix_shift(uint32_t lest) {
  const uint32_t x = lest > (1u << kMassBits) ? lest - 1u : (1u << kMassBits) - 1u;
  return 30 - kMassBits + __builtin_clz(x);   // 30 - ceil(log2(lest 2^-16))
}
// 2^e as a float, for |e| < 127
__device__ __forceinline__ float pow2i(int e) { return __builtin_bit_cast(float, uint32_t(127 + e) << 23); }
// one row's mass estimate as a rounded-up fixed-point integer
__device__ __forceinline__ uint32_t mass_fix(float row_sum) {
  return uint32_t(__builtin_ceilf(row_sum * float(1u << kMassBits)));
}

// Float <-> int keys whose signed order is the float order (finite values
// and infinities), so an LDS integer max can reduce float maxima.
__device__ __forceinline__ int float_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float key_float(int k) {
  return __builtin_bit_cast(float, k >= 0 ? k : k ^ 0x7fffffff);
}

template <int CTRL>
__device__ __forceinline__ int dpp_int(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}

// (score, index) -> the better of the pair and its DPP partner: the larger
// score, or on equal scores the lower index.
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& s, int& k) {
  const float os = dpp_f<CTRL>(s);
  const int ok = dpp_int<CTRL>(k);
  // bitwise, not short-circuit: three compares and two mask operations, no
  // branches
  const bool take = (os > s) | ((os == s) & (ok < k));
  s = take ? os : s;
  k = take ? ok : k;
}

// The same across rows: lanes l and l ^ 16 (resp. l ^ 32) both end with the
// better (score, index) of the two, taken from the lane-swap pair.
__device__ __forceinline__ void argmax_pick(float& s, int& k, float s0, int k0, float s1, int k1) {
  const bool one = (s1 > s0) | ((s1 == s0) & (k1 < k0));
  s = one ? s1 : s0;
  k = one ? k1 : k0;
}
__device__ __forceinline__ void argmax_pair16(float& s, int& k) {
  const auto rs = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, s), __builtin_bit_cast(int, s), false, false);
  const auto rk = __builtin_amdgcn_permlane16_swap(k, k, false, false);
  argmax_pick(s, k, __builtin_bit_cast(float, int(rs[0])), int(rk[0]), __builtin_bit_cast(float, int(rs[1])), int(rk[1]));
}
__device__ __forceinline__ void argmax_pair32(float& s, int& k) {
  const auto rs = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, s), __builtin_bit_cast(int, s), false, false);
  const auto rk = __builtin_amdgcn_permlane32_swap(k, k, false, false);
  argmax_pick(s, k, __builtin_bit_cast(float, int(rs[0])), int(rk[0]), __builtin_bit_cast(float, int(rs[1])), int(rk[1]));
}

// 64-bit key whose unsigned order is (score, then lower index): the integer
// LDS max of keys is the argmax with the lowest index among equal scores.
// Adding +0 turns a -0 score into +0, so the two zeros count as equal here
// as they do in the float compares.
__device__ __forceinline__ unsigned long long argmax_key(float score, int k) {
  const uint32_t hi = uint32_t(float_key(score + 0.0f)) ^ 0x80000000u;
  return (static_cast<unsigned long long>(hi) << 32) | uint32_t(255 - k);
}
__device__ __forceinline__ int argmax_key_index(unsigned long long key) {
  return 255 - int(key & 0xffu);
}

// Chunk-record access.  COH: agent-scope (device-coherent) atomic stores and
// loads, which the chip keeps coherent across its per-XCD L2 caches without
// cache writebacks or invalidations; used where one workgroup reads records
// that others wrote in the same launch.
template <bool COH>
__device__ __forceinline__ void rec_store(float* p, float v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ float rec_load(const float* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Merge of one output element over C chunk records (m in natural-log units):
//   sum_c w_c o_c / sum_c w_c l_c,  w_c = exp(m_c - max_c m_c),
// 0 when every chunk is empty (m = -inf, l = 0).
template <bool COH = false, bool POLY = false>
__device__ __forceinline__ float merge_chunks(const float* pm, const float* pl, const float* po,
                                              int C, int stride_o) {
  constexpr int kFew = 8;   // up to this many chunks: every record load issued at once
  float m_star = -INFINITY, num = 0.0f, den = 0.0f;
  if (C <= kFew) {
    float m[kFew], l[kFew], o[kFew];
#pragma unroll
    for (int c = 0; c < kFew; ++c) {
      m[c] = c < C ? rec_load<COH>(pm + c) : -INFINITY;
      l[c] = c < C ? rec_load<COH>(pl + c) : 0.0f;
      o[c] = c < C ? rec_load<COH>(po + int64_t(c) * stride_o) : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < kFew; ++c) m_star = max_f(m_star, m[c]);
    if (m_star != -INFINITY) {
#pragma unroll
      for (int c = 0; c < kFew; ++c) {
        if (m[c] == -INFINITY) continue;
        const float w = merge_exp2<POLY>((m[c] - m_star) * kLog2e);
        num = fmaf(w, o[c], num);
        den = fmaf(w, l[c], den);
      }
    }
  } else {
    // one pass in batches of kFew records, all of a batch's loads issued
    // together; the running sums are rescaled when the running max grows
    for (int c0 = 0; c0 < C; c0 += kFew) {
      float m[kFew], l[kFew], o[kFew];
#pragma unroll
      for (int j = 0; j < kFew; ++j) {
        const int c = c0 + j;
        m[j] = c < C ? rec_load<COH>(pm + c) : -INFINITY;
        l[j] = c < C ? rec_load<COH>(pl + c) : 0.0f;
        o[j] = c < C ? rec_load<COH>(po + int64_t(c) * stride_o) : 0.0f;
      }
      float mb = m_star;
#pragma unroll
      for (int j = 0; j < kFew; ++j) mb = max_f(mb, m[j]);
      if (mb == -INFINITY) continue;
      const float r = merge_exp2<POLY>((m_star - mb) * kLog2e);   // 0 while m_star = -inf
      num *= r;
      den *= r;
#pragma unroll
      for (int j = 0; j < kFew; ++j) {
        if (m[j] == -INFINITY) continue;
        const float w = merge_exp2<POLY>((m[j] - mb) * kLog2e);
        num = fmaf(w, o[j], num);
        den = fmaf(w, l[j], den);
      }
      m_star = mb;
    }
  }
  return den > 0.0f ? num / den : 0.0f;
}

// Arrival count for one (request, KV head), called by every thread of a
// workgroup after its chunk records have been stored with rec_store<true>;
// C is the number of workgroups that arrive (one per CPW chunks).
// Memory model: the records are relaxed agent-scope atomic stores; the
// workgroup barrier orders every thread's stores before thread 0's arrival,
// an agent-scope release fetch-add, which makes the workgroup's records
// visible at agent scope before the count can be seen.  The workgroup whose
// add returns C - 1 (the last to arrive) then issues an agent-scope acquire
// fence: it synchronises with the release of every earlier arrival (each
// add reads the value the previous one wrote), so -- after the second
// barrier -- that workgroup's relaxed agent-scope loads (rec_load<true>)
// see all C records.  Only the merging workgroup pays for the acquire.
// Each wave also waits for its own stores (vmcnt = 0) before the barrier.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int C, uint32_t* flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool last =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == uint32_t(C - 1);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *flag = last ? 1u : 0u;
  }
  __syncthreads();
  return *flag != 0;
}

// Raw buffer resources (gfx9 descriptor word 3: raw dword access) let loads
// be issued by every lane without a branch: a lane whose byte offset lies
// past num_records gets 0 and makes no memory access.  Branch-free loads
// also let the compiler count outstanding loads exactly, so a wait for an
// early load (a codebook operand) does not wait for later ones (the codes).
constexpr int kRsrcRaw = 0x00020000;
constexpr uint32_t kOffNone = 0x80000000u;   // an offset past any buffer used here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), kRsrcRaw);
}

// Code bytes of one token: M = 4 -> one dword, M = 8 -> two dwords.
template <int M> struct TokenCodes;
template <> struct TokenCodes<4> {
  uint32_t w = 0;
  __device__ __forceinline__ void set(const int* c) {
    w = uint32_t(c[0]) | (uint32_t(c[1]) << 8) | (uint32_t(c[2]) << 16) | (uint32_t(c[3]) << 24);
  }
  __device__ __forceinline__ void store(uint8_t* p) const { *reinterpret_cast<uint32_t*>(p) = w; }
  __device__ __forceinline__ void load(const uint8_t* p) { w = *reinterpret_cast<const uint32_t*>(p); }
  // from a raw buffer (byte offset; out of range reads 0 and touches no memory)
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    w = uint32_t(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
  __device__ __forceinline__ int get(int m) const { return (w >> (8 * m)) & 0xff; }
  // the codes with byte j holding segment (j + r) % 4
  __device__ __forceinline__ TokenCodes rotated(int r) const {
    TokenCodes o;
    o.w = __builtin_amdgcn_alignbit(w, w, 8 * r);
    return o;
  }
};
template <> struct TokenCodes<8> {
  uint2 w = {0, 0};
  __device__ __forceinline__ void set(const int* c) {
    w.x = uint32_t(c[0]) | (uint32_t(c[1]) << 8) | (uint32_t(c[2]) << 16) | (uint32_t(c[3]) << 24);
    w.y = uint32_t(c[4]) | (uint32_t(c[5]) << 8) | (uint32_t(c[6]) << 16) | (uint32_t(c[7]) << 24);
  }
  __device__ __forceinline__ void store(uint8_t* p) const { *reinterpret_cast<uint2*>(p) = w; }
  __device__ __forceinline__ void load(const uint8_t* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w = make_uint2(v[0], v[1]);
  }
  __device__ __forceinline__ int get(int m) const {
    return ((m < 4 ? w.x : w.y) >> (8 * (m & 3))) & 0xff;
  }
  // the codes with byte j holding segment (j + r) % 8: a 64-bit rotation
  __device__ __forceinline__ TokenCodes rotated(int r) const {
    const uint32_t lo = (r & 4) ? w.y : w.x;
    const uint32_t hi = (r & 4) ? w.x : w.y;
    const uint32_t sh = 8 * (r & 3);
    TokenCodes o;
    o.w = make_uint2(__builtin_amdgcn_alignbit(hi, lo, sh), __builtin_amdgcn_alignbit(lo, hi, sh));
    return o;
  }
};

// Lookup-table layout: for G >= 4 the heads of one (segment, codeword) are
// split in quads stored as [m][quad][k] float4 -- 16-byte entries spread a
// random codeword over 8 LDS bank groups (32-byte entries would use 4); for
// G <= 2 the layout is [m][k][G].
template <int G, int K>
__device__ __forceinline__ int lut_index(int m, int k, int quad) {
  if constexpr (G >= 4) return ((m * (G / 4) + quad) * K + k) * 4;
  else return (m * K + k) * G;
}

// Scores of one token: the M * ceil(G/4) table reads are issued before any
// sum so their LDS latencies overlap.
template <int G, int M, int K, typename Codes>
__device__ __forceinline__ void token_scores(const float* lut, const Codes& code, float* s) {
  if constexpr (G >= 4) {
    // in groups of 4 segments: 4 * G/4 reads in flight, half the registers
    // of issuing all M at once
    float4 acc[G / 4];
#pragma unroll
    for (int m0 = 0; m0 < M; m0 += 4) {
      float4 e[4][G / 4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < G / 4; ++v)
          e[m][v] = *reinterpret_cast<const float4*>(lut + lut_index<G, K>(m0 + m, code.get(m0 + m), v));
#pragma unroll
      for (int v = 0; v < G / 4; ++v) {
        if (m0 == 0) acc[v] = e[0][v];
        else { acc[v].x += e[0][v].x; acc[v].y += e[0][v].y; acc[v].z += e[0][v].z; acc[v].w += e[0][v].w; }
#pragma unroll
        for (int m = 1; m < 4; ++m) {
          acc[v].x += e[m][v].x; acc[v].y += e[m][v].y; acc[v].z += e[m][v].z; acc[v].w += e[m][v].w;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < G / 4; ++v) {
      s[4 * v + 0] = acc[v].x; s[4 * v + 1] = acc[v].y; s[4 * v + 2] = acc[v].z; s[4 * v + 3] = acc[v].w;
    }
  } else if constexpr (G == 2) {
    float2 e[M];
#pragma unroll
    for (int m = 0; m < M; ++m) e[m] = *reinterpret_cast<const float2*>(lut + lut_index<G, K>(m, code.get(m), 0));
    float2 acc = e[0];
#pragma unroll
    for (int m = 1; m < M; ++m) { acc.x += e[m].x; acc.y += e[m].y; }
    s[0] = acc.x; s[1] = acc.y;
  } else {
    float e[M];
#pragma unroll
    for (int m = 0; m < M; ++m) e[m] = lut[lut_index<G, K>(m, code.get(m), 0)];
    float acc = e[0];
#pragma unroll
    for (int m = 1; m < M; ++m) acc += e[m];
    s[0] = acc;
  }
}

// -|c|^2 / 2 of N codewords whose operand pieces this lane holds (codeword
// n: 4 dims per k-step s in b[n][s]; the four lanes l16, l16+16, l16+32,
// l16+48 hold the rest of it).  Every lane's partial sums (an fdot2 chain
// over its dims) come first, then each round of cross-lane swaps for all N,
// so the swaps' latencies overlap instead of chaining; each codeword gets
// (p0 + p1) + (p2 + p3) of the four lanes' partial sums.
template <int KS, int N>
__device__ __forceinline__ void neg_half_norm2_n(const f16x4 (*b)[KS], float (&out)[N]) {
  float p[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    p[n] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const f16x2 lo = {b[n][s][0], b[n][s][1]};
      const f16x2 hi = {b[n][s][2], b[n][s][3]};
      p[n] = __builtin_amdgcn_fdot2(lo, lo, p[n], false);
      p[n] = __builtin_amdgcn_fdot2(hi, hi, p[n], false);
    }
  }
#pragma unroll
  for (int n = 0; n < N; ++n) p[n] = pair_sum16(p[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) p[n] = pair_sum32(p[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) out[n] = -0.5f * p[n];
}

// The new token's codes from the per-wave argmax keys: waves m, m + M, ...
// searched segment m's codewords.
template <int M, int NW>
__device__ __forceinline__ TokenCodes<M> combine_new_codes(const unsigned long long* keys) {
  int code[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    unsigned long long best = keys[m];
#pragma unroll
    for (int w = m + M; w < NW; w += M) best = keys[w] > best ? keys[w] : best;
    code[m] = argmax_key_index(best);
  }
  TokenCodes<M> t;
  t.set(code);
  return t;
}

// Running merge state of chunk records: max m (natural-log units), and the
// sums num[0..3] = sum_c w_c o_c, den = sum_c w_c l_c with w_c = exp(m_c - m).
struct MergeState {
  float m, num[4], den;
};
// (x, y) -> one state over both record sets; either may be empty (m = -inf)
__device__ __forceinline__ MergeState merge_states(const MergeState& x, const MergeState& y) {
  MergeState r;
  r.m = max_f(x.m, y.m);
  if (r.m == -INFINITY) return x;
  const float sx = fast_exp2((x.m - r.m) * kLog2e), sy = fast_exp2((y.m - r.m) * kLog2e);
#pragma unroll
  for (int e = 0; e < 4; ++e) r.num[e] = x.num[e] * sx + y.num[e] * sy;
  r.den = x.den * sx + y.den * sy;
  return r;
}

// The last workgroup of (request, KV head) bg: the normalised output of its
// G query rows from the first nrec of the C record slots of each row.  Up to 8 chunks, one thread per
// output element with every record load in flight at once.  Beyond that
// the record loads are the critical path, so they are spread and widened:
// thread (h, cq, d4) takes four output columns 4*d4.. of head h and the
// chunks c = cq (mod 4), eight chunks per batch with all their loads in
// flight, and keeps a running merge state (rescaled when its max grows).
// Its column quad is one 16-byte load per chunk; the 32 lanes of a chunk
// class read a record's 512 contiguous bytes.  The four classes then merge:
// lanes l and l ^ 32 of a wave by one lane swap, the head's two waves
// through LDS (scratch: G * 32 * 6 floats).
// The 16-byte record loads are buffer loads with the sc1 cache policy, the
// policy of the device-scope relaxed atomic loads that read m and l (and of
// all of them for C <= 8): served from the device-coherent level, so they
// see the records the other workgroups completed before their arrival.
template <int G>
__device__ __forceinline__ void merge_rows(const DecodeArgs& a, int64_t row0, int64_t cnt, float* scratch,
                                           int nrec) {
  constexpr int D = 128;
  const int C = a.C;   // the records' row stride; the first nrec of a row are merged
  if (nrec <= 8) {
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
      const int64_t row = row0 + i / D;
      const int d = i % D;
      a.out[row * D + d] = merge_chunks<true>(a.part_m + row * C, a.part_l + row * C,
                                              a.part_o + row * C * D + d, nrec, D);
    }
  } else {
    static_assert(G * D <= kDecodeThreads, "one thread per (head, chunk class, column quad)");
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    constexpr int kSc1 = 16;              // buffer cache policy bit SC1
    constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor: raw dword access
    const int tid = threadIdx.x;
    const int d4 = tid & 31, cq = (tid >> 5) & 3, h = tid >> 7;
    const bool second = (tid >> 6) & 1;   // the head's wave with classes 2, 3
    MergeState st = {-INFINITY, {0.0f, 0.0f, 0.0f, 0.0f}, 0.0f};
    const int64_t row = row0 + h;
    if (h < G) {   // whole waves
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          a.part_o + row * C * D, (short)0, C * D * 4, kRsrcWord3);
      constexpr int kB = 8;
      for (int c0 = cq; c0 < nrec; c0 += 4 * kB) {
        float m[kB], l[kB];
        f32x4v o[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int c = c0 + 4 * j;
          const bool in = c < nrec;
          m[j] = in ? rec_load<true>(a.part_m + row * C + c) : -INFINITY;
          l[j] = in ? rec_load<true>(a.part_l + row * C + c) : 0.0f;
          o[j] = in ? __builtin_amdgcn_raw_buffer_load_b128(rs, (c * D + 4 * d4) * 4, 0, kSc1)
                    : f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float mb = st.m;
#pragma unroll
        for (int j = 0; j < kB; ++j) mb = max_f(mb, m[j]);
        if (mb == -INFINITY) continue;
        const float r = fast_exp2((st.m - mb) * kLog2e);   // 0 while st.m = -inf
#pragma unroll
        for (int e = 0; e < 4; ++e) st.num[e] *= r;
        st.den *= r;
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          if (m[j] == -INFINITY) continue;
          const float w = fast_exp2((m[j] - mb) * kLog2e);
          st.den = fmaf(w, l[j], st.den);
#pragma unroll
          for (int e = 0; e < 4; ++e) st.num[e] = fmaf(w, o[j][e], st.num[e]);
        }
        st.m = mb;
      }
      // classes cq and cq ^ 1 (lanes l and l ^ 32): both lanes end with the
      // merge of the pair, taken in the same order
      MergeState x, y;
      {
        const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, st.m), __builtin_bit_cast(int, st.m), false, false);
        x.m = __builtin_bit_cast(float, int(p[0])); y.m = __builtin_bit_cast(float, int(p[1]));
      }
      {
        const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, st.den), __builtin_bit_cast(int, st.den), false, false);
        x.den = __builtin_bit_cast(float, int(p[0])); y.den = __builtin_bit_cast(float, int(p[1]));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, st.num[e]), __builtin_bit_cast(int, st.num[e]), false, false);
        x.num[e] = __builtin_bit_cast(float, int(p[0])); y.num[e] = __builtin_bit_cast(float, int(p[1]));
      }
      st = merge_states(x, y);
      if (second && d4 == (tid & 63)) {   // lanes 0..31 of the second wave
        float* dst = scratch + (h * 32 + d4) * 6;
        dst[0] = st.m; dst[1] = st.den;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[2 + e] = st.num[e];
      }
    }
    __syncthreads();
    if (h < G && !second && d4 == (tid & 63)) {
      const float* src = scratch + (h * 32 + d4) * 6;
      MergeState o2;
      o2.m = src[0]; o2.den = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) o2.num[e] = src[2 + e];
      st = merge_states(st, o2);
      float4 r;
      r.x = st.den > 0.0f ? st.num[0] / st.den : 0.0f;
      r.y = st.den > 0.0f ? st.num[1] / st.den : 0.0f;
      r.z = st.den > 0.0f ? st.num[2] / st.den : 0.0f;
      r.w = st.den > 0.0f ? st.num[3] / st.den : 0.0f;
      *reinterpret_cast<float4*>(a.out + row * D + 4 * d4) = r;
    }
  }
  if (threadIdx.x == 0)   // ready for the next call
    __hip_atomic_store(a.counters + cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// G query heads per KV head, M segments, NT token slots per thread, CPW
// chunks per workgroup (NT / CPW slots each: slot i of a thread is in chunk
// i / (NT / CPW) of its workgroup, every chunk exactly (NT / CPW) * 1024
// tokens; CPW = 2 only with M = 4, where two histograms fit in LDS).  STEP:
// the decode-step variant -- the workgroup whose chunk holds the new token
// (slot lens[b] - 1) encodes the token's K and V into the cache first, and
// with C > 1 the last workgroup of each (request, KV head) merges the chunk
// records into the output.
// PAGED: the codes are read (and the new token's written) through the block
// table of a paged cache.
template <int G, int M, int NT, bool STEP, bool PAGED, int CPW, CbFmt F = CbFmt::F16>
__device__ __forceinline__ void score_chunk(const DecodeArgs& a) {
  constexpr int NTHR = kDecodeThreads;
  constexpr int D = 128;
  constexpr int K = 256;
  constexpr int DS = D / M;
  constexpr int NW = NTHR / 64;
  constexpr int KSTEP_Q = DS / 16;            // MFMA k-steps of the table build
  constexpr int LUT_JOBS = (M * 16) / NW;     // (m, 16-codeword tile) jobs per wave
  constexpr int GP = G >= 2 ? G / 2 : 1;      // 64-bit histogram words per (m, k)
  constexpr int NTILE = M * DS / 16;         // 16-column output tiles of the contraction
  // waves sharing a tile, each a slice of the bins: with one or two heads a
  // single wave takes all 256 bins of its tile (8 waves contract, each on
  // its own, with no cross-wave sum and no barrier before the output)
  constexpr int KSPLIT = G <= 2 ? 1 : NW / NTILE;
  constexpr int KSL = K / KSPLIT;             // bins per slice
  static_assert(NTILE == 8 && (KSPLIT == 1 || KSPLIT == 2), "one or two contraction waves per output tile");
  static_assert(CPW == 1 || (CPW == 2 && M == 4 && NT % 2 == 0), "two chunks per workgroup need M = 4");
  constexpr int NTC = NT / CPW;               // token slots per thread in one chunk
  // The step kernel's records are its own (the caller only sees the merged
  // output): a workgroup of two chunks merges them and writes one record, at
  // its grid index, which halves the records the last workgroup reads.
  constexpr bool kWgRecord = STEP && CPW == 2;

  // Table and histogram live in separate LDS regions, so the histogram can be
  // cleared while the workgroup still waits for its operands.
  // For G >= 2 the histogram is [k][pair][m] 64-bit words (row r = pair * M
  // + m, each word the bins of two heads): a row's banks do not depend on the
  // codeword, so lanes that update different rows do not conflict.  The LDS
  // takes a 64-bit atomic 16 lanes at a time over 32 banks, so 16 lanes must
  // hit rows that differ mod 16; each lane walks the rows in a lane-rotated
  // order that guarantees it (step 4).  For G = 1 it is [m][k] 32-bit words.
  constexpr int R = M * GP;                                                // rows per codeword
  // the table region is reused for the contraction's partial tiles
  // (NTILE * 64 float4) once the scores are in registers
  constexpr int LUT_WORDS = M * K * G > CPW * NTILE * 64 * 4 ? M * K * G : CPW * NTILE * 64 * 4;
  constexpr int HIST_WORDS = G >= 2 ? K * R * 2 : M * K;   // one chunk's histogram
  __shared__ __align__(16) float lut[LUT_WORDS];
  // 256-byte aligned: the pair bit of a row address (step 4) is a bit of the
  // full LDS address
  __shared__ __align__(256) uint32_t hist[CPW * HIST_WORDS];
  uint32_t* hist32 = hist;                                                 // [m][k] (G = 1)
  char* hist_bytes = reinterpret_cast<char*>(hist);                        // [k][R] u64 (G >= 2)
  __shared__ uint32_t lsum[CPW][2 * G];       // l_c per chunk, head and bin slice, fixed point
  __shared__ __align__(16) int mkey[CPW][G];  // chunk max per head, as float_key
  __shared__ uint32_t lest[CPW][G];           // upper estimate of l_c per chunk and head (fix_shift)
  __shared__ unsigned long long new_key[2][NW];  // step: per-wave argmax keys of the new K, V
  __shared__ uint32_t arrive_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  // Grid (hs * Hkv, C / CPW, B), dispatched x fastest: consecutive workgroups
  // go to different XCDs, so with Hkv a multiple of 8 every chunk and head
  // part of one KV head lands on the same XCD and shares its L2 copy of the
  // codebooks (and, with a head split, of the codes).  Workgroup x takes
  // KV head g = x % Hkv and query heads hp*G .. hp*G + G-1 of its group,
  // hp = x / Hkv.
  const int hp = blockIdx.x / a.Hkv;
  const int g = blockIdx.x - hp * a.Hkv;
  const int c = blockIdx.y * CPW;             // first chunk of this workgroup
  const int b = blockIdx.z;
  const int t_begin = c * a.T;
  const int n_own = min(CPW, a.C - c);        // chunks this workgroup owns
  const int64_t row0 = int64_t(b) * a.Hq + int64_t(g) * G * a.hs + int64_t(hp) * G;   // first query row

  // ---- 0. requests --------------------------------------------------------------
  // What does not depend on lens[b] goes out before its value is waited for:
  // the query rows and the K codebook operands of the table build.
  int len = a.lens[b];
  // paged cache: the page of each of this thread's token slots, requested
  // with lens[b] (entries past the request's pages are loaded, never used)
  int32_t page[PAGED ? NT : 1];
  if constexpr (PAGED) {
    const int32_t* row = a.block_table + int64_t(b) * a.max_pages;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = t_begin + i * NTHR + tid;
      page[i] = t < a.Lmax ? row[t >> a.page_shift] : 0;
    }
  }
  const int64_t cb_g = int64_t(g) * M * K * DS;   // first element of KV head g's codebooks
  // table build: wave w owns segment m_l = w % M and codeword tiles
  // nt = w / M + (NW / M) * i
  const int m_l = wave % M;
  // Row 8 of the table build's A operand (unused by the <= 8 heads) carries
  // segment m_l of the new token's K in the step kernel, and xv that of its
  // V, so the same instructions score the token against the codewords.
  constexpr int kNewRow = 8;
  const int64_t bg = int64_t(b) * a.Hkv + g;
  const int64_t cnt = bg * a.hs + hp;         // arrival counter of this head part
  // Rows 0..G-1 of the A operand are the queries, row 8 (step) the new
  // token's K (xv: its V); the other rows only feed output rows that are
  // never read.  With one or two token slots per thread (a latency-bound
  // workgroup) every lane loads with no branch, the other rows' lanes any
  // valid row (query row 0): under branches the loads and zero fills of the
  // same registers take different lane masks, and the compiler then waits
  // for the first loads before the codebook requests below.  With more
  // slots the branch form measured 0.2 us faster on the benchmark's GQA and
  // long-context steps, so it stays there.
  constexpr bool kQBranchFree = NT <= 2;
  f16x4 qa[KSTEP_Q], xv[KSTEP_Q];
  if constexpr (kQBranchFree) {
    const int64_t qoff = (row0 + (l16 < G ? l16 : 0)) * D + m_l * DS + 4 * q4;
    const int64_t noff = bg * D + m_l * DS + 4 * q4;
    const __half* ksrc = (STEP && l16 == kNewRow) ? a.k_new + noff : a.q + qoff;
#pragma unroll
    for (int s = 0; s < KSTEP_Q; ++s) {
      qa[s] = *reinterpret_cast<const f16x4*>(ksrc + s * 16);
      xv[s] = f16x4{0, 0, 0, 0};
      if constexpr (STEP) xv[s] = *reinterpret_cast<const f16x4*>(a.v_new + noff + s * 16);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KSTEP_Q; ++s) {
      qa[s] = f16x4{0, 0, 0, 0};
      xv[s] = f16x4{0, 0, 0, 0};
      if (l16 < G) {
        qa[s] = *reinterpret_cast<const f16x4*>(a.q + (row0 + l16) * D + m_l * DS + s * 16 + 4 * q4);
      } else if (STEP && l16 == kNewRow) {
        qa[s] = *reinterpret_cast<const f16x4*>(a.k_new + bg * D + m_l * DS + s * 16 + 4 * q4);
        xv[s] = *reinterpret_cast<const f16x4*>(a.v_new + bg * D + m_l * DS + s * 16 + 4 * q4);
      }
    }
  }
  f16x4 ckb[LUT_JOBS][KSTEP_Q];
#pragma unroll
  for (int i = 0; i < LUT_JOBS; ++i) {
    const int nt = wave / M + (NW / M) * i;
    const int64_t row = cb_g + (int64_t(m_l) * K + nt * 16 + l16) * DS + 4 * q4;
#pragma unroll
    for (int s = 0; s < KSTEP_Q; ++s) ckb[i][s] = cb_load4<F>(a.k_cb, row + s * 16);
  }

  len = len < 0 ? 0 : (len > a.Lmax ? a.Lmax : len);
  const int t_end = min(t_begin + n_own * a.T, len);
  if (t_begin >= t_end) {   // empty chunks (uniform over the workgroup)
    // A use of the codebook and query operands on this path too, so the
    // compiler keeps their loads ahead of the wait for lens[b] instead of
    // sinking them into the other branch (which would put one memory latency
    // after the other).
#pragma unroll
    for (int i = 0; i < LUT_JOBS; ++i)
#pragma unroll
      for (int s = 0; s < KSTEP_Q; ++s) asm volatile("" ::"v"(ckb[i][s]));
    if constexpr (kQBranchFree) {
#pragma unroll
      for (int s = 0; s < KSTEP_Q; ++s) {
        asm volatile("" ::"v"(qa[s]));
        if constexpr (STEP) asm volatile("" ::"v"(xv[s]));
      }
    }
    const int n_rec = kWgRecord ? 1 : n_own;
    for (int i = tid; i < n_rec * G * D; i += NTHR) {
      const int cc = (kWgRecord ? int(blockIdx.y) : c) + i / (G * D), h = (i / D) % G, d = i % D;
      if (a.part_o == nullptr) {
        a.out[(row0 + h) * D + d] = 0.0f;
      } else {
        rec_store<STEP>(a.part_o + ((row0 + h) * a.C + cc) * D + d, 0.0f);
        if (d == 0) {
          rec_store<STEP>(a.part_m + (row0 + h) * a.C + cc, -INFINITY);
          rec_store<STEP>(a.part_l + (row0 + h) * a.C + cc, 0.0f);
        }
      }
    }
    if constexpr (STEP) {
      if (a.part_o != nullptr && arrive_last(a.counters + cnt, int(gridDim.y), &arrive_flag))
        merge_rows<G>(a, row0, cnt, lut, kWgRecord ? int(gridDim.y) : a.C);
    }
    return;
  }

  // step kernel: does this chunk hold the new token (slot lens[b] - 1)?
  const int t_new = STEP ? len - 1 : -1;
  const bool has_new = STEP && t_new >= t_begin && t_new < t_end;   // uniform
  // step kernel: the V codebook in the table build's B layout, for the new
  // token's V code.  With one or two token slots per thread and fp16
  // codebooks it is requested here, as soon as lens[b] is known, so its
  // latency overlaps the table build; E4M3 codebooks request it after the
  // table build, and with more slots the registers are needed by the scores
  // and it is requested after them.
  f16x4 cvl[STEP ? LUT_JOBS : 1][KSTEP_Q];
  auto load_cvl = [&]() {
#pragma unroll
    for (int i = 0; i < LUT_JOBS; ++i) {
      const int nt = wave / M + (NW / M) * i;
      const int64_t row = cb_g + (int64_t(m_l) * K + nt * 16 + l16) * DS + 4 * q4;
#pragma unroll
      for (int s = 0; s < KSTEP_Q; ++s) cvl[i][s] = cb_load4<F>(a.v_cb, row + s * 16);
    }
  };
  // With fp16 codebooks the early request is made by every wave as raw
  // buffer loads, with an offset past the buffer where the chunk lacks the
  // new token (no memory access): no branch, so the compiler's count of
  // loads in flight stays exact and the table build waits only for its own.
  constexpr bool kCvlEarly = NT <= 2;
  constexpr bool kCvlRaw = STEP && kCvlEarly && F == CbFmt::F16;
  typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
  u32x2v cvl_raw[kCvlRaw ? LUT_JOBS : 1][KSTEP_Q];
  if constexpr (kCvlRaw) {
    const __amdgpu_buffer_rsrc_t vr =
        raw_buffer(static_cast<const _Float16*>(a.v_cb) + cb_g, uint32_t(M * K * DS * 2));
#pragma unroll
    for (int i = 0; i < LUT_JOBS; ++i) {
      const int nt = wave / M + (NW / M) * i;
#pragma unroll
      for (int s = 0; s < KSTEP_Q; ++s) {
        const uint32_t off = has_new ? uint32_t(((m_l * K + nt * 16 + l16) * DS + 4 * q4 + s * 16) * 2) : kOffNone;
        cvl_raw[i][s] = __builtin_amdgcn_raw_buffer_load_b64(vr, off, 0, 0);
      }
    }
  }

  // this (b, KV head)'s codes: a row of the dense cache, or a head's pool
  const int64_t code_base = PAGED ? int64_t(g) * a.pool_head_bytes : bg * a.Lmax * M;
  uint8_t* const kc = a.k_codes + code_base;
  uint8_t* const vc = a.v_codes + code_base;
  // the slot of token t; pg is the table entry of its page (paged cache)
  auto slot = [&](int t, int32_t pg) -> int64_t {
    if constexpr (PAGED) {
      const uint32_t p = min(uint32_t(pg), a.n_pages - 1u);
      return (int64_t(p) << a.page_shift) | int64_t(t & ((1 << a.page_shift) - 1));
    } else {
      return t;
    }
  };
  int32_t page_new = 0;   // step kernel, paged: the new token's page (thread 0)
  if constexpr (STEP && PAGED) {
    if (has_new && tid == 0) page_new = a.block_table[int64_t(b) * a.max_pages + (t_new >> a.page_shift)];
  }
  // The chunk's K or V codes: raw buffer loads from every lane (no branch);
  // slots past lens[b] -- and, in the step kernel, the new token's slot,
  // whose codes it computes and one workgroup writes -- get an offset past
  // the buffer, so they read nothing.  Dense: the buffer is the chunk's
  // valid tokens; paged: the KV head's pool (under 2 GiB, checked on the
  // host).
  auto load_codes = [&](TokenCodes<M> (&dst)[NT], const uint8_t* codes) {
    const uint8_t* base = PAGED ? codes : codes + int64_t(t_begin) * M;
    const uint32_t nbytes = PAGED ? uint32_t(a.pool_head_bytes) : uint32_t(t_end - t_begin) * M;
    const __amdgpu_buffer_rsrc_t r = raw_buffer(base, nbytes);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = t_begin + i * NTHR + tid;
      const bool use = t < t_end && t != t_new;
      uint32_t off;
      if constexpr (PAGED) off = use ? uint32_t(slot(t, page[i])) * M : kOffNone;
      else off = use ? uint32_t(t - t_begin) * M : kOffNone;
      dst[i].load(r, off);
    }
  };
  // The V codes are requested after the table build (the histogram needs
  // them, after the scores), so less traffic is queued ahead of the table's
  // operands.  With four or more token slots per thread the K codes wait
  // too, until the codebook operands are in: the workgroup's table reads
  // then start on codes that arrive behind a codebook that came alone
  // (measured faster on the GQA step, the same on the long-context one);
  // with one or two slots (latency-bound) they go out with the codebook.
  constexpr bool kKcLate = NT >= 4;
  TokenCodes<M> kcode[NT], vcode[NT];
  if constexpr (!kKcLate) load_codes(kcode, kc);

  // the histograms are cleared while the operands are in flight
  for (int i = tid; i < CPW * HIST_WORDS / 4; i += NTHR)
    reinterpret_cast<uint4*>(hist)[i] = make_uint4(0, 0, 0, 0);
  if (tid < CPW * G) {
    mkey[tid / G][tid % G] = float_key(-INFINITY);
    lest[tid / G][tid % G] = 0;
  }

  // ---- 1. lookup table on the matrix cores ----------------------------------
  // Step kernel, chunk with the new token: row 8 of every product starts at
  // -|c|^2/2 of its codeword c, so it ends at x.c - |c|^2/2, whose argmax is
  // the nearest codeword (the arithmetic of pq_encode, decision for decision).
  // The K code is needed by the scores, so it is found here; the V code only
  // by the histogram, so it is found while the scores are gathered.
  float best_k = -INFINITY;
  int idx_k = 0;
  float cnorm[STEP ? LUT_JOBS : 1];   // -|c|^2/2 of this lane's codeword per job, all first
  if constexpr (STEP) {
    if (has_new) {
      neg_half_norm2_n<KSTEP_Q, LUT_JOBS>(ckb, cnorm);
    }
  }
#pragma unroll
  for (int i = 0; i < LUT_JOBS; ++i) {
    const int nt = wave / M + (NW / M) * i;
    const int k = nt * 16 + l16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (STEP) {
      if (has_new && q4 == kNewRow / 4) acc[0] = cnorm[i];
    }
#pragma unroll
    for (int s = 0; s < KSTEP_Q; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[s], ckb[i][s], acc, 0, 0, 0);
    if constexpr (STEP) {
      if (has_new && acc[0] > best_k) { best_k = acc[0]; idx_k = k; }   // ascending k: ties keep the lower
    }
    // lane holds LUT[h = 4*q4 + r][k = nt*16 + l16], r < 4
    if constexpr (G >= 4) {
      if (4 * q4 < G)
        *reinterpret_cast<float4*>(lut + lut_index<G, K>(m_l, k, q4)) =
            make_float4(acc[0] * a.qscale, acc[1] * a.qscale, acc[2] * a.qscale, acc[3] * a.qscale);
    } else if constexpr (G == 2) {
      float* dst = lut + lut_index<G, K>(m_l, k, 0);
      if (q4 == 0) *reinterpret_cast<float2*>(dst) = make_float2(acc[0] * a.qscale, acc[1] * a.qscale);
    } else {
      if (q4 == 0) lut[lut_index<G, K>(m_l, k, 0)] = acc[0] * a.qscale;
    }
  }
  if constexpr (STEP) {
    if (has_new) {   // argmax over the row's 16 lanes; the segment's waves are combined below
      argmax_step<kDppXor1>(best_k, idx_k); argmax_step<kDppXor2>(best_k, idx_k);
      argmax_step<kDppRor4>(best_k, idx_k); argmax_step<kDppRor8>(best_k, idx_k);
      if (lane == 16 * (kNewRow / 4)) new_key[0][wave] = argmax_key(best_k, idx_k);
    }
  }
  if constexpr (kKcLate) load_codes(kcode, kc);
  __syncthreads();

  // step kernel: the new token's K codes, into the cache (one head part
  // writes) and, where its slot's codes are used below, in place of them
  // (selected there, so nothing here waits for the codes in flight)
  TokenCodes<M> nk;
  if constexpr (STEP) {
    if (has_new) {
      nk = combine_new_codes<M, NW>(new_key[0]);
      if (tid == 0 && hp == 0) nk.store(kc + slot(t_new, page_new) * M);
    }
  }

  // V codebook operands of the contraction.  Wave w owns segment m_v and 16
  // output columns jt*16..+15.  With 32-codeword steps lane (l16, q4) needs
  // rows 8*q4 .. 8*q4+7 of column l16 of each block: eight 16-bit loads
  // straight into the halves of the operand registers (the 16 lanes of a row
  // group read 32 contiguous bytes), so no VALU work puts them in MFMA order.
  // A wave waits for these loads where it issues them (two halves are packed
  // per register as they arrive), so they are requested inside the histogram,
  // before its last quarter of token slots: the issuing waves wait there
  // while the others keep the LDS busy with their updates, instead of every
  // wave waiting at a barrier.  With one slot per thread they go out just
  // before the histogram.
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const int tile = wave % NTILE;
  const int ksl = wave / NTILE;               // bins [ksl * KSL, (ksl + 1) * KSL)
  const bool cwave = wave < NTILE * KSPLIT;   // this wave takes part in the contraction
  const int m_v = tile % M;
  const int jt = tile / M;
  f16x8 cvb[KSL / 32];
  // With two or four heads the histogram's bins of one segment lie 64 or
  // 128 bytes apart, so the four bins a lane reads per step share a bank
  // group with every other lane's: lane group q4 reads them in an order
  // rotated by q4 instead (four bank groups), and the operands' k order
  // within each lane follows -- position j holds bin perm(j) in both the
  // histogram and the codebook operand, which leaves the sum over k as it is.
  constexpr bool kRot = G == 2 || G == 4;
  auto perm = [&](int j) { return kRot ? ((((j & 3) + q4) & 3) | (j & 4)) : j; };
  auto load_cvb = [&]() {
    if (!cwave) return;
#pragma unroll
    for (int st = 0; st < KSL / 32; ++st) {
      const int64_t src = cb_g + (int64_t(m_v) * K + ksl * KSL + st * 32 + 8 * q4) * DS + jt * 16 + l16;
#pragma unroll
      for (int j = 0; j < 8; ++j) cvb[st][j] = cb_load1<F>(a.v_cb, src + perm(j) * DS);
    }
  };
  load_codes(vcode, vc);
  if constexpr (STEP && kCvlEarly && !kCvlRaw) {
    if (has_new) load_cvl();
  }

  // ---- 2. scores --------------------------------------------------------------
  float s[NT][G];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = t_begin + i * NTHR + tid;
    if (t < t_end) {
      TokenCodes<M> code = kcode[i];
      if constexpr (STEP) {
        if (t == t_new) code = nk;
      }
      token_scores<G, M, K>(lut, code, s[i]);
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) s[i][h] = -INFINITY;
    }
  }

  if constexpr (STEP) {
    if (has_new) {   // the new token's V: same products as its K above, per-wave argmax
      if constexpr (!kCvlEarly) load_cvl();
      if constexpr (kCvlRaw) {
#pragma unroll
        for (int i = 0; i < LUT_JOBS; ++i)
#pragma unroll
          for (int s = 0; s < KSTEP_Q; ++s) cvl[i][s] = __builtin_bit_cast(f16x4, cvl_raw[i][s]);
      }
      float best_v = -INFINITY;
      int idx_v = 0;
      // four jobs at a time: norms (cross-lane sums), products, then compares
      constexpr int VB = NT >= 4 ? 2 : (LUT_JOBS < 4 ? LUT_JOBS : 4);
#pragma unroll
      for (int i0 = 0; i0 < LUT_JOBS; i0 += VB) {
        float vn[VB];
        neg_half_norm2_n<KSTEP_Q, VB>(cvl + i0, vn);
        f32x4 accv[VB];
#pragma unroll
        for (int j = 0; j < VB; ++j) {
          accv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (q4 == kNewRow / 4) accv[j][0] = vn[j];
#pragma unroll
          for (int s = 0; s < KSTEP_Q; ++s)
            accv[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(xv[s], cvl[i0 + j][s], accv[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < VB; ++j) {   // ascending codewords: ties keep the lower
          const int nt = wave / M + (NW / M) * (i0 + j);
          if (accv[j][0] > best_v) { best_v = accv[j][0]; idx_v = nt * 16 + l16; }
        }
      }
      argmax_step<kDppXor1>(best_v, idx_v); argmax_step<kDppXor2>(best_v, idx_v);
      argmax_step<kDppRor4>(best_v, idx_v); argmax_step<kDppRor8>(best_v, idx_v);
      if (lane == 16 * (kNewRow / 4)) new_key[1][wave] = argmax_key(best_v, idx_v);
    }
  }

  // ---- 3. chunk max and probabilities ----------------------------------------
  float m_c[CPW][G];
#pragma unroll
  for (int p = 0; p < CPW; ++p) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[p * NTC][h];
#pragma unroll
      for (int i = 1; i < NTC; ++i) mx = max_f(mx, s[p * NTC + i][h]);
      m_c[p][h] = mx;
    }
    row_max_n<G>(m_c[p]);
    if (l16 < G) {   // lane h of each row of 16: one integer LDS max for head h
      float mine = m_c[p][0];
#pragma unroll
      for (int h = 1; h < G; ++h) mine = (l16 == h) ? m_c[p][h] : mine;
      atomicMax(&mkey[p][l16], float_key(mine));
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < CPW; ++p)
#pragma unroll
    for (int h = 0; h < G; ++h) m_c[p][h] = key_float(mkey[p][h]);
  // p_t = 2^(s_t - m_c) in place of the scores, and the chunk's mass: row
  // sums, then one rounded-up integer LDS add per (row, head)
  {
    float psum[CPW][G];
#pragma unroll
    for (int p = 0; p < CPW; ++p)
#pragma unroll
      for (int h = 0; h < G; ++h) psum[p][h] = 0.0f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const bool valid = t_begin + i * NTHR + tid < t_end;
      const int pc = i / NTC;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float e = valid ? fast_exp2(s[i][h] - m_c[pc][h]) : 0.0f;
        s[i][h] = e;
        psum[pc][h] += e;
      }
    }
#pragma unroll
    for (int p = 0; p < CPW; ++p) {
      row_sum_n<G>(psum[p]);
      if (l16 < G) {
        float mine = psum[p][0];
#pragma unroll
        for (int h = 1; h < G; ++h) mine = (l16 == h) ? psum[p][h] : mine;
        atomicAdd(&lest[p][l16], mass_fix(mine));
      }
    }
  }
  if constexpr (STEP) {
    if (has_new) {   // the new token's V codes (per-wave keys written before the barrier above)
      const TokenCodes<M> nv = combine_new_codes<M, NW>(new_key[1]);
      if (tid == 0 && hp == 0) nv.store(vc + slot(t_new, page_new) * M);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (t_begin + i * NTHR + tid == t_new) vcode[i] = nv;
      }
    }
  }
  constexpr int kCvbSlot = NT >= 2 ? (NT * 3) / 4 : 0;   // histogram slot before which they are requested
  if constexpr (kCvbSlot == 0) load_cvb();

  // ---- 4. V histogram (fixed point, integer LDS atomics) -----------------------
  // Lane rotation (G >= 2): at step (jm, jp) a lane updates segment
  // (jm + om) % M, om = lane % M, and head pair jp, or pair jp XOR 1 on the
  // lanes whose bit log2(M) is set.  With rows pair * M + m, the 16 lanes of
  // a group then hit 2M rows that differ mod 16 (all 16 lanes for M = 8).
  // Codes are rotated once per token (one 64-bit funnel shift), pairs by one
  // swap of neighbours; the address is a per-lane base per segment plus an
  // immediate per pair.
  const int om = lane & (M - 1);
  const bool swap_pairs = GP >= 2 && ((lane / M) & 1) != 0;
  // LDS byte address of rotated segment jm in the row of pair 0 (or pair 1
  // when swapping) of codeword 0; pair 2q + b lives at (this ^ b*8M) +
  // q*16M.  The empty asm hides the histogram's (constant) LDS address from
  // the optimiser, which would otherwise merge it with the pair offsets into
  // constants too large for the instruction's 16-bit offset field and spend
  // two more VALU instructions per segment on them.
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t hist_lds = uint32_t(reinterpret_cast<uintptr_t>((lds_char*)hist_bytes));
  uint32_t row_m[M];
#pragma unroll
  for (int jm = 0; jm < M; ++jm) {
    row_m[jm] = hist_lds + uint32_t(((jm + om) & (M - 1)) * 8) + (swap_pairs ? M * 8 : 0);
    asm("" : "+v"(row_m[jm]));
  }

  __syncthreads();   // mass estimates complete
  // the bin value before rounding is p * 2^S (exact: a power-of-two scale)
  float fscale[CPW][G];
#pragma unroll
  for (int p = 0; p < CPW; ++p)
#pragma unroll
    for (int h = 0; h < G; ++h) fscale[p][h] = pow2i(fix_shift(lest[p][h]));
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if (kCvbSlot != 0 && i == kCvbSlot) load_cvb();
    const int t = t_begin + i * NTHR + tid;
    constexpr int kHistBytes = HIST_WORDS * 4;
    const int pc = i / NTC;                   // chunk of this slot (compile time)
    if (t < t_end) {
      uint32_t u[G];
#pragma unroll
      for (int h = 0; h < G; ++h)
        u[h] = uint32_t(fmaf(s[i][h], fscale[pc][h], 0.5f));   // round(p 2^S)
      if constexpr (G >= 2) {
        uint64_t pv[GP];
#pragma unroll
        for (int pp = 0; pp < GP; ++pp)
          pv[pp] = __builtin_bit_cast(uint64_t, make_uint2(u[2 * pp], u[2 * pp + 1]));
        if constexpr (GP >= 2) {   // pv[j] <- pv[j ^ 1] on swapping lanes
#pragma unroll
          for (int j = 0; j < GP; j += 2) {
            const uint64_t x = pv[j], y = pv[j + 1];
            pv[j] = swap_pairs ? y : x;
            pv[j + 1] = swap_pairs ? x : y;
          }
        }
        const TokenCodes<M> rc = vcode[i].rotated(om);
#pragma unroll
        for (int jm = 0; jm < M; ++jm) {
          typedef __attribute__((address_space(3))) unsigned long long lds_u64;
          const uint32_t b0 = uint32_t(rc.get(jm)) * (R * 8) + row_m[jm] + uint32_t(pc * kHistBytes);
          lds_u64* p0 = reinterpret_cast<lds_u64*>(uintptr_t(b0));
          if constexpr (GP == 1) {
            __hip_atomic_fetch_add(p0, (unsigned long long)pv[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          } else {
            lds_u64* p1 = reinterpret_cast<lds_u64*>(uintptr_t(b0 ^ uint32_t(M * 8)));
#pragma unroll
            for (int q = 0; q < GP / 2; ++q) {
              __hip_atomic_fetch_add(p0 + q * 2 * M, (unsigned long long)pv[2 * q],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              __hip_atomic_fetch_add(p1 + q * 2 * M, (unsigned long long)pv[2 * q + 1],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < M; ++m) atomicAdd(hist32 + pc * HIST_WORDS + m * K + vcode[i].get(m), u[0]);
      }
    }
  }

  __syncthreads();   // histogram complete

  // ---- 5. contraction with the V codebook on the matrix cores ----------------
  // A[i][k]: rows i < 8 carry the fp16 high part of Hist[m_v][k][i], rows
  // i >= 8 the low part of Hist[m_v][k][i - 8] (zero for heads >= G), so one
  // 16x16x32 instruction covers both parts; o[h] = C[h] + C[h + 8].
  // Lane (i, q4) needs bins 8*q4 .. 8*q4+7 of a 32-bin step (position j
  // holding bin perm(j), in the order its codebook operand was loaded in).  The lanes i and
  // i + 8 (same head, hi and lo) each convert half of them -- bins +0..3 on
  // the hi lane, +4..7 on the lo lane -- into both parts, and swap the part
  // the other one needs with one DPP move per word.
  const int hh = l16 & 7;
  const bool lo_row = l16 >= 8;
  const int kh = lo_row ? 4 : 0;
  float4* part_tile = reinterpret_cast<float4*>(lut);   // [CPW][NTILE][64]; the table is dead
  f32x4 o_own[CPW];
  uint32_t lwave[CPW];   // KSPLIT == 1: l_c of head l16 & 7, from this wave's bins
#pragma unroll
  for (int p = 0; p < CPW; ++p) {
    lwave[p] = 0;
    o_own[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!cwave) continue;
    const char* hb = hist_bytes + p * HIST_WORDS * 4;
    const uint32_t* h32 = hist32 + p * HIST_WORDS;
    const float unfix = pow2i(-fix_shift(lest[p][hh < G ? hh : 0]));   // 2^-S of this row's head
    uint32_t raw[KSL / 32][4];
#pragma unroll
    for (int st = 0; st < KSL / 32; ++st) {
      const int k0 = ksl * KSL + st * 32 + 8 * q4 + kh;
#pragma unroll
      for (int v = 0; v < 4; ++v) raw[st][v] = 0;
      if (hh < G) {
        if constexpr (G >= 2) {
          const char* src = hb + (k0 * R + (hh >> 1) * M + m_v) * 8 + (hh & 1) * 4;
#pragma unroll
          for (int v = 0; v < 4; ++v) raw[st][v] = *reinterpret_cast<const uint32_t*>(src + perm(v) * R * 8);
        } else {
          const uint4 w = *reinterpret_cast<const uint4*>(h32 + m_v * K + k0);
          raw[st][0] = w.x; raw[st][1] = w.y; raw[st][2] = w.z; raw[st][3] = w.w;
        }
      }
    }
    // l_c: the waves of segment 0, first column tile (one per bin slice), add
    // their bins in integers; lanes (h, q4) and (h + 8, q4) hold complementary
    // bins of head h, so a row_ror:8 and two lane swaps complete the slice.
    if (KSPLIT == 1 || tile == 0) {
      uint32_t lpart = 0;
#pragma unroll
      for (int st = 0; st < KSL / 32; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) lpart += raw[st][v];
      lpart += uint32_t(__builtin_amdgcn_mov_dpp(int(lpart), kDppRor8, 0xf, 0xf, true));
      {
        const auto r = __builtin_amdgcn_permlane16_swap(lpart, lpart, false, false);
        lpart = uint32_t(r[0]) + uint32_t(r[1]);
      }
      {
        const auto r = __builtin_amdgcn_permlane32_swap(lpart, lpart, false, false);
        lpart = uint32_t(r[0]) + uint32_t(r[1]);
      }
      if constexpr (KSPLIT == 2) {
        if (lane < G) lsum[p][ksl * G + lane] = lpart;
      } else {
        lwave[p] = lpart;
      }
    }
    f32x4 oa = {0.f, 0.f, 0.f, 0.f}, ob = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KSL / 32; ++st) {
      uint32_t hw[2], lw[2];   // packed fp16 pairs: high parts, low parts
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const float f0 = float(raw[st][2 * v]) * unfix;
        const float f1 = float(raw[st][2 * v + 1]) * unfix;
        const _Float16 h0 = (_Float16)f0, h1 = (_Float16)f1;
        const _Float16 e0 = (_Float16)(f0 - (float)h0), e1 = (_Float16)(f1 - (float)h1);
        hw[v] = uint32_t(__builtin_bit_cast(uint16_t, h0)) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
        lw[v] = uint32_t(__builtin_bit_cast(uint16_t, e0)) | (uint32_t(__builtin_bit_cast(uint16_t, e1)) << 16);
      }
      // the hi lane sends its low parts, the lo lane its high parts; row_ror:8
      // delivers lane i+8's word to lane i and lane i's to lane i+8
      const uint32_t r0 = uint32_t(__builtin_amdgcn_mov_dpp(int(lo_row ? hw[0] : lw[0]), kDppRor8, 0xf, 0xf, true));
      const uint32_t r1 = uint32_t(__builtin_amdgcn_mov_dpp(int(lo_row ? hw[1] : lw[1]), kDppRor8, 0xf, 0xf, true));
      uint4 aw;
      aw.x = lo_row ? r0 : hw[0];
      aw.y = lo_row ? r1 : hw[1];
      aw.z = lo_row ? lw[0] : r0;
      aw.w = lo_row ? lw[1] : r1;
      const f16x8 av = __builtin_bit_cast(f16x8, aw);
      if (st & 1) ob = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, cvb[st], ob, 0, 0, 0);
      else        oa = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, cvb[st], oa, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o_own[p][r] = pair_sum32(oa[r] + ob[r]);   // rows 4*q4 + r and 4*q4 + r + 8 (lane + 32)
    }
    // lane holds the slice's o[h = 4*q4 + r][d = m_v*DS + jt*16 + l16]; the
    // second slice's waves leave theirs in the (dead) table region and the
    // first slice's waves add it and write.
    if (ksl == 1)
      part_tile[(p * NTILE + tile) * 64 + lane] = make_float4(o_own[p][0], o_own[p][1], o_own[p][2], o_own[p][3]);
  }

  // ---- 6. write (m, l, o) of each chunk, or the normalised output --------------
  if constexpr (KSPLIT == 2) __syncthreads();
  // the integer l_c of the heads 4*q4 + r this lane writes (whole waves)
  auto lsums = [&](int p, uint32_t (&l)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = min(4 * q4 + r, G - 1);
      if constexpr (KSPLIT == 2) l[r] = lsum[p][h] + lsum[p][G + h];
      else l[r] = uint32_t(__shfl(int(lwave[p]), h, 64));
    }
  };
  if (kWgRecord && cwave && ksl == 0) {
    // both chunks' (m, l, o) merged into the workgroup's record (the max in
    // log2 units inside the kernel, natural log in the records)
    const int d = m_v * DS + jt * 16 + l16;
    f32x4 o[2];
    uint32_t lr[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      o[p] = o_own[p];
      if constexpr (KSPLIT == 2) {
        const float4 other = part_tile[(p * NTILE + tile) * 64 + lane];
        o[p][0] += other.x; o[p][1] += other.y; o[p][2] += other.z; o[p][3] += other.w;
      }
      lsums(p, lr[p]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * q4 + r;
      if (h < G) {
        float mp[2], lp[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const bool own = p < n_own;
          mp[p] = own ? key_float(mkey[p][h]) : -INFINITY;
          lp[p] = own ? float(lr[p][r]) * pow2i(-fix_shift(lest[p][h])) : 0.0f;
        }
        const float mh = max_f(mp[0], mp[1]);
        float om = 0.0f, lm = 0.0f;
        if (mh != -INFINITY) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float w = mp[p] == -INFINITY ? 0.0f : fast_exp2(mp[p] - mh);
            om = fmaf(w, o[p][r], om);
            lm = fmaf(w, lp[p], lm);
          }
        }
        const int64_t slot = (row0 + h) * a.C + blockIdx.y;
        rec_store<STEP>(a.part_o + slot * D + d, om);
        if (d == 0) {
          rec_store<STEP>(a.part_m + slot, mh * kLn2);
          rec_store<STEP>(a.part_l + slot, lm);
        }
      }
    }
  }
  if (!kWgRecord && cwave && ksl == 0) {
    const int d = m_v * DS + jt * 16 + l16;
#pragma unroll
    for (int p = 0; p < CPW; ++p) {
      if (p >= n_own) break;   // the grid's last workgroup may own fewer chunks
      const int cc = c + p;
      f32x4 o = o_own[p];
      if constexpr (KSPLIT == 2) {
        const float4 other = part_tile[(p * NTILE + tile) * 64 + lane];
        o[0] += other.x; o[1] += other.y; o[2] += other.z; o[3] += other.w;
      }
      uint32_t lr[4];
      lsums(p, lr);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * q4 + r;
        if (h < G) {
          const float mh = key_float(mkey[p][h]);
          const float lh = float(lr[r]) * pow2i(-fix_shift(lest[p][h]));
          if (a.part_o == nullptr) {   // one chunk in all (C == 1)
            a.out[(row0 + h) * D + d] = lh > 0.0f ? o[r] * __builtin_amdgcn_rcpf(lh) : 0.0f;
          } else {
            rec_store<STEP>(a.part_o + ((row0 + h) * a.C + cc) * D + d, o[r]);
            if (d == 0) {
              rec_store<STEP>(a.part_m + (row0 + h) * a.C + cc, mh * kLn2);
              rec_store<STEP>(a.part_l + (row0 + h) * a.C + cc, lh);
            }
          }
        }
      }
    }
  }
  if constexpr (STEP) {
    if (a.part_o != nullptr && arrive_last(a.counters + cnt, int(gridDim.y), &arrive_flag))
      merge_rows<G>(a, row0, cnt, lut, kWgRecord ? int(gridDim.y) : a.C);
  }
}

// G query heads per KV head, M segments, NT token slots per thread, STEP as
// above; the codes in a dense [B][Hkv][Lmax][M] cache.
// F: the codebooks' element format.
template <int G, int M, int NT, bool STEP, int CPW = 1, CbFmt F = CbFmt::F16>
__global__ __launch_bounds__(kDecodeThreads) void decode_partials_kernel(DecodeArgs a) {
  score_chunk<G, M, NT, STEP, false, CPW, F>(a);
}

// The same over a paged cache (block table and per-head page pools).
template <int G, int M, int NT, bool STEP, int CPW = 1>
__global__ __launch_bounds__(kDecodeThreads) void decode_paged_kernel(DecodeArgs a) {
  score_chunk<G, M, NT, STEP, true, CPW>(a);
}

// Merge of chunk statistics: one workgroup of D threads per row.
struct ReduceArgs {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  float* out;
  int32_t C;
};

template <int D, bool POLY = false>
__global__ __launch_bounds__(D) void reduce_kernel(ReduceArgs a) {
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  a.out[row * D + d] = merge_chunks<false, POLY>(a.part_m + row * a.C, a.part_l + row * a.C,
                                                 a.part_o + row * a.C * D + d, a.C, D);
}

}  // namespace pqattn
