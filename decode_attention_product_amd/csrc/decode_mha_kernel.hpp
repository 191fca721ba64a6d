// Request-batched score kernel for one query head per KV head (gfx950).
//
// With one query head per KV head, a workgroup of decode_partials_kernel
// per (request, KV head, chunk) loads a whole K and V codebook pair (128 KB)
// and runs its table build and its contraction with a single useful matrix
// row, for at most a few thousand tokens: with many requests those fixed
// costs, and the codebook reads from L2, dominate.  Here one workgroup takes
// R requests of the same KV head and the same chunk.  They share the
// codebook loads; the table build takes their R queries as matrix rows and
// the contraction their R histograms; every request keeps its own token
// stream, chunk max, sum and histogram (AQPIM page, section 4.1; PAM page,
// section 2.2.3 (1)).  Per request the arithmetic is the per-request
// kernel's: table gathers in fp32, base-2 exponentials, a fixed-point
// histogram, an fp16 hi + lo contraction on the matrix cores.
//
// The R requests are taken in passes of RP = 4: in pass p thread t serves
// request p*RP + t / TPR (TPR = 1024 / RP threads, whole waves) and its
// tokens chunk_start + t % TPR + j*TPR, j < NT.  The table build and the
// contraction take all R requests at once (R <= 8 rows of the matrix-core
// tiles), so R = 8 halves the workgroups, and with them the codebook loads,
// table builds and contractions per request, against R = 4; the next pass's
// codes are requested as soon as the current pass's K codes are consumed.
// LDS: the table
// [m][r][k] (fp32), the histogram [r][m][k] (32-bit fixed point scaled by
// each request's mass, as in the per-request kernel); a request's l_c is the
// integer sum of its segment-0 bins.
#pragma once

#include "decode_kernel.hpp"
#include "plan.h"   // kMhaPassRequests

namespace pqattn {

template <int M, int R, int NT, bool PAGED>
__global__ __launch_bounds__(kDecodeThreads) void decode_mha_kernel(DecodeArgs a) {
  constexpr int RP = kMhaPassRequests;          // requests per pass
  constexpr int NP = R / RP;                    // passes
  constexpr int NTHR = kDecodeThreads;
  constexpr int D = 128;
  constexpr int K = 256;
  constexpr int DS = D / M;
  constexpr int NW = NTHR / 64;
  constexpr int TPR = NTHR / RP;                // threads per request in a pass
  constexpr int KSTEP_Q = DS / 16;              // MFMA k-steps of the table build
  constexpr int LUT_JOBS = (M * 16) / NW;       // (m, 16-codeword tile) jobs per wave
  constexpr int NTILE = M * DS / 16;            // 16-column output tiles of the contraction
  constexpr int KSPLIT = NW / NTILE;            // waves sharing a tile, each a slice of the bins
  constexpr int KSL = K / KSPLIT;
  static_assert(R == 4 || R == 8, "requests per workgroup");
  static_assert(R % RP == 0, "whole passes");
  static_assert(NTILE == 8 && KSPLIT == 2, "two contraction waves per output tile");

  __shared__ __align__(16) float lut[M * R * K];         // [m][r][k]
  __shared__ __align__(16) uint32_t hist[R * M * K];     // [r][m][k]
  __shared__ uint32_t lsum[2 * R];                       // l_c per request and bin slice
  __shared__ int mkey[R];
  __shared__ uint32_t lest[R];                           // upper estimate of l_c (fix_shift)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int g = blockIdx.x;
  const int c = blockIdx.y;
  const int b0 = blockIdx.z * R;                // first request of the group
  const int rl = tid / TPR;                     // this thread's request within a pass, uniform per wave
  const int li = tid % TPR;
  const int t_begin = c * a.T;

  // ---- 0. requests ------------------------------------------------------------
  // per pass: the request, whether it exists, its tokens' end in the chunk
  int t_end[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int b = b0 + p * RP + rl;
    int len = b < a.B ? a.lens[b] : 0;
    len = len < 0 ? 0 : (len > a.Lmax ? a.Lmax : len);
    t_end[p] = min(t_begin + a.T, len);         // t_end <= t_begin: no token of b here
  }
  // the code bytes of token slot j of pass p (the slot must hold a token)
  auto code_offset = [&](int p, int t, int32_t pg) -> int64_t {
    if constexpr (PAGED) {
      const uint32_t pp = min(uint32_t(pg), a.n_pages - 1u);
      return int64_t(g) * a.pool_head_bytes +
             ((int64_t(pp) << a.page_shift) | int64_t(t & ((1 << a.page_shift) - 1))) * M;
    } else {
      return ((int64_t(b0 + p * RP + rl) * a.Hkv + g) * a.Lmax + t) * M;
    }
  };
  // paged cache: the pages of this thread's slots in a pass
  auto load_pages = [&](int p, int32_t (&pg)[PAGED ? NT : 1]) {
    if constexpr (PAGED) {
      const int b = b0 + p * RP + rl;
      const int32_t* row = a.block_table + int64_t(b < a.B ? b : 0) * a.max_pages;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int t = t_begin + li + j * TPR;
        pg[j] = (b < a.B && t < a.Lmax) ? row[t >> a.page_shift] : 0;
      }
    }
  };
  int32_t page[PAGED ? NT : 1];
  load_pages(0, page);
  // table build operands: lane l16 < R carries the query of request b0 + l16
  const int m_l = wave % M;
  f16x4 qa[KSTEP_Q];
#pragma unroll
  for (int s = 0; s < KSTEP_Q; ++s) {
    qa[s] = f16x4{0, 0, 0, 0};
    if (l16 < R && b0 + l16 < a.B)
      qa[s] = *reinterpret_cast<const f16x4*>(a.q + (int64_t(b0 + l16) * a.Hq + g) * D + m_l * DS +
                                              s * 16 + 4 * q4);
  }
  const __half* ckg = static_cast<const __half*>(a.k_cb) + int64_t(g) * M * K * DS;
  f16x4 ckb[LUT_JOBS][KSTEP_Q];
#pragma unroll
  for (int i = 0; i < LUT_JOBS; ++i) {
    const int nt = wave / M + (NW / M) * i;
    const __half* row = ckg + (int64_t(m_l) * K + nt * 16 + l16) * DS + 4 * q4;
#pragma unroll
    for (int s = 0; s < KSTEP_Q; ++s) ckb[i][s] = *reinterpret_cast<const f16x4*>(row + s * 16);
  }

  TokenCodes<M> kcode[NT], vcode[NP][NT];
  auto load_codes = [&](int p) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int t = t_begin + li + j * TPR;
      if (t < t_end[p]) {
        const int64_t off = code_offset(p, t, PAGED ? page[j] : 0);
        kcode[j].load(a.k_codes + off);
        vcode[p][j].load(a.v_codes + off);
      }
    }
  };
  load_codes(0);
  for (int i = tid; i < R * M * K / 4; i += NTHR)
    reinterpret_cast<uint4*>(hist)[i] = make_uint4(0, 0, 0, 0);
  if (tid < R) {
    mkey[tid] = float_key(-INFINITY);
    lest[tid] = 0;
  }

  // ---- 1. lookup tables of the R queries on the matrix cores --------------------
#pragma unroll
  for (int i = 0; i < LUT_JOBS; ++i) {
    const int nt = wave / M + (NW / M) * i;
    const int k = nt * 16 + l16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEP_Q; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[s], ckb[i][s], acc, 0, 0, 0);
    // lane holds LUT[request 4*q4 + e][k], e < 4
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 4 * q4 + e;
      if (rr < R) lut[(m_l * R + rr) * K + k] = acc[e] * a.qscale;
    }
  }
  __syncthreads();

  // V codebook operands of the contraction, in MFMA order by 16-bit loads
  // (as in the per-request kernel)
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const _Float16* cvg = reinterpret_cast<const _Float16*>(a.v_cb) + int64_t(g) * M * K * DS;
  const int tile = wave % NTILE;
  const int ksl = wave / NTILE;
  const int m_v = tile % M;
  const int jt = tile / M;
  f16x8 cvb[KSL / 32];

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = p * RP + rl;                  // this thread's request in the pass
    // ---- 2. scores ----------------------------------------------------------------
    float s[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int t = t_begin + li + j * TPR;
      s[j] = -INFINITY;
      if (t < t_end[p]) {
        float v[M];
#pragma unroll
        for (int m = 0; m < M; ++m) v[m] = lut[(m * R + r) * K + kcode[j].get(m)];
        float acc = v[0];
#pragma unroll
        for (int m = 1; m < M; ++m) acc += v[m];
        s[j] = acc;
      }
    }
    if (p + 1 < NP) {   // the next pass's pages and codes, while this pass finishes
      load_pages(p + 1, page);
      load_codes(p + 1);
    }

    // ---- 3. chunk max per request ---------------------------------------------------
    {
      float mx[1] = {s[0]};
#pragma unroll
      for (int j = 1; j < NT; ++j) mx[0] = max_f(mx[0], s[j]);
      row_max_n<1>(mx);
      if (l16 == 0) atomicMax(&mkey[r], float_key(mx[0]));
    }
    __syncthreads();
    const float m_r = key_float(mkey[r]);
    // p_t = 2^(s_t - m_r) in place of the scores, and the request's mass (an
    // upper estimate of l_c, which sets the histogram's fixed point)
    {
      float psum[1] = {0.0f};
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float e = t_begin + li + j * TPR < t_end[p] ? fast_exp2(s[j] - m_r) : 0.0f;
        s[j] = e;
        psum[0] += e;
      }
      row_sum_n<1>(psum);
      if (l16 == 0) atomicAdd(&lest[r], mass_fix(psum[0]));
    }

    // the contraction's codebook operands (last pass): a wave waits for
    // them where it requests them (two 16-bit values packed per register),
    // so they go out inside the histogram, before its last quarter of slots
    auto load_cvb = [&]() {
#pragma unroll
      for (int st = 0; st < KSL / 32; ++st) {
        const _Float16* src = cvg + (int64_t(m_v) * K + ksl * KSL + st * 32 + 8 * q4) * DS + jt * 16 + l16;
#pragma unroll
        for (int j = 0; j < 8; ++j) cvb[st][j] = src[j * DS];
      }
    };
    constexpr int kCvbSlot = NT >= 2 ? (NT * 3) / 4 : 0;
    if (p == NP - 1 && kCvbSlot == 0) load_cvb();

    // ---- 4. the request's V histogram ---------------------------------------------------
    __syncthreads();   // mass estimates complete
    const float fscale = pow2i(fix_shift(lest[r]));   // bins hold round(p 2^S)
    uint32_t* hr = hist + r * M * K;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (kCvbSlot != 0 && p == NP - 1 && j == kCvbSlot) load_cvb();
      const int t = t_begin + li + j * TPR;
      if (t < t_end[p]) {
        const uint32_t u = uint32_t(fmaf(s[j], fscale, 0.5f));
#pragma unroll
        for (int m = 0; m < M; ++m) atomicAdd(hr + m * K + vcode[p][j].get(m), u);
      }
    }
  }
  __syncthreads();   // histograms complete

  // ---- 5. contraction with the V codebook on the matrix cores ----------------------
  // A rows i < 8: fp16 high part of request i's bins, rows i >= 8 the low
  // part of request i - 8's; the hi and lo lanes each convert half of a
  // step's bins and swap with one DPP move per word.
  const int hh = l16 & 7;
  const bool lo_row = l16 >= 8;
  const int kh = lo_row ? 4 : 0;
  uint32_t raw[KSL / 32][4];
#pragma unroll
  for (int st = 0; st < KSL / 32; ++st) {
    const int k0 = ksl * KSL + st * 32 + 8 * q4 + kh;
#pragma unroll
    for (int v = 0; v < 4; ++v) raw[st][v] = 0;
    if (hh < R) {
      const uint4 w = *reinterpret_cast<const uint4*>(hist + (hh * M + m_v) * K + k0);
      raw[st][0] = w.x; raw[st][1] = w.y; raw[st][2] = w.z; raw[st][3] = w.w;
    }
  }
  // l_c of request hh: the segment-0 waves of the first column tile add
  // their bins in integers (lanes hh and hh + 8 hold complementary bins)
  if (tile == 0) {
    uint32_t lpart = 0;
#pragma unroll
    for (int st = 0; st < KSL / 32; ++st)
#pragma unroll
      for (int v = 0; v < 4; ++v) lpart += raw[st][v];
    lpart += uint32_t(__builtin_amdgcn_mov_dpp(int(lpart), kDppRor8, 0xf, 0xf, true));
    {
      const auto x = __builtin_amdgcn_permlane16_swap(lpart, lpart, false, false);
      lpart = uint32_t(x[0]) + uint32_t(x[1]);
    }
    {
      const auto x = __builtin_amdgcn_permlane32_swap(lpart, lpart, false, false);
      lpart = uint32_t(x[0]) + uint32_t(x[1]);
    }
    if (lane < R) lsum[ksl * R + lane] = lpart;
  }
  f32x4 oa = {0.f, 0.f, 0.f, 0.f}, ob = {0.f, 0.f, 0.f, 0.f};
  const float unfix = pow2i(-fix_shift(lest[hh < R ? hh : 0]));   // 2^-S of this row's request
#pragma unroll
  for (int st = 0; st < KSL / 32; ++st) {
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const float f0 = float(raw[st][2 * v]) * unfix;
      const float f1 = float(raw[st][2 * v + 1]) * unfix;
      const _Float16 h0 = (_Float16)f0, h1 = (_Float16)f1;
      const _Float16 e0 = (_Float16)(f0 - (float)h0), e1 = (_Float16)(f1 - (float)h1);
      hw[v] = uint32_t(__builtin_bit_cast(uint16_t, h0)) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
      lw[v] = uint32_t(__builtin_bit_cast(uint16_t, e0)) | (uint32_t(__builtin_bit_cast(uint16_t, e1)) << 16);
    }
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
  f32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pair_sum32(oa[e] + ob[e]);   // rows 4*q4 + e (hi) and + 8 (lo)

  // ---- 6. write (m, l, o) or the normalised output, per request ----------------------
  float4* part_tile = reinterpret_cast<float4*>(lut);   // [NTILE][64]; the table is dead
  if (ksl == 1) part_tile[tile * 64 + lane] = make_float4(o[0], o[1], o[2], o[3]);
  __syncthreads();
  if (ksl == 0) {
    const float4 other = part_tile[tile * 64 + lane];
    o[0] += other.x; o[1] += other.y; o[2] += other.z; o[3] += other.w;
    const int d = m_v * DS + jt * 16 + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 4 * q4 + e;
      if (rr < R && b0 + rr < a.B) {
        const int64_t row = int64_t(b0 + rr) * a.Hq + g;
        const float mh = key_float(mkey[rr]);
        const float lh = float(lsum[rr] + lsum[R + rr]) * pow2i(-fix_shift(lest[rr]));
        if (a.part_o == nullptr) {
          a.out[row * D + d] = lh > 0.0f ? o[e] * __builtin_amdgcn_rcpf(lh) : 0.0f;
        } else {
          a.part_o[(row * a.C + c) * D + d] = o[e];
          if (d == 0) {
            a.part_m[row * a.C + c] = mh * kLn2;
            a.part_l[row * a.C + c] = lh;
          }
        }
      }
    }
  }
}

}  // namespace pqattn
