// Fused PQ decode-attention score kernel and chunk-merge kernel (gfx950).
//
// One workgroup owns one (request b, KV head g, chunk c) and the G query
// heads that share g.  It
//   1. builds the lookup table LUT[m][k][h] = q_h[m] . Ck_g[m][k] in LDS
//      (the query's partial dot products with every K codeword, AQPIM page
//      section 4.1, kept on chip as the page's GPU note suggests),
//   2. streams the chunk's K indices from HBM and sums M table entries per
//      token and head -- the score, without rebuilding K,
//   3. keeps the chunk's running max and exp-sum (PAM page, section
//      2.2.3 (1)), rescaling when the max grows between passes,
//   4. streams the V indices and adds each token's probability into a
//      per-(segment, codeword, head) histogram in LDS,
//   5. contracts the histogram with the V codebook,
//        o[h][m*DS + j] = sum_k Hist[m][k][h] * Cv_g[m][k][j],
//      which equals sum_t p_t V_t because V_t is made of codewords,
//   6. writes (m, l, o) for the merge, or the normalised output when the
//      whole cache is one chunk.
// Scores are kept in base-2 units (q is pre-multiplied by scale*log2(e)) so
// the exponentials are single v_exp_f32 instructions; m is written back in
// natural-log units.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace pqattn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeArgs {
  const __half* q;           // [B][Hq][D]
  const uint8_t* k_codes;    // [B][Hkv][Lmax][M]
  const uint8_t* v_codes;
  const __half* k_cb;        // [Hkv][M][K][DS]
  const __half* v_cb;
  const int32_t* lens;       // [B]
  float* part_m;             // [B*Hq][C]
  float* part_l;             // [B*Hq][C]
  float* part_o;             // [B*Hq][C][D]
  float* out;                // [B*Hq][D]; when non-null (C == 1) the normalised
                             // output is written instead of the partials
  int32_t Hq, Hkv, Lmax, T, C;
  float qscale;              // scale * log2(e)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Code bytes of one token: M = 4 -> one dword, M = 8 -> two dwords.
template <int M> struct TokenCodes;
template <> struct TokenCodes<4> {
  uint32_t w;
  __device__ __forceinline__ void load(const uint8_t* p) { w = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ int get(int m) const { return (w >> (8 * m)) & 0xff; }
};
template <> struct TokenCodes<8> {
  uint2 w;
  __device__ __forceinline__ void load(const uint8_t* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ int get(int m) const {
    return ((m < 4 ? w.x : w.y) >> (8 * (m & 3))) & 0xff;
  }
};

// G query heads per KV head, M segments, NT tokens per thread per pass,
// NTHR threads per workgroup.
template <int G, int M, int NT, int NTHR>
__global__ __launch_bounds__(NTHR) void decode_partials_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int K = 256;
  constexpr int DS = D / M;
  constexpr int NW = NTHR / 64;
  constexpr int PASS = NT * NTHR;
  static_assert(NTHR % D == 0, "contraction splits k over NTHR / D slices");

  __shared__ float lut[M * K * G];      // [m][k][h], base-2 scaled scores
  __shared__ float hist[M * K * G];     // [m][k][h], probability mass
  __shared__ float qs[G * D];           // q * scale * log2(e)
  __shared__ float red[NW * G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // XCD-aware order: consecutive workgroups go to different XCDs, so the
  // KV head is the fastest index -- all chunks of one head share an XCD and
  // its L2 copy of that head's codebooks.
  const int64_t id = blockIdx.x;
  const int g = int(id % a.Hkv);
  const int64_t rest = id / a.Hkv;
  const int c = int(rest % a.C);
  const int b = int(rest / a.C);

  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.Lmax ? a.Lmax : len);
  const int t_begin = c * a.T;
  const int t_end = min(t_begin + a.T, len);
  const int64_t row0 = int64_t(b) * a.Hq + int64_t(g) * G;   // first query row

  if (t_begin >= t_end) {   // empty chunk (uniform over the workgroup)
    for (int i = tid; i < G * D; i += NTHR) {
      const int h = i / D, d = i % D;
      if (a.out != nullptr) {
        a.out[(row0 + h) * D + d] = 0.0f;
      } else {
        a.part_o[((row0 + h) * a.C + c) * D + d] = 0.0f;
        if (d == 0) {
          a.part_m[(row0 + h) * a.C + c] = -INFINITY;
          a.part_l[(row0 + h) * a.C + c] = 0.0f;
        }
      }
    }
    return;
  }

  // ---- stage the G queries, pre-scaled ------------------------------------
  for (int i = tid; i < G * D; i += NTHR)
    qs[i] = __half2float(a.q[row0 * D + i]) * a.qscale;
  for (int i = tid; i < M * K * G; i += NTHR) hist[i] = 0.0f;
  __syncthreads();

  // ---- LUT build: one (m, k) codeword per thread iteration ----------------
  {
    const __half* cbk = a.k_cb + int64_t(g) * M * K * DS;
    for (int p = tid; p < M * K; p += NTHR) {
      const int m = p / K;
      float cw[DS];
      const uint4* src = reinterpret_cast<const uint4*>(cbk + int64_t(p) * DS);
#pragma unroll
      for (int v = 0; v < DS / 8; ++v) {
        uint4 u = src[v];
        const __half* hh = reinterpret_cast<const __half*>(&u);
#pragma unroll
        for (int e = 0; e < 8; ++e) cw[v * 8 + e] = __half2float(hh[e]);
      }
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < DS; ++j) s = fmaf(qs[h * D + m * DS + j], cw[j], s);
        acc[h] = s;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) lut[p * G + h] = acc[h];
    }
  }
  __syncthreads();

  const int64_t bg = int64_t(b) * a.Hkv + g;
  const uint8_t* kc = a.k_codes + bg * a.Lmax * M;
  const uint8_t* vc = a.v_codes + bg * a.Lmax * M;

  float m_run[G], l_thr[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m_run[h] = -INFINITY; l_thr[h] = 0.0f; }

  for (int tp = t_begin; tp < t_end; tp += PASS) {
    // ---- scores of this pass ----------------------------------------------
    float s[NT][G];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = tp + i * NTHR + tid;
      if (t < t_end) {
        TokenCodes<M> code;
        code.load(kc + int64_t(t) * M);
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = 0.0f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float* e = lut + (m * K + code.get(m)) * G;
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] += e[h];
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = -INFINITY;
      }
    }
    // ---- pass max over the workgroup ----------------------------------------
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int i = 1; i < NT; ++i) mx = fmaxf(mx, s[i][h]);
      mx = wave_max(mx);
      if (lane == 0) red[wave * G + h] = mx;
    }
    __syncthreads();
    bool grew = false;
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = red[h];
#pragma unroll
      for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red[w * G + h]);
      const float m_new = fmaxf(m_run[h], mx);
      alpha[h] = (m_run[h] == -INFINITY) ? 0.0f : fast_exp2(m_run[h] - m_new);
      grew |= (m_run[h] != -INFINITY) && (m_new > m_run[h]);
      m_run[h] = m_new;
      l_thr[h] *= alpha[h];
    }
    if (grew) {   // uniform: every thread saw the same maxima
      // NTHR is a multiple of G, so this thread always touches head tid % G
      float a_mine = alpha[0];
#pragma unroll
      for (int h = 1; h < G; ++h) a_mine = (tid % G == h) ? alpha[h] : a_mine;
      for (int i = tid; i < M * K * G; i += NTHR) hist[i] *= a_mine;
    }
    __syncthreads();
    // ---- probabilities into the V histogram ---------------------------------
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = tp + i * NTHR + tid;
      if (t < t_end) {
        float p[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          p[h] = fast_exp2(s[i][h] - m_run[h]);
          l_thr[h] += p[h];
        }
        TokenCodes<M> code;
        code.load(vc + int64_t(t) * M);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float* e = hist + (m * K + code.get(m)) * G;
#pragma unroll
          for (int h = 0; h < G; ++h) atomicAdd(e + h, p[h]);
        }
      }
    }
  }

  // ---- chunk sum l ------------------------------------------------------------
  __syncthreads();   // histogram complete; red free
  float l_sum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = wave_sum(l_thr[h]);
    if (lane == 0) red[wave * G + h] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w * G + h];
    l_sum[h] = v;
  }

  // ---- contraction with the V codebook ---------------------------------------
  // thread -> column (m, j) and a slice of the codewords; slices are summed
  // through LDS (the LUT is no longer needed).
  constexpr int KS = NTHR / D;            // codeword slices
  constexpr int KPER = K / KS;
  {
    const int col = tid % D;
    const int ks = tid / D;
    const int m = col / DS;
    const int j = col % DS;
    const __half* cbv = a.v_cb + int64_t(g) * M * K * DS + int64_t(m) * K * DS + j;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0f;
    const int k0 = ks * KPER;
    for (int k = k0; k < k0 + KPER; ++k) {
      const float w = __half2float(cbv[int64_t(k) * DS]);
      const float* e = hist + (m * K + k) * G;
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fmaf(e[h], w, acc[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) lut[(ks * G + h) * D + col] = acc[h];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += NTHR) {
    const int h = i / D, d = i % D;
    float o = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) o += lut[(ks * G + h) * D + d];
    if (a.out != nullptr) {
      const float l = l_sum[h];
      a.out[(row0 + h) * D + d] = l > 0.0f ? o / l : 0.0f;
    } else {
      a.part_o[((row0 + h) * a.C + c) * D + d] = o;
      if (d == 0) {
        a.part_m[(row0 + h) * a.C + c] = m_run[h] * kLn2;
        a.part_l[(row0 + h) * a.C + c] = l_sum[h];
      }
    }
  }
}

// Merge of chunk statistics: one workgroup of D threads per row.
struct ReduceArgs {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  float* out;
  int32_t C;
};

__global__ __launch_bounds__(128) void reduce_kernel(ReduceArgs a) {
  constexpr int D = 128;
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float* pm = a.part_m + row * a.C;
  const float* pl = a.part_l + row * a.C;
  const float* po = a.part_o + row * a.C * D + d;
  float m_star = -INFINITY;
  for (int c = 0; c < a.C; ++c) m_star = fmaxf(m_star, pm[c]);
  float num = 0.0f, den = 0.0f;
  if (m_star != -INFINITY) {
    for (int c = 0; c < a.C; ++c) {
      const float mc = pm[c];
      if (mc == -INFINITY) continue;
      const float w = fast_exp2((mc - m_star) * kLog2e);
      num = fmaf(w, po[int64_t(c) * D], num);
      den = fmaf(w, pl[c], den);
    }
  }
  a.out[row * D + d] = den > 0.0f ? num / den : 0.0f;
}

}  // namespace pqattn
