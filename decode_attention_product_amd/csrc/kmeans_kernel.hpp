// Codebook learning by Lloyd iterations (gfx950): the update step.
//
// The pages fit each head's codebooks online, on the first vectors of a
// sequence, with a fast K-means over a small sample, and refresh them with a
// few K-means updates every so many tokens (AQPIM page, sections 3.2 (2),
// 5.2 (1) and 6.1 (3)).  One Lloyd iteration is an assignment -- the nearest
// codeword of every segment, which is exactly what encode_kernel computes --
// followed by this update: codeword k of (head h, segment m) moves to the
// mean of the segments assigned to it; a codeword nobody chose keeps its
// value.
//
// One workgroup per (segment m, head h).  An fp16 value times 2^24 is an
// integer of at most 40 bits, so the members' sums are accumulated exactly
// as 64-bit integers with LDS atomics (the order of the additions does not
// matter); the mean is that sum, converted to double, divided by the count
// in double precision (one IEEE rounding) and rounded to the nearest fp16,
// ties to even, straight from the double.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace pqattn {

constexpr int kUpdateThreads = 512;
constexpr int64_t kMaxUpdateVectors = int64_t(1) << 22;   // keeps every sum below 2^62

struct UpdateArgs {
  const __half* x;         // element (n, h, d) at x[n*sxv + h*sxh + d]
  const uint8_t* codes;    // code (n, h, m) at codes[n*scs + h*sch + m]
  __half* cb;              // [H][M][K][DS], updated in place
  uint32_t* counts;        // [H][M][K] members per codeword, or null
  int64_t N;
  int64_t sxv, sxh, scs, sch;
};

// Round a double to the nearest fp16, ties to even, from the double's bits
// (a double -> float -> half chain would round twice).
__device__ __forceinline__ uint16_t f16_bits_rne(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint16_t sign = uint16_t((b >> 48) & 0x8000u);
  const int e = int((b >> 52) & 0x7ff);
  const uint64_t frac = b & ((uint64_t(1) << 52) - 1);
  if (e == 0x7ff) return sign | (frac ? 0x7e00 : 0x7c00);   // NaN, infinity
  if (e == 0) return sign;                                  // below 2^-1022: zero
  const int ex = e - 1023;
  if (ex > 15) return sign | 0x7c00;                        // beyond the fp16 range
  const uint64_t sig = frac | (uint64_t(1) << 52);          // 53-bit significand
  int shift;                                                // significand bits dropped
  uint32_t hexp;
  if (ex >= -14) {
    shift = 42;
    hexp = uint32_t(ex + 15);
  } else {
    shift = 42 + (-14 - ex);                                // fp16 subnormal
    hexp = 0;
    if (shift > 63) return sign;
  }
  const uint64_t kept = sig >> shift;
  const uint64_t rem = sig & ((uint64_t(1) << shift) - 1);
  const uint64_t half = uint64_t(1) << (shift - 1);
  uint32_t r = (hexp << 10) | uint32_t(kept & 0x3ff);
  if (hexp == 0) r = uint32_t(kept);
  if (rem > half || (rem == half && (r & 1u))) r += 1;      // a carry moves into the exponent
  return uint16_t(sign | r);
}

template <int M>
__global__ __launch_bounds__(kUpdateThreads) void codebook_update_kernel(UpdateArgs a) {
  constexpr int D = 128;
  constexpr int K = 256;
  constexpr int DS = D / M;
  constexpr int NTHR = kUpdateThreads;
  constexpr int VPP = NTHR / DS;       // vectors per pass, one lane per dimension
  constexpr int U = 4;                 // passes whose loads are issued together

  __shared__ unsigned long long sums[K * DS];   // x * 2^24 summed per (codeword, dim)
  __shared__ uint32_t cnt[K];

  const int tid = threadIdx.x;
  const int m = blockIdx.x;
  const int h = blockIdx.y;
  for (int i = tid; i < K * DS; i += NTHR) sums[i] = 0;
  for (int i = tid; i < K; i += NTHR) cnt[i] = 0;
  __syncthreads();

  const int j = tid % DS;
  const int v = tid / DS;
  const __half* xh = a.x + int64_t(h) * a.sxh + m * DS + j;
  const uint8_t* ch = a.codes + int64_t(h) * a.sch + m;
  for (int64_t n0 = v; n0 < a.N; n0 += int64_t(U) * VPP) {
    int k[U];
    float xf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t n = n0 + int64_t(u) * VPP;
      k[u] = -1;
      xf[u] = 0.0f;
      if (n < a.N) {
        k[u] = ch[n * a.scs];
        xf[u] = __half2float(xh[n * a.sxv]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k[u] >= 0) {
        // exact: an fp16 value times 2^24 is an integer below 2^40
        const long long fx = (long long)(xf[u] * 16777216.0f);
        atomicAdd(&sums[k[u] * DS + j], (unsigned long long)fx);
        if (j == 0) atomicAdd(&cnt[k[u]], 1u);
      }
    }
  }
  __syncthreads();

  uint16_t* cbh = reinterpret_cast<uint16_t*>(a.cb) + (int64_t(h) * M + m) * K * DS;
  for (int i = tid; i < K * DS; i += NTHR) {
    const uint32_t c = cnt[i / DS];
    if (c > 0) {
      const double sum = double((long long)sums[i]) * 0x1p-24;
      cbh[i] = f16_bits_rne(sum / double(c));
    }
  }
  if (a.counts != nullptr) {
    for (int i = tid; i < K; i += NTHR) a.counts[(int64_t(h) * M + m) * K + i] = cnt[i];
  }
}

}  // namespace pqattn
