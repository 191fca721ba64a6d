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
// An fp16 value times 2^24 is an integer of at most 40 bits, so the
// members' sums are accumulated exactly as 64-bit integers with LDS atomics
// (the order of the additions does not matter); the mean is that sum,
// converted to double, divided by the count in double precision (one IEEE
// rounding) and rounded to the nearest fp16, ties to even, straight from the
// double.
//
// codebook_update_kernel: the update step alone, one workgroup per (segment
// m, head h).  kmeans_kernel: whole Lloyd runs in one launch, one workgroup
// per (segment, head, plane) holding the segment's codebook in LDS and
// alternating the assignment -- the encode kernel's own score and argmax
// functions, so the same decisions -- with the update, for samples of up to
// kMaxFusedVectors vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "encode_kernel.hpp"   // score_inits, tile_scores, tiles_best_key

namespace pqattn {

constexpr int kUpdateThreads = 512;
constexpr int64_t kMaxUpdateVectors = int64_t(1) << 22;   // keeps every sum below 2^62
constexpr int kKmeansThreads = 512;
constexpr int kMaxFusedVectors = 8192;
constexpr int kMaxKmeansPlanes = 2;
constexpr int kStageVectors = 1024;   // samples up to this size are kept in LDS

struct UpdateArgs {
  const __half* x;         // element (n, h, d) at x[n*sxv + h*sxh + d]
  const uint8_t* codes;    // code (n, h, m) at codes[n*scs + h*sch + m]
  __half* cb;              // [H][M][K][DS], updated in place
  uint32_t* counts;        // [H][M][K] members per codeword, or null
  int64_t N;
  int64_t sxv, sxh, scs, sch;
};

// Round a double to the nearest fp16, ties to even, with one rounding:
// first to float rounding to odd (truncate toward zero, then set the last
// bit if anything was cut off), then the hardware's round-to-nearest-even
// to fp16.  Float keeps 13 more bits than fp16, more than the 2 that make
// the two steps equal one correct rounding; a plain double -> float -> fp16
// chain would round twice.
__device__ __forceinline__ uint16_t f16_bits_rne(double v) {
  const float f = float(v);
  uint32_t fb = __builtin_bit_cast(uint32_t, f);
  const double back = double(f);
  if (back != v) {
    if (__builtin_fabs(back) > __builtin_fabs(v)) fb -= 1u;   // it went away from zero
    fb |= 1u;
  }
  return __builtin_bit_cast(uint16_t, (_Float16)__builtin_bit_cast(float, fb));
}

// x * 2^24 as an integer, exactly, from the bits of a finite fp16 x:
// (1024 + mantissa) << (exponent - 1) for normal numbers, the mantissa for
// subnormal ones; below 2^41 in magnitude.
__device__ __forceinline__ long long f16_fixed24(uint32_t hb) {
  const uint32_t e = (hb >> 10) & 31u;
  const uint32_t mnt = hb & 1023u;
  const uint32_t sig = e ? (mnt | 1024u) : mnt;
  const long long mag = (long long)((unsigned long long)sig << (e ? e - 1 : 0));
  return (hb & 0x8000u) ? -mag : mag;
}

// Adds every member's segment (x * 2^24, exact) into sums[code][j] and
// counts it in cnt[code], code = code_of(n), for n < N; x_bits(n, j) gives
// the fp16 bits of dimension j of vector n's segment.  Called by all NTHR
// threads; sums and cnt must be zero and visible.
template <int DS, int NTHR, class CodeOf, class XBits>
__device__ __forceinline__ void accumulate_members(int64_t N, CodeOf code_of, XBits x_bits,
                                                   unsigned long long* sums, uint32_t* cnt) {
  constexpr int VPP = NTHR / DS;       // vectors per pass, one lane per dimension
  constexpr int U = 8;                 // passes whose loads are issued together
  const int j = threadIdx.x % DS;
  const int v = threadIdx.x / DS;
  for (int64_t n0 = v; n0 < N; n0 += int64_t(U) * VPP) {
    int k[U];
    uint32_t xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t n = n0 + int64_t(u) * VPP;
      k[u] = -1;
      xv[u] = 0;
      if (n < N) {
        k[u] = code_of(n);
        xv[u] = x_bits(n, j);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k[u] >= 0) {
        atomicAdd(&sums[k[u] * DS + j], (unsigned long long)f16_fixed24(xv[u]));
        if (j == 0) atomicAdd(&cnt[k[u]], 1u);
      }
    }
  }
}

// The mean of codeword k's members, rounded to fp16 (bits).
template <int DS>
__device__ __forceinline__ uint16_t member_mean(const unsigned long long* sums, uint32_t c, int i) {
  const double sum = double((long long)sums[i]) * 0x1p-24;
  return f16_bits_rne(sum / double(c));
}

// The means of the codewords with members, rounded to fp16, into dst (fp16
// bits, [K][DS]); the others are left as they are.
template <int DS, int NTHR>
__device__ __forceinline__ void store_means(const unsigned long long* sums, const uint32_t* cnt,
                                            uint16_t* dst) {
  constexpr int K = 256;
  for (int i = threadIdx.x; i < K * DS; i += NTHR) {
    const uint32_t c = cnt[i / DS];
    if (c > 0) dst[i] = member_mean<DS>(sums, c, i);
  }
}

template <int M>
__global__ __launch_bounds__(kUpdateThreads) void codebook_update_kernel(UpdateArgs a) {
  constexpr int K = 256;
  constexpr int DS = 128 / M;
  constexpr int NTHR = kUpdateThreads;
  __shared__ unsigned long long sums[K * DS];   // x * 2^24 summed per (codeword, dim)
  __shared__ uint32_t cnt[K];

  const int m = blockIdx.x;
  const int h = blockIdx.y;
  for (int i = threadIdx.x; i < K * DS; i += NTHR) sums[i] = 0;
  for (int i = threadIdx.x; i < K; i += NTHR) cnt[i] = 0;
  __syncthreads();
  const uint8_t* ch = a.codes + int64_t(h) * a.sch + m;
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.x) + int64_t(h) * a.sxh + m * DS;
  accumulate_members<DS, NTHR>(
      a.N, [&](int64_t n) { return int(ch[n * a.scs]); },
      [&](int64_t n, int j) { return uint32_t(xb[n * a.sxv + j]); }, sums, cnt);
  __syncthreads();
  store_means<DS, NTHR>(sums, cnt, reinterpret_cast<uint16_t*>(a.cb) + (int64_t(h) * M + m) * K * DS);
  if (a.counts != nullptr) {
    for (int i = threadIdx.x; i < K; i += NTHR) a.counts[(int64_t(h) * M + m) * K + i] = cnt[i];
  }
}

// Lloyd runs of 1 or 2 planes (e.g. the K and V samples of one layer).
struct KmeansArgs {
  const __half* x[kMaxKmeansPlanes];   // element (n, h, d) at x[n*sxv + h*sxh + d]
  __half* cb[kMaxKmeansPlanes];        // [H][M][K][DS]: the start in, the learned codebook out
  uint8_t* codes[kMaxKmeansPlanes];    // code (n, h, m) at codes[n*scs + h*sch + m]
  int64_t N;                           // <= kMaxFusedVectors
  int64_t sxv, sxh, scs, sch, codes_bytes;
  int32_t n_iter;
};

// Where a staged sample keeps group g (4 dims, 8 bytes) of vector v's
// segment, in halves: rows of DS halves with the groups XOR-swizzled by the
// row's place in its bank cycle, so 16 lanes reading one group of 16
// consecutive rows hit 16 different bank pairs.
template <int DS>
__device__ __forceinline__ int staged_offset(int v, int g) {
  constexpr int G = DS / 4;              // groups per row
  constexpr int RPB = 128 / DS;          // rows per 256-byte bank cycle
  return v * DS + ((g ^ ((v / RPB) & (G - 1))) * 4);
}

// The Lloyd iterations of one (segment, head) workgroup.  x_group(v, g)
// gives group g (dims 4g .. 4g+3) of vector v's segment as f16x4 and
// x_bits(n, j) dimension j's fp16 bits.  cbs holds the codebook segment,
// rows CP halves apart (padded so that 16 lanes reading 16 rows hit
// different banks); on return it holds the learned one and code[] the
// sample's final codes.  sums and cnt start at zero, nlist[0..1] too.
template <int M, int CP, class XGroup, class XBits>
__device__ __forceinline__ void lloyd_iterations(XGroup x_group, XBits x_bits, int N, int n_iter,
                                                 uint16_t* cbs, float* cnorm,
                                                 unsigned long long* sums, uint32_t* cnt,
                                                 uint8_t* code, uint8_t* list, uint32_t* nlist) {
  constexpr int K = 256;
  constexpr int DS = 128 / M;
  constexpr int KS = DS / 16;          // MFMA k-steps per segment
  constexpr int NCT = K / 16;          // all 16 codeword tiles in every wave
  constexpr int NTHR = kKmeansThreads;
  constexpr int NW = NTHR / 64;
  constexpr int GD = DS * K / NTHR;    // dims per thread when the means are formed
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int ntile = (N + 15) / 16;
  auto load_x = [&](int t, f16x4 (&xv)[KS]) {
    const int v = t * 16 + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) xv[s] = v < N ? x_group(v, s * 4 + q4) : f16x4{0, 0, 0, 0};
  };
  for (int it = 0;; ++it) {
    const int par = it & 1;
    // ---- the codewords' -|c|^2/2 once, one thread per codeword; the codewords
    // the last update listed get their counts cleared for this one ----------
    if (tid < K) cnorm[tid] = neg_half_norm2_row<KS>(reinterpret_cast<const _Float16*>(cbs + tid * CP));
    {
      const uint32_t nl = nlist[par ^ 1];
      for (uint32_t i = tid; i < nl; i += NTHR) cnt[list[i]] = 0;
    }
    __syncthreads();
    if (tid == 0) nlist[par ^ 1] = 0;   // read by no thread until two iterations on

    // ---- assignment: the nearest codeword of every vector's segment --------
    f16x4 c[NCT][KS];
    f32x4 cinit[NCT];
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        c[nt][s] = *reinterpret_cast<const f16x4*>(cbs + (nt * 16 + l16) * CP + s * 16 + 4 * q4);
      const float4 cn = *reinterpret_cast<const float4*>(cnorm + nt * 16 + 4 * q4);
      cinit[nt] = f32x4{cn.x, cn.y, cn.z, cn.w};
    }
    f16x4 xcur[KS], xnext[KS];
    if (wave < ntile) load_x(wave, xcur);
    for (int t = wave; t < ntile; t += NW) {
      if (t + NW < ntile) load_x(t + NW, xnext);
      // the two codeword halves one after the other (as the encode kernel's
      // two waves do), the larger key wins
      unsigned long long key = 0;
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        f32x4 acc[NCT / 2];
#pragma unroll
        for (int nt = 0; nt < NCT / 2; ++nt)
          acc[nt] = tile_scores<KS>(c[g2 * (NCT / 2) + nt], xcur, cinit[g2 * (NCT / 2) + nt]);
        const unsigned long long kh = tiles_best_key<NCT / 2>(acc, g2 * (K / 2), q4);
        key = kh > key ? kh : key;
      }
      const int v = t * 16 + l16;
      if (q4 == 0 && v < N) code[v] = uint8_t(argmax_key_index(key));
#pragma unroll
      for (int s = 0; s < KS; ++s) xcur[s] = xnext[s];
    }
    __syncthreads();
    if (it == n_iter) break;

    // ---- update: every chosen codeword to the mean of its members ----------
    accumulate_members<DS, NTHR>(N, [&](int64_t n) { return int(code[n]); }, x_bits, sums, cnt);
    __syncthreads();
    if (tid < K) {   // list the codewords with members: one slot range per wave
      const bool has = cnt[tid] > 0;
      const unsigned long long mask = __ballot(has);
      uint32_t base = 0;
      if (lane == 0 && mask != 0) base = atomicAdd(&nlist[par], uint32_t(__popcll(mask)));
      base = __shfl(base, 0, 64);
      if (has) list[base + __popcll(mask & ((1ull << lane) - 1))] = uint8_t(tid);
    }
    __syncthreads();
    {   // thread t: listed codeword t / (DS / GD), GD of its dims; sums back to zero
      const uint32_t e = uint32_t(tid) / (DS / GD);
      if (e < nlist[par]) {
        const int k = list[e];
        const uint32_t n = cnt[k];
        const int j0 = (tid % (DS / GD)) * GD;
#pragma unroll
        for (int jj = 0; jj < GD; ++jj) {
          cbs[k * CP + j0 + jj] = member_mean<DS>(sums, n, k * DS + j0 + jj);
          sums[k * DS + j0 + jj] = 0;
        }
      }
    }
    __syncthreads();
  }
}

template <int M>
__global__ __launch_bounds__(kKmeansThreads) void kmeans_kernel(KmeansArgs a) {
  constexpr int K = 256;
  constexpr int DS = 128 / M;
  constexpr int CP = DS + 4;           // padded row pitch of the LDS codebook, halves
  constexpr int NTHR = kKmeansThreads;

  __shared__ __align__(16) uint16_t cbs[K * CP];          // the current codebook segment
  __shared__ __align__(16) float cnorm[K];                // its -|c|^2/2
  __shared__ unsigned long long sums[K * DS];
  __shared__ uint32_t cnt[K];
  __shared__ uint8_t list[K];                             // codewords with members
  __shared__ uint32_t nlist[2];
  __shared__ uint8_t code[kMaxFusedVectors];
  __shared__ __align__(16) uint16_t xst[kStageVectors * DS];   // the sample's segments, when staged

  const int tid = threadIdx.x;
  const int m = blockIdx.x;
  const int h = blockIdx.y;
  const int plane = blockIdx.z;
  const int N = int(a.N);
  const __half* xh = a.x[plane] + int64_t(h) * a.sxh + m * DS;   // vector n at xh + n*sxv
  uint16_t* cbg = reinterpret_cast<uint16_t*>(a.cb[plane]) + (int64_t(h) * M + m) * K * DS;

  for (int i = tid; i < K * DS / 4; i += NTHR) {   // 8 bytes at a time into the padded rows
    const int k = i / (DS / 4), q = i % (DS / 4);
    *reinterpret_cast<uint2*>(cbs + k * CP + 4 * q) = reinterpret_cast<const uint2*>(cbg)[i];
  }
  for (int i = tid; i < K * DS; i += NTHR) sums[i] = 0;
  for (int i = tid; i < K; i += NTHR) cnt[i] = 0;
  if (tid < 2) nlist[tid] = 0;
  const bool staged = N <= kStageVectors;   // uniform
  if (staged) {   // each vector's segment once, 8 bytes per thread and step
    for (int i = tid; i < N * (DS / 4); i += NTHR) {
      const int v = i / (DS / 4), g = i % (DS / 4);
      *reinterpret_cast<uint2*>(xst + staged_offset<DS>(v, g)) =
          *reinterpret_cast<const uint2*>(xh + int64_t(v) * a.sxv + 4 * g);
    }
  }
  __syncthreads();
  if (staged) {
    lloyd_iterations<M, CP>(
        [&](int v, int g) { return *reinterpret_cast<const f16x4*>(xst + staged_offset<DS>(v, g)); },
        [&](int64_t n, int j) { return uint32_t(xst[staged_offset<DS>(int(n), j >> 2) + (j & 3)]); },
        N, a.n_iter, cbs, cnorm, sums, cnt, code, list, nlist);
  } else {
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(xh);
    lloyd_iterations<M, CP>(
        [&](int v, int g) {
          return *reinterpret_cast<const f16x4*>(xh + int64_t(v) * a.sxv + 4 * g);
        },
        [&](int64_t n, int j) { return uint32_t(xb[n * a.sxv + j]); },
        N, a.n_iter, cbs, cnorm, sums, cnt, code, list, nlist);
  }

  for (int i = tid; i < K * DS / 4; i += NTHR) {
    const int k = i / (DS / 4), q = i % (DS / 4);
    reinterpret_cast<uint2*>(cbg)[i] = *reinterpret_cast<const uint2*>(cbs + k * CP + 4 * q);
  }
  uint8_t* cp = a.codes[plane];
  for (int v = tid; v < N; v += NTHR) {
    const int64_t off = int64_t(v) * a.scs + int64_t(h) * a.sch + m;
    if (off >= 0 && off < a.codes_bytes) cp[off] = code[v];
  }
}

}  // namespace pqattn
