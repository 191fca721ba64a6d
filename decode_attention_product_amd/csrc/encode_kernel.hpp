// Nearest-codeword PQ encode kernel (gfx950).
//
// For every vector, head and segment m the index of the codeword at the
// smallest squared Euclidean distance (AQPIM page, sections 3.1 and
// 5.2 (2)); the lowest index wins a tie.  Since |x - c|^2 = |x|^2 + |c|^2 -
// 2 x.c and |x|^2 does not depend on the codeword, the kernel ranks
// |c|^2 - 2 x.c, with x.c from v_dot2_f32_f16 (fp16 products, fp32 sums).
//
// One workgroup owns one head and a tile of NV vectors, staged in LDS.  For
// each segment every lane holds four codewords of that segment in registers
// (k = lane, lane+64, lane+128, lane+192); a wave takes one vector at a
// time, each lane ranks its four codewords, and a butterfly of cross-lane
// exchanges finds the wave's (distance, index) minimum.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace pqattn {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct EncodeArgs {
  const __half* x;           // element (n, h, d) at x[n*sxv + h*sxh + d]
  const __half* cb;          // [H][M][K][DS]
  const int64_t* slots;      // [N] or null
  uint8_t* codes;            // code (n, h, m) at codes[s*scs + h*sch + m]
  int64_t N;
  int64_t codes_bytes;       // writes outside [0, codes_bytes) are skipped
  int64_t sxv, sxh, scs, sch;
};

template <int M, int NV, int NTHR>
__global__ __launch_bounds__(NTHR) void encode_kernel(EncodeArgs a) {
  constexpr int D = 128;
  constexpr int K = 256;
  constexpr int DS = D / M;
  constexpr int NW = NTHR / 64;
  constexpr int R = K / 64;            // codewords per lane

  __shared__ uint4 xs[NV * D / 8];     // the tile's vectors, fp16
  __shared__ __align__(16) uint8_t cs[NV * M];   // chosen codes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  const int64_t n0 = int64_t(blockIdx.x) * NV;
  const int nv = int(min<int64_t>(NV, a.N - n0));

  for (int e = tid; e < nv * (D / 8); e += NTHR) {
    const int v = e / (D / 8), part = e % (D / 8);
    xs[e] = *reinterpret_cast<const uint4*>(a.x + (n0 + v) * a.sxv + int64_t(h) * a.sxh + part * 8);
  }
  __syncthreads();

  for (int m = 0; m < M; ++m) {
    // this lane's codewords of segment m, and their squared norms
    f16x2 cw[R][DS / 2];
    float nrm[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int k = lane + 64 * r;
      const uint4* src = reinterpret_cast<const uint4*>(a.cb + ((int64_t(h) * M + m) * K + k) * DS);
#pragma unroll
      for (int v = 0; v < DS / 8; ++v) {
        uint4 u = src[v];
        const f16x2* p2 = reinterpret_cast<const f16x2*>(&u);
#pragma unroll
        for (int e = 0; e < 4; ++e) cw[r][v * 4 + e] = p2[e];
      }
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < DS / 2; ++j) s = __builtin_amdgcn_fdot2(cw[r][j], cw[r][j], s, false);
      nrm[r] = s;
    }
    for (int v = wave; v < nv; v += NW) {
      f16x2 xv[DS / 2];
      const uint4* xrow = xs + v * (D / 8) + m * (DS / 8);
#pragma unroll
      for (int q = 0; q < DS / 8; ++q) {
        uint4 u = xrow[q];
        const f16x2* p2 = reinterpret_cast<const f16x2*>(&u);
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[q * 4 + e] = p2[e];
      }
      float best = INFINITY;
      int bi = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < DS / 2; ++j) dot = __builtin_amdgcn_fdot2(xv[j], cw[r][j], dot, false);
        const float dist = fmaf(-2.0f, dot, nrm[r]);
        if (dist < best) { best = dist; bi = lane + 64 * r; }   // r ascending: lower k kept on ties
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ob = __shfl_xor(best, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (lane == 0) cs[v * M + m] = uint8_t(bi);
    }
  }
  __syncthreads();

  for (int v = tid; v < nv; v += NTHR) {
    const int64_t n = n0 + v;
    const int64_t s = a.slots ? a.slots[n] : n;
    if (s < 0 || (a.scs > 0 && s > a.codes_bytes / a.scs)) continue;
    const int64_t off = s * a.scs + int64_t(h) * a.sch;
    if (off + M > a.codes_bytes) continue;
    uint8_t* dst = a.codes + off;
    if constexpr (M == 4) {
      *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(cs + v * M);
    } else {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(cs + v * M);
    }
  }
}

}  // namespace pqattn
