// Nearest-codeword PQ encode kernel (gfx950).
//
// For every vector, head and segment m, the index of the codeword at the
// smallest squared Euclidean distance (AQPIM page, sections 3.1 and
// 5.2 (2)); the lowest index wins a tie.  Since
//   |x - c|^2 = |x|^2 - 2 (x.c - |c|^2 / 2)
// and |x|^2 does not depend on the codeword, the kernel takes the argmax of
// x.c - |c|^2/2.  The dot products of 16 vectors with 16 codewords are one
// matrix-core instruction (fp16 inputs, exact products, fp32 sums) whose
// accumulator starts at -|c|^2/2, so the scores come out ready to compare.
//
// Workgroup = one head and a tile of NV vectors; wave w handles segment
// m = w, holding that segment's 256 codewords in registers as MFMA B
// operands for the whole tile.  Lane (l16, q4) of an instruction's result
// holds vectors 4*q4 .. 4*q4+3 against codeword nt*16 + l16; each lane keeps
// a running best over the 16 codeword tiles, then the 16 lanes of a row
// reduce (score, index) with DPP -- larger score, or equal score and lower
// index, wins.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "decode_kernel.hpp"   // f16x4, f32x4, DPP and argmax helpers

namespace pqattn {

constexpr int kMaxEncodePlanes = 4;

// Up to kMaxEncodePlanes tensors of one shape (e.g. a token's K and V), each
// with its own codebook and code array; blockIdx.z picks the plane.
struct EncodeArgs {
  const __half* x[kMaxEncodePlanes];       // element (n, h, d) at x[n*sxv + h*sxh + d]
  const __half* cb[kMaxEncodePlanes];      // [H][M][K][DS]
  uint8_t* codes[kMaxEncodePlanes];        // code (n, h, m) at codes[s*scs + h*sch + m]
  const int64_t* slots;                    // [N] or null, shared by the planes
  int64_t N;
  int64_t codes_bytes;       // writes outside [0, codes_bytes) are skipped
  int64_t sxv, sxh, scs, sch;
};

template <int M, int NV>
__global__ __launch_bounds__(64 * M) void encode_kernel(EncodeArgs a) {
  constexpr int D = 128;
  constexpr int K = 256;
  constexpr int DS = D / M;
  constexpr int KS = DS / 16;          // MFMA k-steps per segment
  constexpr int NTILE = NV / 16;       // 16-vector tiles
  constexpr int NCT = K / 16;          // 16-codeword tiles

  __shared__ __align__(16) uint8_t cs[NV * M];   // chosen codes [v][m]

  const int lane = threadIdx.x & 63;
  const int m = threadIdx.x >> 6;      // this wave's segment
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int h = blockIdx.y;
  const int plane = blockIdx.z;
  const __half* xp = a.x[plane];
  uint8_t* codes = a.codes[plane];
  const int64_t n0 = int64_t(blockIdx.x) * NV;
  const int nv = int(min<int64_t>(NV, a.N - n0));

  // ---- codebook of (h, m) as MFMA B operands ------------------------------
  const __half* cb = a.cb[plane] + (int64_t(h) * M + m) * K * DS;
  f16x4 bop[NCT][KS];
#pragma unroll
  for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      bop[nt][s] = *reinterpret_cast<const f16x4*>(cb + (nt * 16 + l16) * DS + s * 16 + 4 * q4);

  // A operands (16 vectors x this segment) of one tile; the next tile's are
  // requested while the current one is scored
  auto load_a = [&](int t, f16x4 (&dst)[KS]) {
    const int v = t * 16 + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (v < nv) {
        dst[s] = *reinterpret_cast<const f16x4*>(xp + (n0 + v) * a.sxv + int64_t(h) * a.sxh +
                                                 m * DS + s * 16 + 4 * q4);
      } else {
        dst[s] = f16x4{0, 0, 0, 0};
      }
    }
  };
  f16x4 acur[KS], anext[KS];
  load_a(0, acur);

  // -|c|^2 / 2 of codeword nt*16 + l16: this lane's 4*KS elements, then the
  // four lanes l16, l16+16, l16+32, l16+48 that share the codeword
  float cinit[NCT];
#pragma unroll
  for (int nt = 0; nt < NCT; ++nt) cinit[nt] = neg_half_norm2<KS>(bop[nt]);

  // ---- scores, running argmax, row reduction ------------------------------
  for (int t = 0; t < NTILE; ++t) {
    if (t * 16 >= nv) break;           // uniform over the workgroup
    if (t + 1 < NTILE) load_a(t + 1, anext);
    float best[4];
    int bk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { best[r] = -INFINITY; bk[r] = l16; }
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) {
      f32x4 acc = {cinit[nt], cinit[nt], cinit[nt], cinit[nt]};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(acur[s], bop[nt][s], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool take = acc[r] > best[r];   // ascending codewords: ties keep the lower
        best[r] = take ? acc[r] : best[r];
        bk[r] = take ? nt * 16 + l16 : bk[r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      argmax_step<kDppXor1>(best[r], bk[r]);
      argmax_step<kDppXor2>(best[r], bk[r]);
      argmax_step<kDppRor4>(best[r], bk[r]);
      argmax_step<kDppRor8>(best[r], bk[r]);
    }
    if (l16 == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = t * 16 + 4 * q4 + r;
        if (v < nv) cs[v * M + m] = uint8_t(bk[r]);
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) acur[s] = anext[s];
  }
  __syncthreads();

  for (int v = threadIdx.x; v < nv; v += 64 * M) {
    const int64_t n = n0 + v;
    const int64_t s = a.slots ? a.slots[n] : n;
    if (s < 0 || (a.scs > 0 && s > a.codes_bytes / a.scs)) continue;
    const int64_t off = s * a.scs + int64_t(h) * a.sch;
    if (off < 0 || off + M > a.codes_bytes) continue;
    uint8_t* dst = codes + off;
    if constexpr (M == 4) {
      *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(cs + v * M);
    } else {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(cs + v * M);
    }
  }
}

}  // namespace pqattn
