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
// Workgroup = one head and a tile of NV vectors (grid: heads fastest, then
// tiles, then planes), 2M waves: wave w handles segment m = w % M against
// codeword half w / M (codewords 128*(w/M) .. +127), holding those 128
// codewords in registers for the whole tile -- half the registers of a
// whole codebook, so four waves fit on a SIMD.  The codewords are the A
// operand of each product and 16 vectors the B operand, so lane (j, q4) of
// a result holds vector j against codewords 4*q4 .. 4*q4+3 of the tile; each
// lane keeps a running best over its half's 8 tiles (larger score, or equal
// score and lower index, wins), two lane swaps combine the four rows, and
// the two halves meet in LDS as order-preserving 64-bit keys.
//
// score_inits, tile_scores and tiles_best_key are the whole arithmetic of a
// decision; codebook learning (kmeans_kernel) calls the same functions, so
// its assignments are this kernel's, decision for decision.
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
  const void* cb[kMaxEncodePlanes];        // [H][M][K][DS], fp16 or E4M3 (the kernel's CbFmt)
  uint8_t* codes[kMaxEncodePlanes];        // code (n, h, m) at codes[s*scs + h*sch + m]
  const int64_t* slots;                    // [N] or null, shared by the planes
  int64_t N;
  int64_t codes_bytes;       // writes outside [0, codes_bytes) are skipped
  int64_t sxv, sxh, scs, sch;
  // Decode step (lens non-null): vector n is request n's new token, written
  // at the slot of token lens[n] - 1 (lens clamped to [0, Lmax]; 0: not
  // written) of its cache -- slot n*Hkv*Lmax + t of a dense one, or through
  // the block table of a paged one (table non-null).
  const int32_t* lens;
  const int32_t* table;      // [N][max_pages]
  int32_t Lmax, Hkv, max_pages, page_shift;
  uint32_t n_pages;
};

// -|c|^2/2 of the codewords of NCT tiles, given as A operands (lane (l16,
// q4) holds dims 4*q4 .. of codeword nt*16 + l16 for every k-step), laid out
// as the accumulator inputs of the products: lane (j, q4) gets those of
// codewords nt*16 + 4*q4 + r, r = 0..3.
template <int KS, int NCT>
__device__ __forceinline__ void score_inits(const f16x4 (&c)[NCT][KS], f32x4 (&cinit)[NCT], int q4) {
  float cn[NCT];
  neg_half_norm2_n<KS, NCT>(c, cn);
#pragma unroll
  for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) cinit[nt][r] = __shfl(cn[nt], 4 * q4 + r, 64);
}

// -|c|^2/2 of one codeword from its DS fp16 values: the value score_inits
// gives it, by the same operations in the same order -- per group q of four
// dimensions (dims s*16 + 4q .. +3 of every k-step s) the fdot2 chain of one
// lane, then (p0 + p1) + (p2 + p3) as the two lane swaps add them.
template <int KS>
__device__ __forceinline__ float neg_half_norm2_row(const _Float16* c) {
  float p[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p[q] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const f16x2 lo = {c[s * 16 + 4 * q], c[s * 16 + 4 * q + 1]};
      const f16x2 hi = {c[s * 16 + 4 * q + 2], c[s * 16 + 4 * q + 3]};
      p[q] = __builtin_amdgcn_fdot2(lo, lo, p[q], false);
      p[q] = __builtin_amdgcn_fdot2(hi, hi, p[q], false);
    }
  }
  return -0.5f * ((p[0] + p[1]) + (p[2] + p[3]));
}

// x.c - |c|^2/2 of 16 vectors (B operand, one f16x4 per k-step) against the
// 16 codewords of one tile (A operand): fp16 products, fp32 sums starting
// from the tile's score_inits.  Lane (j, q4) gets vector j against
// codewords 4*q4 + r.
template <int KS>
__device__ __forceinline__ f32x4 tile_scores(const f16x4 (&c)[KS], const f16x4 (&x)[KS],
                                             const f32x4& init) {
  f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x16f16(c[0], x[0], init, 0, 0, 0);
#pragma unroll
  for (int s = 1; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x16f16(c[s], x[s], acc, 0, 0, 0);
  return acc;
}

// The best (score, index) over NCT tiles of scores (codeword kbase + nt*16 +
// 4*q4 + r for acc[nt][r]) as an argmax key, the same in the four lanes of
// column j.  Each lane takes the largest of its scores (the compiler forms
// three-operand maxima: one instruction per two scores), then the lowest of
// its codewords that holds it, by a scan from the top; rows q4 ^ 1 and
// q4 ^ 2 are then combined by lane swaps.  Ties go to the lowest index, -0
// and +0 counting as equal.
template <int NCT>
__device__ __forceinline__ unsigned long long tiles_best_key(const f32x4 (&acc)[NCT], int kbase,
                                                             int q4) {
  float best = acc[0][0];
#pragma unroll
  for (int i = 1; i < 4 * NCT; ++i) best = fmaxf(best, acc[i / 4][i % 4]);
  int off = (NCT - 1) * 16 + 3;   // the last codeword, unless a lower one holds the maximum
#pragma unroll
  for (int nt = NCT - 1; nt >= 0; --nt)
#pragma unroll
    for (int r = (nt == NCT - 1 ? 2 : 3); r >= 0; --r) off = acc[nt][r] == best ? nt * 16 + r : off;
  int bk = kbase + 4 * q4 + off;
  argmax_pair16(best, bk);   // rows q4 and q4 ^ 1
  argmax_pair32(best, bk);   // rows q4 and q4 ^ 2
  return argmax_key(best, bk);
}

// F: the codebooks' element format (converted to fp16 on load).  SEG: one
// segment per workgroup (two waves, grid z = plane * M + segment), so a
// workgroup loads 1/M of the codebook; for one-tile launches (a decode
// step's new tokens), where the codebook's arrival is most of the time.
template <int M, int NV, CbFmt F = CbFmt::F16, bool SEG = false>
__global__ __launch_bounds__(SEG ? 128 : 128 * M) void encode_kernel(EncodeArgs a) {
  constexpr int D = 128;
  constexpr int K = 256;
  constexpr int DS = D / M;
  constexpr int KS = DS / 16;          // MFMA k-steps per segment
  constexpr int NTILE = NV / 16;       // 16-vector tiles
  constexpr int NCT = K / 32;          // 16-codeword tiles per half

  constexpr int NTHR = SEG ? 128 : 128 * M;
  constexpr int MK = SEG ? 1 : M;      // segments per workgroup
  // per (vector, segment, half): the half's best as an argmax key
  __shared__ unsigned long long keys[NV][MK][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = SEG ? int(blockIdx.z) % M : wave % M;   // this wave's segment
  const int mk = SEG ? 0 : m;
  const int half = SEG ? wave : wave / M;               // and codeword half
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int h = blockIdx.x;            // heads fastest: the heads of one vector row are read together
  const int plane = SEG ? int(blockIdx.z) / M : int(blockIdx.z);
  const __half* xp = a.x[plane];
  uint8_t* codes = a.codes[plane];
  const int64_t n0 = int64_t(blockIdx.y) * NV;
  const int nv = int(min<int64_t>(NV, a.N - n0));

  // ---- this half of the codebook of (h, m) as MFMA A operands ----------------
  const int64_t cb0 = (int64_t(h) * M + m) * K * DS + int64_t(half) * (K / 2) * DS;
  f16x4 bop[NCT][KS];
#pragma unroll
  for (int nt = 0; nt < NCT; ++nt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      bop[nt][s] = cb_load4<F>(a.cb[plane], cb0 + (nt * 16 + l16) * DS + s * 16 + 4 * q4);

  // B operands (16 vectors x this segment) of one tile; the next tile's are
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

  // Where vector v of this workgroup goes: the slot map, or the decode
  // step's lens and block-table lookups; -1: not written.  With one tile of
  // vectors (a decode step's new tokens) the lookups are requested here, so
  // that their round trips overlap the products instead of following the
  // last barrier; with 256-vector tiles (a prefill) they stay at the end,
  // where they measured faster.
  static_assert(NV <= NTHR, "one vector per thread in the write-out");
  auto dest = [&](int v) -> int64_t {
    const int64_t n = n0 + v;
    int64_t s = a.slots ? a.slots[n] : n;
    if (a.lens != nullptr) {
      int l = a.lens[n];
      l = l < 0 ? 0 : (l > a.Lmax ? a.Lmax : l);
      const int t = l - 1;
      if (l == 0) return -1;
      if (a.table != nullptr) {
        const uint32_t pg = min(uint32_t(a.table[n * a.max_pages + (t >> a.page_shift)]), a.n_pages - 1u);
        s = (int64_t(pg) << a.page_shift) | int64_t(t & ((1 << a.page_shift) - 1));
      } else {
        s = n * a.Hkv * a.Lmax + t;
      }
    }
    return s;
  };
  constexpr bool kEarlyDest = NTILE == 1;
  const int vw = threadIdx.x;
  int64_t s_early = -1;
  if constexpr (kEarlyDest) {
    if (vw < nv) s_early = dest(vw);
  }

  f32x4 cinit[NCT];
  score_inits<KS, NCT>(bop, cinit, q4);

  // ---- scores, running argmax, cross-row reduction ---------------------------
  // Transposed products C[i = codeword][j = vector] (the codeword operands
  // are the A side, the vectors the B side; same registers): lane (j, q4)
  // holds vector j against codewords nt*16 + 4*q4 + r, so its running best
  // walks codewords in ascending order within the lane, and the four rows
  // q4 meet in two lane-swap steps.
  const int kbase = half * (K / 2);
  for (int t = 0; t < NTILE; ++t) {
    if (t * 16 >= nv) break;           // uniform over the workgroup
    if (t + 1 < NTILE) load_a(t + 1, anext);
    f32x4 acc[NCT];
#pragma unroll
    for (int nt = 0; nt < NCT; ++nt) acc[nt] = tile_scores<KS>(bop[nt], acur, cinit[nt]);
    const unsigned long long key = tiles_best_key<NCT>(acc, kbase, q4);
    if (q4 == 0) {
      const int v = t * 16 + l16;
      if (v < nv) keys[v][mk][half] = key;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) acur[s] = anext[s];
  }
  __syncthreads();

  if (vw < nv) {
    const int v = vw;
    const int64_t s = kEarlyDest ? s_early : dest(v);
    const bool slot_ok = s >= 0 && !(a.scs > 0 && s > a.codes_bytes / a.scs);
    const int64_t off = slot_ok ? s * a.scs + int64_t(h) * a.sch : -1;
    if (slot_ok && off >= 0 && off + M <= a.codes_bytes) {
      if constexpr (SEG) {   // this workgroup's segment: one byte
        const unsigned long long k0 = keys[v][0][0], k1 = keys[v][0][1];
        codes[off + m] = uint8_t(argmax_key_index(k1 > k0 ? k1 : k0));
      } else {
        int code[M];
#pragma unroll
        for (int j = 0; j < M; ++j) {
          const unsigned long long k0 = keys[v][j][0], k1 = keys[v][j][1];
          code[j] = argmax_key_index(k1 > k0 ? k1 : k0);
        }
        TokenCodes<M> tc;
        tc.set(code);
        tc.store(codes + off);
      }
    }
  }
}

}  // namespace pqattn
