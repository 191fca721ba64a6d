// Read-only HBM streaming reference for the benchmark (libpqbench.so): one
// launch reads a buffer once, 16 bytes per load, and folds it into one 32-bit
// XOR checksum per workgroup (reduced in LDS, one plain store each: no
// atomics on a shared address), so nothing is written but four bytes per
// workgroup.  What it reaches for a given size and grid is the ceiling a
// single launch of a bandwidth-bound kernel of that size has on the box.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kInFlight = 4;   // 16-byte loads each thread keeps in flight

__global__ void stream_read_kernel(const uint4* __restrict__ src, uint64_t n16, uint32_t* checksums) {
  __shared__ uint32_t wave_acc[16];
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    uint4 v[kInFlight];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) v[j] = src[i + j * stride];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // the last (fewer than kInFlight) rounds: every load issued before any use
  uint4 v[kInFlight - 1];
#pragma unroll
  for (int j = 0; j < kInFlight - 1; ++j)
    v[j] = i + j * stride < n16 ? src[i + j * stride] : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < kInFlight - 1; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) wave_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (unsigned w = 0; w < blockDim.x / 64; ++w) x ^= wave_acc[w];
    checksums[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16; src 16-byte aligned) from src once with
// a grid of `grid` workgroups of `block` threads (a multiple of 64, at most
// 1024) and writes checksums[g] = the XOR of the 32-bit words workgroup g
// read (checksums has `grid` entries; their XOR is the buffer's).  Returns
// the hipError_t of the launch (0 = success); invalid arguments return
// hipErrorInvalidValue and launch nothing.
int pqbench_stream_read(const void* src, uint64_t bytes, uint32_t* checksums, int grid, int block,
                        void* stream) {
  if (!src || !checksums || (bytes & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u) || grid < 1 ||
      block < 64 || block > 1024 || (block & 63))
    return int(hipErrorInvalidValue);
  const uint4* s = static_cast<const uint4*>(src);
  uint64_t n16 = bytes / 16;
  uint32_t* c = checksums;
  void* args[] = {&s, &n16, &c};
  return int(hipLaunchKernel(reinterpret_cast<const void*>(&stream_read_kernel), dim3(unsigned(grid)),
                             dim3(unsigned(block)), args, 0, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
