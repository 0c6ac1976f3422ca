// Load-time weight repack: canonical NVFP4 [E, N, K/2] nibbles + [E, N, K/16] scales
// <-> the library's packed tile layout (described in common.h).  A pure byte permutation,
// run once per projection when weights are loaded.
#include "common.h"

namespace moe {

// One thread per (expert, 16-row tile, 128-column chunk, lane) unit: 16 nibble bytes
// and 2 scale bytes.
__global__ void k_pack(const uint8_t* __restrict__ nib, const uint8_t* __restrict__ scl,
                       uint8_t* __restrict__ packed, int E, int N, int K, bool unpack,
                       uint8_t* __restrict__ nib_out, uint8_t* __restrict__ scl_out) {
  const int NC = K / 128, TILES = N / 16;
  const size_t units = (size_t)E * TILES * NC * 64;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(u % 64);
    const size_t chunk = u / 64;               // global chunk index: (e, t, c) row-major
    const int c = (int)(chunk % NC);
    const size_t et = chunk / NC;              // e * TILES + t
    const int t = (int)(et % TILES);
    const size_t e = et / TILES;
    const size_t row = e * N + 16 * (size_t)t + (l & 15);
    const int col = 128 * c + 32 * (l >> 4);  // first of the lane's 32 elements
    const size_t base = chunk * kChunkBytes;
    const size_t cn = row * (K / 2) + col / 2;
    const size_t cs = row * (K / 16) + col / 16;
    if (!unpack) {
      *(u32x4*)(packed + base + 16 * l) = *(const u32x4*)(nib + cn);
      packed[base + 1024 + 2 * l] = scl[cs];
      packed[base + 1024 + 2 * l + 1] = scl[cs + 1];
    } else {
      *(u32x4*)(nib_out + cn) = *(const u32x4*)(packed + base + 16 * l);
      scl_out[cs] = packed[base + 1024 + 2 * l];
      scl_out[cs + 1] = packed[base + 1024 + 2 * l + 1];
    }
  }
}

hipError_t launch_pack(const uint8_t* nib, const uint8_t* scl, int E, int N, int K, uint8_t* packed,
                       bool unpack, uint8_t* nib_out, uint8_t* scl_out, hipStream_t s) {
  const size_t units = (size_t)E * (N / 16) * (K / 128) * 64;
  if (units == 0) return hipSuccess;
  const size_t blocks = (units + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(k_pack, dim3(grid), dim3(256), 0, s, nib, scl, packed, E, N, K, unpack,
                     nib_out, scl_out);
  return hipGetLastError();
}

}  // namespace moe
