// Load-time weight repack: canonical NVFP4 [E, N, K/2] nibbles + [E, N, K/16] scales
// <-> the library's packed tile layout (described in common.h).  A byte permutation (plus
// the sign move of negative block scales, which keeps every value), run once per
// projection when weights are loaded.
#include "common.h"

namespace moe {

// One thread per (expert, 16-row tile, 128-column chunk, lane) unit: 16 nibble bytes
// and 2 scale bytes (layout in common.h).
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
    const int S = scale_group(NC), g = c / S, j = c % S;
    const size_t group = et * NC * kChunkBytes + (size_t)g * S * kChunkBytes;
    const size_t pn = group + (size_t)j * 1024 + 16 * l;     // nibble bytes
    const size_t ps = group + (size_t)S * 1024 + 2 * S * l + 2 * j;  // scale bytes
    const size_t cn = row * (K / 2) + col / 2;
    const size_t cs = row * (K / 16) + col / 16;
    if (!unpack) {
      // a negative block scale: store its magnitude and flip the block's e2m1 signs
      u32x4 v = *(const u32x4*)(nib + cn);
      const uint8_t s0 = scl[cs], s1 = scl[cs + 1];
      const uint32_t f0 = (s0 & 0x80u) ? 0x88888888u : 0u, f1 = (s1 & 0x80u) ? 0x88888888u : 0u;
      v[0] ^= f0;
      v[1] ^= f0;
      v[2] ^= f1;
      v[3] ^= f1;
      *(u32x4*)(packed + pn) = v;
      packed[ps] = s0 & 0x7Fu;
      packed[ps + 1] = s1 & 0x7Fu;
    } else {
      *(u32x4*)(nib_out + cn) = *(const u32x4*)(packed + pn);
      scl_out[cs] = packed[ps];
      scl_out[cs + 1] = packed[ps + 1];
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
