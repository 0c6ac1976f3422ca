// HBM read probe: how fast this GPU streams a large buffer with 128-bit loads, the
// ceiling the weight-streaming GEMMs are measured against (a measured read roofline, as
// the pages set their layer roofline from a measured read bandwidth rather than the
// spec sheet).  Not part of the layer.
//
// Two load patterns, both non-temporal 16-byte loads per lane (each byte read once):
//  * k_read_stream<U>: every wave owns a contiguous run of 1 KiB pieces (a wave-wide load
//    covers 1 KiB) and keeps U pieces in flight (U = 8, 16, 32);
//  * k_read_items<D>: the grouped GEMM's pattern: a workgroup of 4 waves covers 8
//    consecutive 36 KiB tiles (one work item of the w13 GEMM at K = 4096), each wave
//    walking two tiles side by side, 1 KiB at a time, with D pieces of each in flight.
// The loaded words are XOR-folded per lane and stored only if the fold equals `key`, so
// the loads cannot be dropped and (for all practical keys) nothing is written.
#include "common.h"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kItemTileBytes = 36 * 1024;             // 9 K bytes per 16-row tile at K = 4096
constexpr int kItemBytes = 8 * kItemTileBytes;        // 4 waves x 2 tiles

__device__ __forceinline__ u32x4 load_nt(const uint8_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ void fold_store(u32x4 acc, uint32_t key, uint32_t* sink) {
  const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (f == key) *sink = f;
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void k_read_stream(const uint8_t* __restrict__ src,
                                                               long long npieces, uint32_t key,
                                                               uint32_t* sink) {
  constexpr long long kPiece = 1024LL * U;  // bytes one wave loads per step
  const int lane = threadIdx.x & 63;
  const long long waves = (long long)gridDim.x * (kProbeThreads / 64);
  const long long w = (long long)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  // contiguous run [p0, p1) of U-KiB pieces for this wave
  const long long per = npieces / waves, rem = npieces % waves;
  const long long p0 = w * per + (w < rem ? w : rem);
  const long long p1 = p0 + per + (w < rem ? 1 : 0);
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (p0 >= p1) {
    fold_store(acc, key, sink);
    return;
  }
  const uint8_t* base = src + 16 * lane;
  u32x4 r[U];
#pragma unroll
  for (int u = 0; u < U; ++u) r[u] = load_nt(base + p0 * kPiece + 1024 * u);
  for (long long p = p0; p < p1; ++p) {
    const bool more = p + 1 < p1;  // uniform across the wave
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc ^= r[u];
      if (more) r[u] = load_nt(base + (p + 1) * kPiece + 1024 * u);
    }
  }
  fold_store(acc, key, sink);
}

template <int D>
__global__ __launch_bounds__(kProbeThreads) void k_read_items(const uint8_t* __restrict__ src,
                                                              uint32_t key, uint32_t* sink) {
  constexpr int kPieces = kItemTileBytes / 1024;  // 1 KiB pieces per tile
  static_assert(kPieces % D == 0, "the ring divides the tile");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* t0 = src + (size_t)blockIdx.x * kItemBytes + (size_t)(2 * wave) * kItemTileBytes +
                      16 * lane;
  const uint8_t* t1 = t0 + kItemTileBytes;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 a[D], b[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    a[d] = load_nt(t0 + 1024 * d);
    b[d] = load_nt(t1 + 1024 * d);
  }
  for (int c = 0; c < kPieces; c += D) {
    const bool more = c + D < kPieces;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      acc ^= a[d];
      acc ^= b[d];
      if (more) {
        a[d] = load_nt(t0 + 1024 * (c + D + d));
        b[d] = load_nt(t1 + 1024 * (c + D + d));
      }
    }
  }
  fold_store(acc, key, sink);
}

int probe_variants() { return 5; }

hipError_t launch_read_probe(const uint8_t* src, size_t bytes, int variant, uint32_t key,
                             uint32_t* sink, hipStream_t s) {
  switch (variant) {
    case 0:  // 8 workgroups (32 waves) per CU, 8 KiB in flight per wave
      hipLaunchKernelGGL(k_read_stream<8>, dim3(2048), dim3(kProbeThreads), 0, s, src,
                         (long long)(bytes / 8192), key, sink);
      break;
    case 1:  // the same with 16 KiB in flight per wave
      hipLaunchKernelGGL(k_read_stream<16>, dim3(2048), dim3(kProbeThreads), 0, s, src,
                         (long long)(bytes / 16384), key, sink);
      break;
    case 2:  // 4 workgroups (16 waves) per CU, 16 KiB in flight per wave
      hipLaunchKernelGGL(k_read_stream<16>, dim3(1024), dim3(kProbeThreads), 0, s, src,
                         (long long)(bytes / 16384), key, sink);
      break;
    case 3:  // the GEMM's items, 4 pieces of each tile in flight per wave
      hipLaunchKernelGGL(k_read_items<4>, dim3((unsigned)(bytes / kItemBytes)),
                         dim3(kProbeThreads), 0, s, src, key, sink);
      break;
    default:  // 8 workgroups (32 waves) per CU, 32 KiB in flight per wave: measured on
              // MI355X the fastest of these patterns (1% above 16 KiB; cached instead of
              // non-temporal loads were 12% slower, 64 KiB with 16 waves per CU 9%)
      hipLaunchKernelGGL(k_read_stream<32>, dim3(2048), dim3(kProbeThreads), 0, s, src,
                         (long long)(bytes / 32768), key, sink);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
