// Grouped NVFP4 GEMM: out[i, n] = sum_k a(i, k) * w_e(n, k) for every row i of every
// non-empty expert group e (alpha = 1; the globals are applied by the next kernel).
//
// The GEMM is weight-stream bound: every active expert's packed weights are read from HBM
// exactly once, with one 16-byte (nibbles) and one 2-byte (scales) load per lane per
// 16-row tile per 128-column chunk — 1152 contiguous bytes per wave — and a ring of D
// chunks in flight per wave.
//
// Work decomposition: a work item is (expert, 4 * NS consecutive 16-row tiles); each of
// the 4 waves of a workgroup streams NS tiles over all of K.  A persistent grid walks the
// items round-robin, so workgroups differ by at most one item.
//
// Two kernels, each over the groups its path owns (chosen per group on the device, so
// the host never needs the group sizes):
//  * k_gemm_mfma: the weight tile is the A operand of v_mfma_f32_16x16x32_f16 (16 weight
//    rows x 32 k), the group's activation rows the B operand (16 columns, zero-padded),
//    CT column tiles (16 * CT rows) per pass.  Lane l holds weight row l & 15 and the 32
//    k of quarter l >> 4 of each 128-column chunk; MFMA j of the chunk takes word j
//    (8 k) of that quarter, and the B operand uses the same k assignment.
//  * k_gemm_gemv (groups of at most 4 rows): each lane dots its weight row segment with
//    each activation row's matching segment, 16 elements (one scale block) at a time with
//    v_dot2_f32_f16, then multiplies by the weight block scale; the four k-quarters are
//    summed across lanes at the end in a fixed tree.
// Both dequantize exactly (dequant8 in common.h) and accumulate in fp32 in an order that
// depends only on (N, K) and the path, never on the other rows of the group.
#include "common.h"

#include <mutex>

#ifndef MOE_GEMM_NS
#define MOE_GEMM_NS 4  // 16-row tiles per wave, MFMA kernel
#endif
#ifndef MOE_GEMM_D
#define MOE_GEMM_D 2   // chunks in flight per wave, MFMA kernel
#endif
#ifndef MOE_GEMM_CT
#define MOE_GEMM_CT 2  // 16-row activation column tiles per MFMA pass
#endif
#ifndef MOE_GEMV_NS
#define MOE_GEMV_NS 2  // 16-row tiles per wave, GEMV kernel
#endif
#ifndef MOE_GEMV_D
#define MOE_GEMV_D 2
#endif

namespace moe {

constexpr int kGemmWaves = 4;
constexpr int kGemvRows = 4;

struct GemmArgs {
  const uint8_t* aq;
  const uint8_t* as;
  const int32_t* off;
  int E;
  const uint8_t* w;
  int N, K;
  float* out;
  int gmin, gmax;  // this kernel's groups: gmin <= G <= gmax
};

// Ids of the experts whose group size is in [gmin, gmax], ascending, into LDS (wave 0).
__device__ __forceinline__ int build_active_list(const GemmArgs& p, uint16_t* s_act, int* s_nact) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int n = 0;
    for (int base = 0; base < p.E; base += 64) {
      const int e = base + lane;
      bool a = false;
      if (e < p.E) {
        const int g = p.off[e + 1] - p.off[e];
        a = g >= p.gmin && g <= p.gmax;
      }
      const uint64_t m = __ballot(a);
      if (a) s_act[n + __popcll(m & below)] = (uint16_t)e;
      n += __popcll(m);
    }
    if (lane == 0) *s_nact = n;
  }
  __syncthreads();
  return *s_nact;
}

// ------------------------------------------------------------------------- MFMA path
template <int NS, int D, int CT>
__device__ __forceinline__ void mfma_pass(const GemmArgs& p, const uint8_t* __restrict__ wt,
                                          int nsv, int arow0, int nrows, int col0) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, r = lane & 15;
  const int K = p.K, NC = K / 128;
  const size_t tstride = (size_t)NC * kChunkBytes;

  const uint8_t* aqp[CT];
  const uint8_t* asp[CT];
  bool av[CT];
#pragma unroll
  for (int a = 0; a < CT; ++a) {
    av[a] = 16 * a + r < nrows;
    const int row = arow0 + (av[a] ? 16 * a + r : 0);
    aqp[a] = p.aq + (size_t)row * (K / 2) + 16 * kq;
    asp[a] = p.as + (size_t)row * (K / 16) + 2 * kq;
  }

  u32x4 wn[D][NS];
  uint32_t ws[D][NS];
  u32x4 an[D][CT];
  uint32_t asc[D][CT];
  f32x4 acc[NS][CT];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int a = 0; a < CT; ++a) acc[s][a] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int c, int slot) {
    const size_t off = (size_t)c * kChunkBytes;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s < nsv) {
        const uint8_t* t = wt + s * tstride + off;
        wn[slot][s] = *(const u32x4*)(t + 16 * lane);
        ws[slot][s] = *(const uint16_t*)(t + 1024 + 2 * lane);
      }
    }
#pragma unroll
    for (int a = 0; a < CT; ++a) {
      u32x4 z = {0u, 0u, 0u, 0u};
      uint32_t zs = 0u;
      if (av[a]) {
        z = *(const u32x4*)(aqp[a] + 64 * c);
        zs = *(const uint16_t*)(asp[a] + 8 * c);
      }
      an[slot][a] = z;
      asc[slot][a] = zs;
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < NC) load(d, d);

  for (int c0 = 0; c0 < NC; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = c0 + d;
      if (c >= NC) break;
      f16x8 bop[CT][4];
#pragma unroll
      for (int a = 0; a < CT; ++a) {
        const uint32_t s0 = e4m3_to_f16x2_scaled(asc[d][a] & 0xFFu);
        const uint32_t s1 = e4m3_to_f16x2_scaled(asc[d][a] >> 8);
        bop[a][0] = dequant8(an[d][a][0], s0);
        bop[a][1] = dequant8(an[d][a][1], s0);
        bop[a][2] = dequant8(an[d][a][2], s1);
        bop[a][3] = dequant8(an[d][a][3], s1);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s >= nsv) continue;
        const uint32_t w0 = e4m3_to_f16x2_scaled(ws[d][s] & 0xFFu);
        const uint32_t w1 = e4m3_to_f16x2_scaled(ws[d][s] >> 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 aop = dequant8(wn[d][s][j], j < 2 ? w0 : w1);
#pragma unroll
          for (int a = 0; a < CT; ++a)
            acc[s][a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[a][j], acc[s][a], 0, 0, 0);
        }
      }
      if (c + D < NC) load(c + D, d);
    }
  }

  // lane l holds out rows (16a + r) x weight rows 4 kq .. 4 kq + 3 of each tile
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s >= nsv) continue;
#pragma unroll
    for (int a = 0; a < CT; ++a) {
      if (!av[a]) continue;
      const int row = arow0 + 16 * a + r;
      *(f32x4*)(p.out + (size_t)row * p.N + col0 + 16 * s + 4 * kq) = acc[s][a];
    }
  }
}

template <int NS, int D, int CT>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs p) {
  extern __shared__ uint16_t s_act[];
  __shared__ int s_nact;
  const int nact = build_active_list(p, s_act, &s_nact);
  const int wave = threadIdx.x >> 6;
  const int tiles = p.N / 16;
  const int per_item = kGemmWaves * NS;
  const int items_per_e = (tiles + per_item - 1) / per_item;
  const int total = nact * items_per_e;
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int e = s_act[it / items_per_e];
    const int t0 = (it % items_per_e) * per_item + wave * NS;
    const int nsv = min(NS, tiles - t0);
    if (nsv <= 0) continue;
    const int r0 = p.off[e], G = p.off[e + 1] - r0;
    const uint8_t* wt = p.w + (size_t)e * expert_bytes + (size_t)t0 * tile_bytes;
    for (int b = 0; b < G; b += 16 * CT)
      mfma_pass<NS, D, CT>(p, wt, nsv, r0 + b, min(16 * CT, G - b), 16 * t0);
  }
}

// ------------------------------------------------------------------------- GEMV path
template <int NS, int D>
__device__ __forceinline__ void gemv_pass(const GemmArgs& p, const uint8_t* __restrict__ wt,
                                          int nsv, int arow0, int nrows, int col0) {
  constexpr int NR = kGemvRows;
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4;
  const int K = p.K, NC = K / 128;
  const size_t tstride = (size_t)NC * kChunkBytes;

  const uint8_t* aqp[NR];
  const uint8_t* asp[NR];
#pragma unroll
  for (int a = 0; a < NR; ++a) {
    const int row = arow0 + (a < nrows ? a : 0);
    aqp[a] = p.aq + (size_t)row * (K / 2) + 16 * kq;
    asp[a] = p.as + (size_t)row * (K / 16) + 2 * kq;
  }

  u32x4 wn[D][NS];
  uint32_t ws[D][NS];
  u32x4 an[D][NR];
  uint32_t asc[D][NR];
  float acc[NS][NR];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int a = 0; a < NR; ++a) acc[s][a] = 0.f;

  auto load = [&](int c, int slot) {
    const size_t off = (size_t)c * kChunkBytes;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s < nsv) {
        const uint8_t* t = wt + s * tstride + off;
        wn[slot][s] = *(const u32x4*)(t + 16 * lane);
        ws[slot][s] = *(const uint16_t*)(t + 1024 + 2 * lane);
      }
    }
#pragma unroll
    for (int a = 0; a < NR; ++a) {
      u32x4 z = {0u, 0u, 0u, 0u};
      uint32_t zs = 0u;
      if (a < nrows) {
        z = *(const u32x4*)(aqp[a] + 64 * c);
        zs = *(const uint16_t*)(asp[a] + 8 * c);
      }
      an[slot][a] = z;
      asc[slot][a] = zs;
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < NC) load(d, d);

  for (int c0 = 0; c0 < NC; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = c0 + d;
      if (c >= NC) break;
      // activation segments, exact f16 (codes times their block scales)
      f16x2 xa[NR][16];
#pragma unroll
      for (int a = 0; a < NR; ++a) {
        const uint32_t s0 = e4m3_to_f16x2_scaled(asc[d][a] & 0xFFu);
        const uint32_t s1 = e4m3_to_f16x2_scaled(asc[d][a] >> 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 v = dequant8(an[d][a][j], j < 2 ? s0 : s1);
#pragma unroll
          for (int m = 0; m < 4; ++m) xa[a][4 * j + m] = f16x2{v[2 * m], v[2 * m + 1]};
        }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s >= nsv) continue;
        const float sw0 = e4m3_to_f32(ws[d][s] & 0xFFu), sw1 = e4m3_to_f32(ws[d][s] >> 8);
        f16x2 wv[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) e2m1x8_to_f16(wn[d][s][j], &wv[4 * j]);
#pragma unroll
        for (int a = 0; a < NR; ++a) {
          if (a >= nrows) continue;
          float b0 = 0.f, b1 = 0.f;
#pragma unroll
          for (int m = 0; m < 8; ++m) b0 = __builtin_amdgcn_fdot2(wv[m], xa[a][m], b0, false);
#pragma unroll
          for (int m = 8; m < 16; ++m) b1 = __builtin_amdgcn_fdot2(wv[m], xa[a][m], b1, false);
          acc[s][a] = fmaf(sw0, b0, acc[s][a]);
          acc[s][a] = fmaf(sw1, b1, acc[s][a]);
        }
      }
      if (c + D < NC) load(c + D, d);
    }
  }

#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int a = 0; a < NR; ++a) {
      float v = acc[s][a];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (s < nsv && a < nrows && lane < 16)
        p.out[(size_t)(arow0 + a) * p.N + col0 + 16 * s + lane] = v;
    }
  }
}

template <int NS, int D>
__global__ __launch_bounds__(256) void k_gemm_gemv(GemmArgs p) {
  extern __shared__ uint16_t s_act[];
  __shared__ int s_nact;
  const int nact = build_active_list(p, s_act, &s_nact);
  const int wave = threadIdx.x >> 6;
  const int tiles = p.N / 16;
  const int per_item = kGemmWaves * NS;
  const int items_per_e = (tiles + per_item - 1) / per_item;
  const int total = nact * items_per_e;
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int e = s_act[it / items_per_e];
    const int t0 = (it % items_per_e) * per_item + wave * NS;
    const int nsv = min(NS, tiles - t0);
    if (nsv <= 0) continue;
    const int r0 = p.off[e], G = p.off[e + 1] - r0;
    const uint8_t* wt = p.w + (size_t)e * expert_bytes + (size_t)t0 * tile_bytes;
    for (int b = 0; b < G; b += kGemvRows)
      gemv_pass<NS, D>(p, wt, nsv, r0 + b, min(kGemvRows, G - b), 16 * t0);
  }
}

// ------------------------------------------------------------------------- launch
struct LaunchLimits {
  int occ = 0;  // workgroups per CU
  int cus = 0;
};

template <typename Kern>
static hipError_t limits_for(Kern kern, LaunchLimits* cache, std::mutex& mu, LaunchLimits* out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev].occ) {
    int o = 0, c = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, 256, 16384);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    cache[dev].occ = o > 0 ? o : 1;
    cache[dev].cus = c > 0 ? c : 1;
  }
  *out = cache[dev];
  return hipSuccess;
}

static int persistent_grid(const LaunchLimits& l, int per_item, const GemmArgs& a) {
  const long items_per_e = (a.N / 16 + per_item - 1) / per_item;
  const long max_items = items_per_e * a.E;
  const long slots = (long)l.occ * l.cus;
  return (int)(max_items < slots ? max_items : slots);
}

hipError_t launch_grouped_gemm(const uint8_t* aq, const uint8_t* as, const int32_t* off, int E,
                               int R, const uint8_t* w, int N, int K, float* out, int flags,
                               int gemv_max_rows, hipStream_t s) {
  (void)R;
  static std::mutex mu;
  static LaunchLimits mfma_cache[64], gemv_cache[64];
  const size_t lds = sizeof(uint16_t) * (size_t)E;
  const int big = 0x7FFFFFFF;
  // which groups each kernel owns
  int gemv_lo = 1, gemv_hi = 0, mfma_lo = 1;
  if (flags == MOE_PATH_FORCE_GEMV) {
    gemv_hi = big;
    mfma_lo = big;
  } else if (flags == MOE_PATH_AUTO) {
    gemv_hi = gemv_max_rows;
    mfma_lo = gemv_max_rows + 1;
  }
  if (gemv_hi >= gemv_lo) {
    GemmArgs a{aq, as, off, E, w, N, K, out, gemv_lo, gemv_hi};
    auto kern = k_gemm_gemv<MOE_GEMV_NS, MOE_GEMV_D>;
    LaunchLimits l;
    hipError_t err = limits_for(kern, gemv_cache, mu, &l);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(persistent_grid(l, kGemmWaves * MOE_GEMV_NS, a)), dim3(256), lds, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (mfma_lo < big) {
    GemmArgs a{aq, as, off, E, w, N, K, out, mfma_lo < 1 ? 1 : mfma_lo, big};
    auto kern = k_gemm_mfma<MOE_GEMM_NS, MOE_GEMM_D, MOE_GEMM_CT>;
    LaunchLimits l;
    hipError_t err = limits_for(kern, mfma_cache, mu, &l);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(persistent_grid(l, kGemmWaves * MOE_GEMM_NS, a)), dim3(256), lds, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
