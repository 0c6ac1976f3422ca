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
#define MOE_GEMM_NS 2  // 16-row tiles per wave, MFMA kernel
#endif
#ifndef MOE_GEMM_D
#define MOE_GEMM_D 4   // chunks in flight per wave, MFMA kernel
#endif
#ifndef MOE_GEMM_CT
#define MOE_GEMM_CT 1  // 16-row activation column tiles per MFMA pass
#endif
#ifndef MOE_GEMV_NS
#define MOE_GEMV_NS 2  // 16-row tiles per wave, GEMV kernel
#endif
#ifndef MOE_GEMV_D
#define MOE_GEMV_D 2
#endif
#ifndef MOE_GEMM_WGS_PER_CU
#define MOE_GEMM_WGS_PER_CU 0  // 0: one work item per workgroup; n > 0: persistent, n per CU
#endif

namespace moe {

constexpr int kGemmWaves = 4;
constexpr int kGemvRows = 4;

struct GemmArgs {
  const uint8_t* aq;     // activation rows [A, K/2] (A = a_rows)
  const uint8_t* as;     // their scales [A, K/16]
  const int32_t* amap;   // grouped row i reads activation row amap[i]; nullptr: row i
  int a_rows;
  const int32_t* off;
  int E;
  const uint8_t* w;
  int N, K;
  float* out;
  int gmin, gmax;  // this kernel's groups: gmin <= G <= gmax
};

// Activation row of grouped row i (i < rows of the pass); -1 when the lane has no row.
__device__ __forceinline__ int act_row(const GemmArgs& p, int i, bool valid) {
  if (!valid) return -1;
  return p.amap ? p.amap[i] : i;
}

// Ids of the experts whose group size is in [gmin, gmax], ascending, into LDS (wave 0).
__device__ __forceinline__ int build_active_list(const GemmArgs& p, uint16_t* s_act, int* s_nact) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int n = 0;
    for (int base = 0; base < p.E; base += 256) {
      int g[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // four independent loads in flight
        const int e = base + 64 * u + lane;
        g[u] = e < p.E ? p.off[e + 1] - p.off[e] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = base + 64 * u + lane;
        const bool a = e < p.E && g[u] >= p.gmin && g[u] <= p.gmax;
        const uint64_t m = __ballot(a);
        if (a) s_act[n + __popcll(m & below)] = (uint16_t)e;
        n += __popcll(m);
      }
    }
    if (lane == 0) *s_nact = n;
  }
  __syncthreads();
  return *s_nact;
}

// Buffer resource over [base, base + bytes): loads at offsets beyond the range return 0,
// which zero-fills the activation rows a pass does not own without any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

#ifndef MOE_W_CPOL
#define MOE_W_CPOL 2  // cache policy of the weight-stream loads: non-temporal (read once)
#endif

// ------------------------------------------------------------------------- MFMA path
// One pass over K for NS weight tiles (wt: first tile, uniform) and CT activation column
// tiles (rows arow0 .. arow0 + nrows - 1).  NC % D == 0.
template <int NS, int D, int CT>
__device__ __forceinline__ void mfma_pass(const GemmArgs& p, const uint8_t* __restrict__ wt,
                                          int nsv, int arow0, int nrows, int col0) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, r = lane & 15;
  const int K = p.K, NC = K / 128;
  const int tstride = NC * kChunkBytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt, nsv * tstride);
  const int abytes = p.a_rows * (K / 2), sbytes = p.a_rows * (K / 16);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.aq, abytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.as, sbytes);
  const int vw = 16 * lane, vws = 1024 + 2 * lane;
  int va[CT], vs[CT];  // lanes without a row point past the end: their loads return 0
#pragma unroll
  for (int a = 0; a < CT; ++a) {
    const int row = act_row(p, arow0 + 16 * a + r, 16 * a + r < nrows);
    va[a] = row >= 0 ? row * (K / 2) + 16 * kq : abytes;
    vs[a] = row >= 0 ? row * (K / 16) + 2 * kq : sbytes;
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
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int so = s * tstride + c * kChunkBytes;
      wn[slot][s] = __builtin_amdgcn_raw_buffer_load_b128(wr, vw, so, MOE_W_CPOL);
      ws[slot][s] = __builtin_amdgcn_raw_buffer_load_b16(wr, vws, so, MOE_W_CPOL);
    }
#pragma unroll
    for (int a = 0; a < CT; ++a) {
      an[slot][a] = __builtin_amdgcn_raw_buffer_load_b128(ar, va[a], 64 * c, 0);
      asc[slot][a] = __builtin_amdgcn_raw_buffer_load_b16(sr, vs[a], 8 * c, 0);
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);

  for (int c0 = 0; c0 < NC; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
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
      if (c0 + d + D < NC) load(c0 + d + D, d);
    }
  }

  // lane l holds out rows (16a + r) x weight rows 4 kq .. 4 kq + 3 of each tile
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s >= nsv) break;
#pragma unroll
    for (int a = 0; a < CT; ++a) {
      if (16 * a + r < nrows) {
        const int row = arow0 + 16 * a + r;
        *(f32x4*)(p.out + (size_t)row * p.N + col0 + 16 * s + 4 * kq) = acc[s][a];
      }
    }
  }
}

// Item loop shared by both kernels: item -> (expert, first tile of this wave).
struct ItemLoop {
  int nact, items_per_e, total, tiles, per_item;
};

__device__ __forceinline__ ItemLoop item_loop(const GemmArgs& p, int nact, int NS) {
  ItemLoop L;
  L.nact = nact;
  L.tiles = p.N / 16;
  L.per_item = kGemmWaves * NS;
  L.items_per_e = (L.tiles + L.per_item - 1) / L.per_item;
  L.total = nact * L.items_per_e;
  return L;
}

template <int NS, int D, int CT>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs p) {
  extern __shared__ uint16_t s_act[];
  __shared__ int s_nact;
  const int nact = build_active_list(p, s_act, &s_nact);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const ItemLoop L = item_loop(p, nact, NS);
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  for (int it = blockIdx.x; it < L.total; it += gridDim.x) {
    const int e = __builtin_amdgcn_readfirstlane(s_act[it / L.items_per_e]);
    const int t0 = (it % L.items_per_e) * L.per_item + wave * NS;
    const int nsv = min(NS, L.tiles - t0);
    if (nsv <= 0) continue;
    const int r0 = __builtin_amdgcn_readfirstlane(p.off[e]);
    const int G = __builtin_amdgcn_readfirstlane(p.off[e + 1]) - r0;
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
  const int tstride = NC * kChunkBytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt, nsv * tstride);
  const int abytes = p.a_rows * (K / 2), sbytes = p.a_rows * (K / 16);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.aq, abytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.as, sbytes);
  const int vw = 16 * lane, vws = 1024 + 2 * lane;
  int va[NR], vs[NR];
#pragma unroll
  for (int a = 0; a < NR; ++a) {
    const int row = act_row(p, arow0 + a, a < nrows);
    va[a] = row >= 0 ? row * (K / 2) + 16 * kq : abytes;
    vs[a] = row >= 0 ? row * (K / 16) + 2 * kq : sbytes;
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
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int so = s * tstride + c * kChunkBytes;
      wn[slot][s] = __builtin_amdgcn_raw_buffer_load_b128(wr, vw, so, MOE_W_CPOL);
      ws[slot][s] = __builtin_amdgcn_raw_buffer_load_b16(wr, vws, so, MOE_W_CPOL);
    }
#pragma unroll
    for (int a = 0; a < NR; ++a) {
      an[slot][a] = __builtin_amdgcn_raw_buffer_load_b128(ar, va[a], 64 * c, 0);
      asc[slot][a] = __builtin_amdgcn_raw_buffer_load_b16(sr, vs[a], 8 * c, 0);
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);

  for (int c0 = 0; c0 < NC; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float sw0 = e4m3_to_f32(ws[d][s] & 0xFFu), sw1 = e4m3_to_f32(ws[d][s] >> 8);
        f16x2 wv[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) e2m1x8_to_f16(wn[d][s][j], &wv[4 * j]);
#pragma unroll
        for (int a = 0; a < NR; ++a) {
          if (a >= nrows) break;  // uniform
          const uint32_t s0 = e4m3_to_f16x2_scaled(asc[d][a] & 0xFFu);
          const uint32_t s1 = e4m3_to_f16x2_scaled(asc[d][a] >> 8);
          float b0 = 0.f, b1 = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f16x8 v = dequant8(an[d][a][j], j < 2 ? s0 : s1);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const f16x2 x2 = f16x2{v[2 * m], v[2 * m + 1]};
              if (j < 2) b0 = __builtin_amdgcn_fdot2(wv[4 * j + m], x2, b0, false);
              else b1 = __builtin_amdgcn_fdot2(wv[4 * j + m], x2, b1, false);
            }
          }
          acc[s][a] = fmaf(sw0, b0, acc[s][a]);
          acc[s][a] = fmaf(sw1, b1, acc[s][a]);
        }
      }
      if (c0 + d + D < NC) load(c0 + d + D, d);
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const ItemLoop L = item_loop(p, nact, NS);
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  for (int it = blockIdx.x; it < L.total; it += gridDim.x) {
    const int e = __builtin_amdgcn_readfirstlane(s_act[it / L.items_per_e]);
    const int t0 = (it % L.items_per_e) * L.per_item + wave * NS;
    const int nsv = min(NS, L.tiles - t0);
    if (nsv <= 0) continue;
    const int r0 = __builtin_amdgcn_readfirstlane(p.off[e]);
    const int G = __builtin_amdgcn_readfirstlane(p.off[e + 1]) - r0;
    const uint8_t* wt = p.w + (size_t)e * expert_bytes + (size_t)t0 * tile_bytes;
    for (int b = 0; b < G; b += kGemvRows)
      gemv_pass<NS, D>(p, wt, nsv, r0 + b, min(kGemvRows, G - b), 16 * t0);
  }
}

// ------------------------------------------------------------------------- launch
static hipError_t cu_count(int* cus) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    int c = 0;
    err = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    cache[dev] = c > 0 ? c : 1;
  }
  *cus = cache[dev];
  return hipSuccess;
}

// Workgroups to launch: every possible item (inactive ones exit after the prologue), or a
// persistent grid of MOE_GEMM_WGS_PER_CU workgroups per CU.
static int gemm_grid(int per_item, const GemmArgs& a, int cus) {
  const long items_per_e = (a.N / 16 + per_item - 1) / per_item;
  const long max_items = items_per_e * a.E;
  if (MOE_GEMM_WGS_PER_CU <= 0) return (int)max_items;
  const long slots = (long)MOE_GEMM_WGS_PER_CU * cus;
  return (int)(max_items < slots ? max_items : slots);
}

// Ring depth: the configured depth, reduced until it divides the chunk count K / 128.
static int ring_depth(int K, int dmax) {
  const int nc = K / 128;
  int d = dmax;
  while (d > 1 && nc % d) d >>= 1;
  return d;
}

template <int D>
static void launch_mfma_d(const GemmArgs& a, int cus, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_mfma<MOE_GEMM_NS, D, MOE_GEMM_CT>),
                     dim3(gemm_grid(kGemmWaves * MOE_GEMM_NS, a, cus)), dim3(256), lds, s, a);
}

template <int D>
static void launch_gemv_d(const GemmArgs& a, int cus, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_gemv<MOE_GEMV_NS, D>),
                     dim3(gemm_grid(kGemmWaves * MOE_GEMV_NS, a, cus)), dim3(256), lds, s, a);
}

hipError_t launch_grouped_gemm(const uint8_t* aq, const uint8_t* as, const int32_t* amap,
                               int a_rows, const int32_t* off, int E, const uint8_t* w, int N, int K,
                               float* out, int flags, int gemv_max_rows, hipStream_t s) {
  int cus = 0;
  hipError_t err = cu_count(&cus);
  if (err != hipSuccess) return err;
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
    const GemmArgs a{aq, as, amap, a_rows, off, E, w, N, K, out, gemv_lo, gemv_hi};
    switch (ring_depth(K, MOE_GEMV_D)) {
      case 1: launch_gemv_d<1>(a, cus, lds, s); break;
      case 2: launch_gemv_d<2>(a, cus, lds, s); break;
      default: launch_gemv_d<(MOE_GEMV_D >= 4 ? 4 : MOE_GEMV_D)>(a, cus, lds, s); break;
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (mfma_lo < big) {
    const GemmArgs a{aq, as, amap, a_rows, off, E, w, N, K, out, mfma_lo < 1 ? 1 : mfma_lo, big};
    switch (ring_depth(K, MOE_GEMM_D)) {
      case 1: launch_mfma_d<1>(a, cus, lds, s); break;
      case 2: launch_mfma_d<2>(a, cus, lds, s); break;
      default: launch_mfma_d<(MOE_GEMM_D >= 4 ? 4 : MOE_GEMM_D)>(a, cus, lds, s); break;
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
