// Row-wise kernels: NVFP4 quantization (optionally gathering its input rows), SwiGLU fused
// with the re-quantization, and the weighted scatter-add.
//
// Quantize / SwiGLU: one workgroup per row, one thread per 16-element scale block (two for
// rows longer than 4096), so the per-element work (a correctly rounded division and an
// e2m1 decision each) is spread over up to 256 threads and a row costs one pass.
#include "common.h"

namespace moe {

// ------------------------------------------------------------------------- quantize
// One workgroup per output row i; its input is row row_map[i] (row_map == nullptr: row i;
// a negative entry: an all-zero row).
template <int BPT>
__global__ __launch_bounds__(256) void k_quantize(const uint16_t* __restrict__ in,
                                                  const int32_t* __restrict__ row_map,
                                                  const int32_t* __restrict__ row_limit, int K,
                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                  float* __restrict__ row_gs) {
  __shared__ float s_red[4];
  const int row = blockIdx.x;
  int src = row_map ? row_map[row] : row;
  if (row_limit && row >= *row_limit) src = -1;
  const int NB = K / 16;
  float v[BPT][16];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int b = threadIdx.x + blockDim.x * k;
    u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
    if (b < NB && src >= 0) {
      const u32x4* p = (const u32x4*)(in + (size_t)src * K + 16 * b);
      w0 = p[0];
      w1 = p[1];
    }
    bf16x16_to_f32(w0, w1, v[k]);
  }
  const float amax = row_amax_threads<BPT>(v, threadIdx.x, blockDim.x, s_red);
  quantize_row_store<BPT>(v, NB, threadIdx.x, blockDim.x, amax, q + (size_t)row * (K / 2),
                          sc + (size_t)row * NB, row_gs + row);
}

hipError_t launch_quantize(const uint16_t* in, const int32_t* row_map, const int32_t* row_limit,
                           int R, int K, uint8_t* q, uint8_t* sc, float* row_gs, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int NB = K / 16, nt = row_threads(NB);
  if (NB <= 256)
    hipLaunchKernelGGL(k_quantize<1>, dim3(R), dim3(nt), 0, s, in, row_map, row_limit, K, q, sc,
                       row_gs);
  else
    hipLaunchKernelGGL(k_quantize<2>, dim3(R), dim3(nt), 0, s, in, row_map, row_limit, K, q, sc,
                       row_gs);
  return hipGetLastError();
}

// Expert of grouped row i (offsets ascending): largest e with off[e] <= i, or E when
// i >= off[E].
__device__ __forceinline__ int expert_of_row(const int32_t* off, int E, int i) {
  if (i >= off[E]) return E;
  int lo = 0, hi = E;  // off[lo] <= i < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------------------- SwiGLU
// One workgroup per row i of acc13 [R, 2I]: h = bf16(silu(zg) * zu) with the gate / up
// globals of the row's expert and the row's activation global.  Optionally writes h (bf16)
// and / or quantizes h in place of a separate nvfp4_quantize_rows pass (same arithmetic).
template <int BPT>
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ acc13, int I,
                                                const int32_t* __restrict__ offsets, int E,
                                                const float* __restrict__ g_gate,
                                                const float* __restrict__ g_up,
                                                const float* __restrict__ row_gs,
                                                const int32_t* __restrict__ gs_map,
                                                uint16_t* __restrict__ h, uint8_t* __restrict__ q,
                                                uint8_t* __restrict__ sc, float* __restrict__ h_gs) {
  __shared__ float s_red[4];
  const int row = blockIdx.x;
  const int e = expert_of_row(offsets, E, row);  // uniform: scalar loads
  const int NB = I / 16;
  float v[BPT][16];
  float cg = 0.0f, cu = 0.0f;
  if (e < E) {
    const float gs = row_gs[gs_map ? gs_map[row] : row];
    cg = gs * g_gate[e];
    cu = gs * g_up[e];
  }
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int b = threadIdx.x + blockDim.x * k;
#pragma unroll
    for (int x = 0; x < 16; ++x) v[k][x] = 0.0f;
    if (b >= NB || e >= E) continue;
    const f32x4* pg = (const f32x4*)(acc13 + (size_t)row * 2 * I + 16 * b);
    const f32x4* pu = (const f32x4*)(acc13 + (size_t)row * 2 * I + I + 16 * b);
    f32x4 ag[4], au[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ag[c] = pg[c];
      au[c] = pu[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        v[k][4 * c + x] = __uint_as_float(swiglu_bf16(cg, ag[c][x], cu, au[c][x]) << 16);
      }
    }
  }
  if (h) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int b = threadIdx.x + blockDim.x * k;
      if (b >= NB) continue;
      u32x4 w[2];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t lo = __float_as_uint(v[k][2 * x]) >> 16;
        const uint32_t hi = __float_as_uint(v[k][2 * x + 1]) & 0xFFFF0000u;
        w[x >> 2][x & 3] = lo | hi;
      }
      u32x4* p = (u32x4*)(h + (size_t)row * I + 16 * b);
      p[0] = w[0];
      p[1] = w[1];
    }
  }
  if (q) {
    const float amax = row_amax_threads<BPT>(v, threadIdx.x, blockDim.x, s_red);
    quantize_row_store<BPT>(v, NB, threadIdx.x, blockDim.x, amax, q + (size_t)row * (I / 2),
                            sc + (size_t)row * NB, h_gs + row);
  }
}

hipError_t launch_swiglu(const float* acc13, int R, int I, const int32_t* offsets, int E,
                         const float* g_gate, const float* g_up, const float* row_gs,
                         const int32_t* gs_map, uint16_t* h, uint8_t* q, uint8_t* sc, float* h_gs,
                         hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int NB = I / 16, nt = row_threads(NB);
  if (NB <= 256)
    hipLaunchKernelGGL(k_swiglu<1>, dim3(R), dim3(nt), 0, s, acc13, I, offsets, E, g_gate, g_up,
                       row_gs, gs_map, h, q, sc, h_gs);
  else
    hipLaunchKernelGGL(k_swiglu<2>, dim3(R), dim3(nt), 0, s, acc13, I, offsets, E, g_gate, g_up,
                       row_gs, gs_map, h, q, sc, h_gs);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- scatter
// Grid (T, ceil(H / 256)), 8 waves per workgroup, 4 columns per lane.  Wave w sums the
// token's rows p = tok_off[t] + w, + 8, ... in ascending order, each scaled by
// row_w * g_down * row_gs (the coefficients of up to 64 rows are computed by the lanes in
// parallel); the eight partial rows are then added in wave order.  The summation order
// depends only on the token's row count, so a token's output does not depend on the
// other tokens of the batch.
constexpr int kScatterWaves = 8;

__global__ __launch_bounds__(64 * kScatterWaves) void k_scatter(
    const float* __restrict__ y, int H, const int32_t* __restrict__ offsets, int E,
    const float* __restrict__ row_w, const float* __restrict__ g_down,
    const float* __restrict__ row_gs, const int32_t* __restrict__ tok_off,
    const int32_t* __restrict__ tok_rows, uint16_t* __restrict__ out) {
  __shared__ f32x4 s_part[kScatterWaves][64];
  extern __shared__ int32_t s_off[];  // expert offsets, for the row -> expert searches
  for (int k = threadIdx.x; k <= E; k += blockDim.x) s_off[k] = offsets[k];
  __syncthreads();
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.y * 256 + 4 * lane;
  const bool cv = col < H;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int p0 = tok_off[t], p1 = tok_off[t + 1];
  for (int base = p0 + wave; base < p1; base += 64 * kScatterWaves) {
    // rows base + 8k, k < 64: coefficients in parallel
    const int p = base + kScatterWaves * lane;
    int i = 0;
    float c = 0.0f;
    if (p < p1) {
      i = tok_rows[p];
      const int e = expert_of_row(s_off, E, i);
      c = (e < E) ? row_w[i] * g_down[e] * row_gs[i] : 0.0f;
    }
    const int n = min(64, (p1 - base + kScatterWaves - 1) / kScatterWaves);
#pragma unroll 4
    for (int k = 0; k < n; ++k) {
      const int ik = __shfl(i, k, 64);
      const float ck = __shfl(c, k, 64);
      if (cv) {
        const f32x4 yv = *(const f32x4*)(y + (size_t)ik * H + col);
        acc[0] = fmaf(ck, yv[0], acc[0]);
        acc[1] = fmaf(ck, yv[1], acc[1]);
        acc[2] = fmaf(ck, yv[2], acc[2]);
        acc[3] = fmaf(ck, yv[3], acc[3]);
      }
    }
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && cv) {
    f32x4 sum = s_part[0][lane];
#pragma unroll
    for (int w = 1; w < kScatterWaves; ++w) {
      const f32x4 o = s_part[w][lane];
      sum[0] += o[0];
      sum[1] += o[1];
      sum[2] += o[2];
      sum[3] += o[3];
    }
    u32x2 ov;
    ov[0] = f32_to_bf16_rne(sum[0]) | (f32_to_bf16_rne(sum[1]) << 16);
    ov[1] = f32_to_bf16_rne(sum[2]) | (f32_to_bf16_rne(sum[3]) << 16);
    *(u32x2*)(out + (size_t)t * H + col) = ov;
  }
}

hipError_t launch_scatter(const float* y, int R, int H, const int32_t* offsets, int E,
                          const float* row_w, const float* g_down, const float* row_gs,
                          const int32_t* tok_off, const int32_t* tok_rows, int T, uint16_t* out,
                          hipStream_t s) {
  (void)R;
  if (T == 0) return hipSuccess;
  const dim3 grid(T, (H + 255) / 256), block(64 * kScatterWaves);
  hipLaunchKernelGGL(k_scatter, grid, block, sizeof(int32_t) * (size_t)(E + 1), s, y, H, offsets, E,
                     row_w, g_down, row_gs, tok_off, tok_rows, out);
  return hipGetLastError();
}

}  // namespace moe
