// Row-wise kernels: NVFP4 quantization (optionally gathering its input rows), SwiGLU fused
// with the re-quantization, and the weighted scatter-add.
//
// Quantize / SwiGLU: one workgroup per row, one thread per 16-element scale block (two for
// rows longer than 4096), so the per-element work (a correctly rounded division and an
// e2m1 decision each) is spread over up to 256 threads and a row costs one pass.
#include "common.h"

namespace moe {

// ------------------------------------------------------------------------- quantize
// nt threads per row (a multiple of 64), blockDim.x / nt rows per workgroup: output row i
// (i < R) quantizes input row row_map[i] (row_map == nullptr: row i; a negative entry: an
// all-zero row); rows at or past *row_limit are all-zero rows.  Without a row map the row
// is loaded before the limit is known (it is in bounds either way), so the two loads
// overlap.  Every thread joins the row-max barrier; only real rows store.
template <int BPT>
__global__ __launch_bounds__(256) void k_quantize(const uint16_t* __restrict__ in,
                                                  const int32_t* __restrict__ row_map,
                                                  const int32_t* __restrict__ row_limit, int R,
                                                  int K, int nt, uint8_t* __restrict__ q,
                                                  uint8_t* __restrict__ sc,
                                                  float* __restrict__ row_gs) {
  __shared__ float s_red[4];
  const int slot = threadIdx.x / nt, t = threadIdx.x - slot * nt;
  const int row = blockIdx.x * (blockDim.x / nt) + slot;
  const bool real = row < R;
  const int src = !real ? -1 : row_map ? row_map[row] : row;
  const bool live = real && (!row_limit || row < *row_limit);
  const int NB = K / 16;
  float v[BPT][16];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int b = t + nt * k;
    u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
    if (b < NB && src >= 0) {
      const u32x4* p = (const u32x4*)(in + (size_t)src * K + 16 * b);
      w0 = p[0];
      w1 = p[1];
    }
    if (!live) w0 = w1 = u32x4{0u, 0u, 0u, 0u};
    bf16x16_to_f32(w0, w1, v[k]);
  }
  const float amax = row_amax_threads<BPT>(v, t, nt, s_red + slot * (nt / 64));
  if (real)
    quantize_row_store<BPT>(v, NB, t, nt, amax, q + (size_t)row * (K / 2),
                            sc + (size_t)row * NB, row_gs + row);
}

hipError_t launch_quantize(const uint16_t* in, const int32_t* row_map, const int32_t* row_limit,
                           int R, int K, uint8_t* q, uint8_t* sc, float* row_gs, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int NB = K / 16;
  const int nt = row_threads(NB);
  if (NB <= 256)
    hipLaunchKernelGGL(k_quantize<1>, dim3(R), dim3(nt), 0, s, in, row_map, row_limit, R, K, nt, q,
                       sc, row_gs);
  else
    hipLaunchKernelGGL(k_quantize<2>, dim3(R), dim3(nt), 0, s, in, row_map, row_limit, R, K, nt, q,
                       sc, row_gs);
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
// Summation order of a token (both scatter kernels below, so the layer's fused path and
// moe_scatter_add give the same bits): the token's rows p = tok_off[t] .. tok_off[t+1] - 1
// are summed as 8 interleaved partial sums, partial j taking p - tok_off[t] = j, j + 8,
// ... in ascending p, each term the fp32 product c_i * y[i] (c_i = row_w[i] * g_down[e] *
// row_gs[i], rounded, no fused multiply-add); the partials are then added in order 0..7.
// The order depends only on the token's own row count, so a token's output does not depend
// on the other tokens of the batch.
constexpr int kSumParts = 8;


// Grid (T, ceil(H / 256)), 8 waves per workgroup (wave w = partial w), 4 columns per lane;
// the coefficients of up to 64 rows are computed by the lanes in parallel.
__global__ __launch_bounds__(64 * kSumParts) void k_scatter(
    const float* __restrict__ y, int H, const int32_t* __restrict__ offsets, int E,
    const float* __restrict__ row_w, const float* __restrict__ g_down,
    const float* __restrict__ row_gs, const int32_t* __restrict__ tok_off,
    const int32_t* __restrict__ tok_rows, uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
  __shared__ f32x4 s_part[kSumParts][64];
  extern __shared__ int32_t s_off[];  // expert offsets, for the row -> expert searches
  for (int k = threadIdx.x; k <= E; k += blockDim.x) s_off[k] = offsets[k];
  __syncthreads();
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.y * 256 + 4 * lane;
  const bool cv = col < H;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int p0 = tok_off[t], p1 = tok_off[t + 1];
  for (int base = p0 + wave; base < p1; base += 64 * kSumParts) {
    // rows base + 8k, k < 64: coefficients in parallel
    const int p = base + kSumParts * lane;
    int i = 0;
    float c = 0.0f;
    if (p < p1) {
      i = tok_rows[p];
      const int e = expert_of_row(s_off, E, i);
      c = (e < E) ? row_w[i] * g_down[e] * row_gs[i] : 0.0f;
    }
    const int n = min(64, (p1 - base + kSumParts - 1) / kSumParts);
#pragma unroll 4
    for (int k = 0; k < n; ++k) {
      const int ik = __shfl(i, k, 64);
      const float ck = __shfl(c, k, 64);
      if (cv) {
        const f32x4 yv = *(const f32x4*)(y + (size_t)ik * H + col);
        acc[0] += ck * yv[0];
        acc[1] += ck * yv[1];
        acc[2] += ck * yv[2];
        acc[3] += ck * yv[3];
      }
    }
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && cv) {
    f32x4 sum = s_part[0][lane];
#pragma unroll
    for (int w = 1; w < kSumParts; ++w) {
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
  const dim3 grid(T, (H + 255) / 256), block(64 * kSumParts);
  hipLaunchKernelGGL(k_scatter, grid, block, sizeof(int32_t) * (size_t)(E + 1), s, y, H, offsets, E,
                     row_w, g_down, row_gs, tok_off, tok_rows, out);
  return hipGetLastError();
}

// The layer's scatter once the terms are computed: yc[i] = c_i * y[i] for grouped row i
// (written so by the w2 GEMM's epilogue, in grouped order: scattering them into token order
// there measured slower than this gather), so token t sums rows yc[tok_rows[p]],
// p = tok_off[t] .. tok_off[t+1] - 1, in the order above.
// WIDE (tokens of many rows): the k_scatter shape, wave w = partial w, 4 columns per lane.
// !WIDE (tokens of few rows): each wave owns 256 columns of the token and keeps the 8
// partials in registers, four waves per workgroup over 1024 columns, so a workgroup is not
// mostly idle waves and every lane has up to 8 independent loads in flight.
template <bool WIDE>
__global__ __launch_bounds__(256 * (WIDE ? 2 : 1)) void k_token_sum(
    const float* __restrict__ yc, int H, const int32_t* __restrict__ tok_off,
    const int32_t* __restrict__ tok_rows, uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p0 = tok_off[t], p1 = tok_off[t + 1];
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  int col;
  if constexpr (WIDE) {
    __shared__ f32x4 s_part[kSumParts][64];
    col = blockIdx.y * 256 + 4 * lane;
    const bool cv = col < H;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = p0 + wave; base < p1; base += 64 * kSumParts) {
      // rows base + 8k, k < 64: their indices in parallel
      const int p = base + kSumParts * lane;
      const int i = p < p1 ? tok_rows[p] : 0;
      const int n = min(64, (p1 - base + kSumParts - 1) / kSumParts);
      // up to 16 rows' loads in flight before the first add (same order of the adds)
      for (int k0 = 0; k0 < n; k0 += 16) {
        f32x4 v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int ik = __builtin_amdgcn_readlane(i, (k0 + k) & 63);
          if (k0 + k < n && cv) v[k] = *(const f32x4*)(yc + (size_t)ik * H + col);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          if (k0 + k < n && cv) {
            acc[0] += v[k][0];
            acc[1] += v[k][1];
            acc[2] += v[k][2];
            acc[3] += v[k][3];
          }
        }
      }
    }
    s_part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0 || !cv) return;
    sum = s_part[0][lane];
#pragma unroll
    for (int w = 1; w < kSumParts; ++w) {
      const f32x4 o = s_part[w][lane];
      sum[0] += o[0];
      sum[1] += o[1];
      sum[2] += o[2];
      sum[3] += o[3];
    }
  } else {
    col = blockIdx.y * 1024 + wave * 256 + 4 * lane;
    if (col >= H) return;  // no barrier in this shape
    f32x4 part[kSumParts];
#pragma unroll
    for (int j = 0; j < kSumParts; ++j) part[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int base = p0; base < p1; base += kSumParts) {
      int i[kSumParts];
#pragma unroll
      for (int j = 0; j < kSumParts; ++j) i[j] = base + j < p1 ? tok_rows[base + j] : 0;
      f32x4 v[kSumParts];
#pragma unroll
      for (int j = 0; j < kSumParts; ++j)
        if (base + j < p1) v[j] = *(const f32x4*)(yc + (size_t)i[j] * H + col);
#pragma unroll
      for (int j = 0; j < kSumParts; ++j) {
        if (base + j < p1) {
          part[j][0] += v[j][0];
          part[j][1] += v[j][1];
          part[j][2] += v[j][2];
          part[j][3] += v[j][3];
        }
      }
    }
    sum = part[0];
#pragma unroll
    for (int j = 1; j < kSumParts; ++j) {
      sum[0] += part[j][0];
      sum[1] += part[j][1];
      sum[2] += part[j][2];
      sum[3] += part[j][3];
    }
  }
  u32x2 ov;
  ov[0] = f32_to_bf16_rne(sum[0]) | (f32_to_bf16_rne(sum[1]) << 16);
  ov[1] = f32_to_bf16_rne(sum[2]) | (f32_to_bf16_rne(sum[3]) << 16);
  *(u32x2*)(out + (size_t)t * H + col) = ov;
}

hipError_t launch_token_sum(const float* yc, int R, int H, const int32_t* tok_off,
                            const int32_t* tok_rows, int T, uint16_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (R >= 16 * T) {  // many rows per token on average: split a token's rows over 8 waves
    hipLaunchKernelGGL(k_token_sum<true>, dim3(T, (H + 255) / 256), dim3(64 * kSumParts), 0, s, yc,
                       H, tok_off, tok_rows, out);
  } else {
    hipLaunchKernelGGL(k_token_sum<false>, dim3(T, (H + 1023) / 1024), dim3(256), 0, s, yc, H,
                       tok_off, tok_rows, out);
  }
  return hipGetLastError();
}

}  // namespace moe
