// Row-wise kernels: NVFP4 quantization (optionally gathering its input rows), SwiGLU fused
// with the re-quantization, and the weighted scatter-add.  One wavefront owns one row, so
// every row reduction (amax, sums) stays inside a wave and its order is fixed.
#include "common.h"

namespace moe {

// Largest power-of-two blocks-per-lane a row kernel keeps in registers (16 values each).
constexpr int kMaxBPL = 8;  // rows of up to 64 * 8 * 16 = 8192 elements

__device__ __forceinline__ float wave_max(float v) {
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

// Quantize one row held in registers: lane owns blocks b = lane + 64k (k < BPL, b < NB),
// v[k][0..15] the block's values.  Follows nvfp4_quantize_rows' definition exactly
// (float32, correctly rounded divisions, no contraction).
template <int BPL>
__device__ __forceinline__ void quantize_row_regs(const float (&v)[BPL][16], int NB, int lane,
                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                  float* __restrict__ gs_out) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < BPL; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, __builtin_fabsf(v[k][e]));
  amax = wave_max(amax);
  const float gs = amax > 0.0f ? amax / 2688.0f : 1.0f;
  const float t = 6.0f * gs;
#pragma unroll
  for (int k = 0; k < BPL; ++k) {
    const int b = lane + 64 * k;
    if (b >= NB) continue;
    float bmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, __builtin_fabsf(v[k][e]));
    const float sf = bmax / t;
    const uint32_t sb = e4m3_encode_pos(sf);
    const float d = e4m3_to_f32(sb) * gs;
    uint32_t lo = 0, hi = 0;
    if (d != 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lo |= e2m1_encode(v[k][e] / d) << (4 * e);
#pragma unroll
      for (int e = 0; e < 8; ++e) hi |= e2m1_encode(v[k][8 + e] / d) << (4 * e);
    }
    u32x2 pk = {lo, hi};
    *(u32x2*)(q + 8 * (size_t)b) = pk;
    sc[b] = (uint8_t)sb;
  }
  if (lane == 0) *gs_out = gs;
}

// ------------------------------------------------------------------------- quantize
// One wave per output row i; its input is row row_map[i] (row_map == nullptr: row i;
// a negative entry: an all-zero row).
template <int BPL>
__global__ __launch_bounds__(256) void k_quantize(const uint16_t* __restrict__ in,
                                                  const int32_t* __restrict__ row_map, int R, int K,
                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                  float* __restrict__ row_gs) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const int src = row_map ? row_map[row] : row;
  const int NB = K / 16;
  float v[BPL][16];
#pragma unroll
  for (int k = 0; k < BPL; ++k) {
    const int b = lane + 64 * k;
    u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
    if (b < NB && src >= 0) {
      const u32x4* p = (const u32x4*)(in + (size_t)src * K + 16 * b);
      w0 = p[0];
      w1 = p[1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[k][2 * e] = __uint_as_float(w0[e] << 16);
      v[k][2 * e + 1] = __uint_as_float(w0[e] & 0xFFFF0000u);
      v[k][8 + 2 * e] = __uint_as_float(w1[e] << 16);
      v[k][8 + 2 * e + 1] = __uint_as_float(w1[e] & 0xFFFF0000u);
    }
  }
  quantize_row_regs<BPL>(v, NB, lane, q + (size_t)row * (K / 2), sc + (size_t)row * NB,
                         row_gs + row);
}

static int bpl_for(int NB) {
  const int need = (NB + 63) / 64;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
}

hipError_t launch_quantize(const uint16_t* in, const int32_t* row_map, int R, int K, uint8_t* q,
                           uint8_t* sc, float* row_gs, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const dim3 grid((R + 3) / 4), block(256);
  switch (bpl_for(K / 16)) {
    case 1: hipLaunchKernelGGL(k_quantize<1>, grid, block, 0, s, in, row_map, R, K, q, sc, row_gs); break;
    case 2: hipLaunchKernelGGL(k_quantize<2>, grid, block, 0, s, in, row_map, R, K, q, sc, row_gs); break;
    case 4: hipLaunchKernelGGL(k_quantize<4>, grid, block, 0, s, in, row_map, R, K, q, sc, row_gs); break;
    default: hipLaunchKernelGGL(k_quantize<8>, grid, block, 0, s, in, row_map, R, K, q, sc, row_gs); break;
  }
  return hipGetLastError();
}

// Expert of grouped row i (offsets in LDS, ascending): largest e with off[e] <= i, or E
// when i >= off[E].
__device__ __forceinline__ int expert_of_row(const int* off, int E, int i) {
  if (i >= off[E]) return E;
  int lo = 0, hi = E;  // off[lo] <= i < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------------------- SwiGLU
// One wave per row i of acc13 [R, 2I]: h = bf16(silu(zg) * zu) with the gate / up globals
// of the row's expert and the row's activation global.  Optionally writes h (bf16) and /
// or quantizes h in place of a separate nvfp4_quantize_rows pass (same arithmetic).
template <int BPL>
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ acc13, int R, int I,
                                                const int32_t* __restrict__ offsets, int E,
                                                const float* __restrict__ g_gate,
                                                const float* __restrict__ g_up,
                                                const float* __restrict__ row_gs,
                                                uint16_t* __restrict__ h, uint8_t* __restrict__ q,
                                                uint8_t* __restrict__ sc, float* __restrict__ h_gs) {
  extern __shared__ int s_off[];
  for (int k = threadIdx.x; k <= E; k += blockDim.x) s_off[k] = offsets[k];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const int e = expert_of_row(s_off, E, row);
  const int NB = I / 16;
  float v[BPL][16];
  float cg = 0.0f, cu = 0.0f;
  if (e < E) {
    const float gs = row_gs[row];
    cg = gs * g_gate[e];
    cu = gs * g_up[e];
  }
#pragma unroll
  for (int k = 0; k < BPL; ++k) {
    const int b = lane + 64 * k;
#pragma unroll
    for (int x = 0; x < 16; ++x) v[k][x] = 0.0f;
    if (b >= NB || e >= E) continue;
    const f32x4* pg = (const f32x4*)(acc13 + (size_t)row * 2 * I + 16 * b);
    const f32x4* pu = (const f32x4*)(acc13 + (size_t)row * 2 * I + I + 16 * b);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 ag = pg[c], au = pu[c];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float zg = cg * ag[x], zu = cu * au[x];
        const float silu = zg / (1.0f + expf(-zg));
        v[k][4 * c + x] = __uint_as_float(f32_to_bf16_rne(silu * zu) << 16);  // bf16 value
      }
    }
  }
  if (h) {
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      const int b = lane + 64 * k;
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
  if (q) quantize_row_regs<BPL>(v, NB, lane, q + (size_t)row * (I / 2), sc + (size_t)row * NB,
                                h_gs + row);
}

hipError_t launch_swiglu(const float* acc13, int R, int I, const int32_t* offsets, int E,
                         const float* g_gate, const float* g_up, const float* row_gs,
                         uint16_t* h, uint8_t* q, uint8_t* sc, float* h_gs, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const dim3 grid((R + 3) / 4), block(256);
  const size_t lds = sizeof(int) * (size_t)(E + 1);
  switch (bpl_for(I / 16)) {
    case 1: hipLaunchKernelGGL(k_swiglu<1>, grid, block, lds, s, acc13, R, I, offsets, E, g_gate, g_up, row_gs, h, q, sc, h_gs); break;
    case 2: hipLaunchKernelGGL(k_swiglu<2>, grid, block, lds, s, acc13, R, I, offsets, E, g_gate, g_up, row_gs, h, q, sc, h_gs); break;
    case 4: hipLaunchKernelGGL(k_swiglu<4>, grid, block, lds, s, acc13, R, I, offsets, E, g_gate, g_up, row_gs, h, q, sc, h_gs); break;
    default: hipLaunchKernelGGL(k_swiglu<8>, grid, block, lds, s, acc13, R, I, offsets, E, g_gate, g_up, row_gs, h, q, sc, h_gs); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------- scatter
// Grid (T, ceil(H / 256)); one wave per (token, 256 columns), 4 columns per lane.  The
// token's rows are taken 64 at a time: each lane finds one row's expert and coefficient
// row_w * g_down * row_gs, then the wave accumulates the rows in ascending order.
__global__ __launch_bounds__(64) void k_scatter(const float* __restrict__ y, int H,
                                                const int32_t* __restrict__ offsets, int E,
                                                const float* __restrict__ row_w,
                                                const float* __restrict__ g_down,
                                                const float* __restrict__ row_gs,
                                                const int32_t* __restrict__ tok_off,
                                                const int32_t* __restrict__ tok_rows,
                                                uint16_t* __restrict__ out) {
  extern __shared__ int s_off[];
  for (int k = threadIdx.x; k <= E; k += blockDim.x) s_off[k] = offsets[k];
  __syncthreads();
  const int t = blockIdx.x, lane = threadIdx.x;
  const int col = blockIdx.y * 256 + 4 * lane;
  const bool cv = col < H;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int p0 = tok_off[t], p1 = tok_off[t + 1];
  for (int base = p0; base < p1; base += 64) {
    const int p = base + lane;
    int i = 0;
    float c = 0.0f;
    if (p < p1) {
      i = tok_rows[p];
      const int e = expert_of_row(s_off, E, i);
      c = (e < E) ? row_w[i] * g_down[e] * row_gs[i] : 0.0f;
    }
    const int n = min(64, p1 - base);
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
  if (cv) {
    u32x2 o;
    o[0] = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o[1] = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *(u32x2*)(out + (size_t)t * H + col) = o;
  }
}

hipError_t launch_scatter(const float* y, int R, int H, const int32_t* offsets, int E,
                          const float* row_w, const float* g_down, const float* row_gs,
                          const int32_t* tok_off, const int32_t* tok_rows, int T, uint16_t* out,
                          hipStream_t s) {
  (void)R;
  if (T == 0) return hipSuccess;
  const dim3 grid(T, (H + 255) / 256), block(64);
  const size_t lds = sizeof(int) * (size_t)(E + 1);
  hipLaunchKernelGGL(k_scatter, grid, block, lds, s, y, H, offsets, E, row_w, g_down, row_gs,
                     tok_off, tok_rows, out);
  return hipGetLastError();
}

}  // namespace moe
