// Row grouping (stable counting sort by expert id, then by output row) and row gather.
//
// One workgroup does the whole grouping: R is at most a few thousand expert-rows per
// layer step, so the work is latency-bound and one CU with LDS histograms is enough.
//   1. every thread validates its assignments, counts them per expert (invalid ones in
//      an extra bucket E) and per output row, ORs error bits;
//   2. exclusive scans of both histograms (expert_offsets, tok_off);
//   3. wave 0 places assignments in (expert, j) order, 64 at a time: within a batch the
//      lanes holding the same key find each other with one ballot per key bit, so a
//      lane's rank is the popcount of equal-key lanes below it — no atomics, stable;
//   4. wave 0 places grouped rows into the token lists the same way, in ascending i.
#include "common.h"

namespace moe {

constexpr int kGroupThreads = 1024;

// Lanes of the wave whose `key` equals this lane's key (keys < 2^bits).
__device__ __forceinline__ uint64_t match_key(uint32_t key, int bits, bool active) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < bits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t v = __ballot(active && bit);
    m &= bit ? v : ~v;
  }
  return active ? m : 0ull;
}

// Exclusive scan of cnt[0..n) in place by the whole workgroup; returns the total.
__device__ int block_exclusive_scan(int* cnt, int n, int* s_part) {
  const int tid = threadIdx.x;
  const int per = (n + kGroupThreads - 1) / kGroupThreads;
  const int lo = tid * per, hi = min(n, lo + per);
  int local = 0;
  for (int k = lo; k < hi; ++k) local += cnt[k];
  // inclusive scan of the per-thread sums across the block (wave scan + wave totals)
  const int lane = tid & 63, wave = tid >> 6;
  int v = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) s_part[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kGroupThreads / 64 ? s_part[lane] : 0;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(w, d, 64);
      if (lane >= d) w += o;
    }
    if (lane < kGroupThreads / 64) s_part[lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  int run = v - local + (wave ? s_part[wave - 1] : 0);  // exclusive prefix of this thread
  for (int k = lo; k < hi; ++k) {
    const int c = cnt[k];
    cnt[k] = run;
    run += c;
  }
  const int total = s_part[kGroupThreads / 64 - 1];
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kGroupThreads) void k_group(
    const int32_t* __restrict__ a_expert, const int32_t* __restrict__ a_src,
    const int32_t* __restrict__ a_dst, const float* __restrict__ a_w, int R, int E, int S, int T,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_src, int32_t* __restrict__ row_dst,
    float* __restrict__ row_w, int32_t* __restrict__ tok_off, int32_t* __restrict__ tok_rows,
    int32_t* __restrict__ err_word) {
  extern __shared__ int lds[];
  int* cnt_e = lds;              // E + 1 (bucket E = dropped assignments)
  int* cnt_t = lds + (E + 1);    // T + 1
  __shared__ int s_part[kGroupThreads / 64];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  for (int k = tid; k < E + 1; k += kGroupThreads) cnt_e[k] = 0;
  for (int k = tid; k < T + 1; k += kGroupThreads) cnt_t[k] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();

  // 1. validate and count
  int err = 0;
  for (int j = tid; j < R; j += kGroupThreads) {
    const int e = a_expert[j], s = a_src[j], d = a_dst[j];
    int bad = 0;
    if (e < 0 || e >= E) bad |= MOE_ERR_EXPERT;
    if (s < 0 || s >= S) bad |= MOE_ERR_SRC;
    if (d < 0 || d >= T) bad |= MOE_ERR_DST;
    err |= bad;
    atomicAdd(&cnt_e[bad ? E : e], 1);
    if (!bad) atomicAdd(&cnt_t[d], 1);
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();

  // 2. scans
  block_exclusive_scan(cnt_e, E + 1, s_part);
  block_exclusive_scan(cnt_t, T + 1, s_part);
  for (int k = tid; k < E + 1; k += kGroupThreads) expert_offsets[k] = cnt_e[k];
  for (int k = tid; k < T + 1; k += kGroupThreads) tok_off[k] = cnt_t[k];
  if (tid == 0) *err_word = s_err;
  __syncthreads();  // offsets read back below from LDS only

  int ebits = 1;
  while ((1 << ebits) < E + 1) ++ebits;
  int tbits = 1;
  while ((1 << tbits) < T + 1) ++tbits;

  // 3. stable placement by expert (wave 0; cnt_e now holds running cursors)
  if (tid < 64) {
    const int lane = tid;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < R; base += 64) {
      const int j = base + lane;
      const bool act = j < R;
      int key = E, s = -1, d = -1;
      float w = 0.f;
      if (act) {
        const int e = a_expert[j];
        s = a_src[j];
        d = a_dst[j];
        const bool ok = e >= 0 && e < E && s >= 0 && s < S && d >= 0 && d < T;
        key = ok ? e : E;
        if (ok) w = a_w[j];
        else { s = -1; d = -1; }
      }
      const uint64_t same = match_key((uint32_t)key, ebits, act);
      const int rank = __popcll(same & below);
      const int cur = act ? cnt_e[key] : 0;
      const int pos = cur + rank;
      if (act) {
        row_src[pos] = s;
        row_dst[pos] = d;
        row_w[pos] = w;
        if (rank == __popcll(same) - 1) cnt_e[key] = pos + 1;  // last lane of its key
      }
    }
  }
  __syncthreads();

  // 4. token lists in ascending grouped row (wave 0; cnt_t holds running cursors)
  if (tid < 64) {
    const int lane = tid;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int Rv = expert_offsets[E];
    for (int base = 0; base < Rv; base += 64) {
      const int i = base + lane;
      const bool act = i < Rv;
      const int d = act ? row_dst[i] : 0;
      const uint64_t same = match_key((uint32_t)d, tbits, act);
      const int rank = __popcll(same & below);
      const int cur = act ? cnt_t[d] : 0;
      if (act) {
        tok_rows[cur + rank] = i;
        if (rank == __popcll(same) - 1) cnt_t[d] = cur + rank + 1;
      }
    }
  }
}

hipError_t launch_group(const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                        const float* a_w, int R, int E, int S, int T, int32_t* expert_offsets,
                        int32_t* row_src, int32_t* row_dst, float* row_w, int32_t* tok_off,
                        int32_t* tok_rows, int32_t* err_word, hipStream_t s) {
  const size_t lds = sizeof(int) * (size_t)(E + 1 + T + 1);
  hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupThreads), lds, s, a_expert, a_src, a_dst, a_w,
                     R, E, S, T, expert_offsets, row_src, row_dst, row_w, tok_off, tok_rows,
                     err_word);
  return hipGetLastError();
}

// xg[i] = x[row_src[i]], zero rows for row_src < 0.  One thread per 16 bytes.
__global__ void k_gather(const uint16_t* __restrict__ x, int H, const int32_t* __restrict__ row_src,
                         int R, uint16_t* __restrict__ xg) {
  const int per_row = H / 8;  // 16-byte units
  const size_t total = (size_t)R * per_row;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(u / per_row), c = (int)(u % per_row);
    const int s = row_src[i];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (s >= 0) v = *(const u32x4*)(x + (size_t)s * H + 8 * c);
    *(u32x4*)(xg + (size_t)i * H + 8 * c) = v;
  }
}

hipError_t launch_gather(const uint16_t* x, int H, const int32_t* row_src, int R, uint16_t* xg,
                         hipStream_t s) {
  const size_t total = (size_t)R * (H / 8);
  if (total == 0) return hipSuccess;
  const size_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_gather, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                     x, H, row_src, R, xg);
  return hipGetLastError();
}

}  // namespace moe
