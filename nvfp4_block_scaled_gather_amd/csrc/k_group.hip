// Row grouping (stable sort by expert id, then by output row), row gather, and the fused
// grouping + source-row quantization launch of the layer.
//
// One workgroup does the whole grouping: R is at most a few thousand expert-rows per
// layer step, so the work is latency-bound and one CU with LDS is enough:
//   1. every thread validates its assignments, counts them per expert (invalid ones in an
//      extra bucket E) and per output row, and ORs error bits;
//   2. exclusive scans of both histograms give expert_offsets and tok_off;
//   3. assignments are placed in (expert, j) order and 4. grouped rows into the token
//      lists in ascending i, both by stable_place: all 16 waves when per-wave histograms
//      of the keys fit in LDS (E and T up to about 900), else one wave.
// A small batch (R <= 32, a decode step of up to 4 tokens at top-8) is grouped by one wave
// with no workgroup barrier and no LDS (group_small): measured on MI355X, 2 us faster for
// one and two tokens, even at 4, and slower than the 16-wave path at 8 (its ranking loops
// grow with R).
#include "common.h"

namespace moe {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kSmallGroupRows = 32;  // group_small: at most one assignment per lane
constexpr int kWorkListUnits = 256;  // units of 64 experts of the work list's two sets

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

// Inclusive prefix sum of v over the 64 lanes of a wave: a scan within each row of 16
// lanes by row shifts (lanes shifted in from outside the row add 0), then the totals of
// the rows below (read from their last lanes) added to each row.  Every lane must call it.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Exclusive scan of cnt[0..n) in place by the whole workgroup; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int* cnt, int n, int* s_part) {
  const int tid = threadIdx.x;
  const int per = (n + kGroupThreads - 1) / kGroupThreads;
  const int lo = tid * per, hi = min(n, lo + per);
  int local = 0;
  for (int k = lo; k < hi; ++k) local += cnt[k];
  // inclusive scan of the per-thread sums across the block (wave scan + wave totals)
  const int lane = tid & 63, wave = tid >> 6;
  const int v = wave_scan_incl(local);
  if (lane == 63) s_part[wave] = v;
  __syncthreads();
  if (wave == 0) {
    const int w = wave_scan_incl(lane < kGroupWaves ? s_part[lane] : 0);
    if (lane < kGroupWaves) s_part[lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  int run = v - local + (wave ? s_part[wave - 1] : 0);  // exclusive prefix of this thread
  for (int k = lo; k < hi; ++k) {
    const int c = cnt[k];
    cnt[k] = run;
    run += c;
  }
  const int total = s_part[kGroupWaves - 1];
  __syncthreads();
  return total;
}

// Stable counting sort of n items by key (< nkeys), into positions starting at
// bucket_start[key] (an exclusive prefix of the key counts; used as scratch).
// With nw = 16 waves, wave w owns the contiguous segment [w*seg, (w+1)*seg): per-wave key
// histograms (hist, 16 x nkeys ints of LDS) turn the bucket starts into per-(wave, key)
// cursors (hist_zeroed: the caller cleared those 16 x nkeys ints already, before a barrier).
// With nw = 1, wave 0 walks all items and bucket_start itself is the cursor.
// Inside a wave items go 64 at a time; a lane's rank is the number of equal-key lanes
// below it.  With `masks` (nw x nkeys 64-bit words of LDS, zero on entry and on return)
// the lanes OR their bit into their key's word and read it back (OR is order-free, so the
// result is deterministic); without, lanes holding equal keys find each other with one
// ballot per key bit (about 20 instructions per bit: the masks are several times cheaper).
// Resulting order: (key, item index) — stable and deterministic.
template <typename KeyFn, typename PlaceFn>
__device__ __forceinline__ void stable_place(int n, int nkeys, int* bucket_start, int* hist, int nw,
                                             KeyFn key_of, PlaceFn place,
                                             unsigned long long* masks = nullptr,
                                             bool hist_zeroed = false) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = (n + nw - 1) / nw;
  const int j0 = wave < nw ? wave * seg : n, j1 = min(n, j0 + seg);
  int* h = bucket_start;
  if (nw > 1) {
    h = hist + wave * nkeys;
    if (!hist_zeroed) {
      for (int k = tid; k < nw * nkeys; k += kGroupThreads) hist[k] = 0;
      __syncthreads();
    }
    for (int j = j0 + lane; j < j1; j += 64) atomicAdd(&h[key_of(j)], 1);
    __syncthreads();
    for (int b = tid; b < nkeys; b += kGroupThreads) {  // (nw == kGroupWaves here)
      int c[kGroupWaves];
#pragma unroll
      for (int w = 0; w < kGroupWaves; ++w) c[w] = hist[w * nkeys + b];  // all reads first
      int run = bucket_start[b];
#pragma unroll
      for (int w = 0; w < kGroupWaves; ++w) {
        hist[w * nkeys + b] = run;
        run += c[w];
      }
    }
    __syncthreads();
  }
  int bits = 1;
  while ((1 << bits) < nkeys) ++bits;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  unsigned long long* mw = masks ? masks + (size_t)(nw > 1 ? wave : 0) * nkeys : nullptr;
  for (int base = j0; base < j1; base += 64) {
    const int j = base + lane;
    const bool act = j < j1;
    const int key = act ? key_of(j) : 0;
    uint64_t same;
    if (mw) {  // uniform
      if (act) atomicOr(&mw[key], 1ull << lane);
      same = act ? mw[key] : 0ull;
      if (act) mw[key] = 0ull;  // after every lane's read (one wave's LDS ops stay in order)
    } else {
      same = match_key((uint32_t)key, bits, act);
    }
    const int rank = __popcll(same & below);
    const int pos = act ? h[key] + rank : 0;
    if (act) {
      place(j, pos);
      if (rank == __popcll(same) - 1) h[key] = pos + 1;  // last lane of its key
    }
  }
  __syncthreads();
}

// LDS ints the grouping needs: the two histograms, plus the per-wave ones when parallel,
// plus (cached) the R assignments, the grouped rows' output rows and the per-wave 64-bit
// key masks of the ranking (two ints each, 8-byte aligned).
constexpr int kCachedInts = 7;  // per assignment: key, src, dst, weight; grouped dst, src, weight
__host__ __device__ inline size_t group_lds_ints(int E, int T, bool parallel, int R, bool cached) {
  const size_t base = (size_t)(E + 1) + (size_t)(T + 1);
  const size_t keys = (size_t)((E > T ? E : T) + 1);
  const size_t par = parallel ? (size_t)kGroupWaves * keys : 0;
  const size_t masks = cached ? 2 * (size_t)(parallel ? kGroupWaves : 1) * keys + 2 : 0;
  return base + par + (cached ? (size_t)kCachedInts * (size_t)R : 0) + masks;
}

// The whole grouping, by one workgroup of kGroupThreads threads.  CACHED: the assignments
// are read from global memory once, into LDS, and every later phase reads LDS (the phases
// are otherwise a chain of dependent global round trips); the grouped rows and token lists
// are placed in LDS too and written out in order, with coalesced stores (measured on
// MI355X, scattered 4-byte stores of the placements from this one CU made the two placing
// phases 2.5 us slower at 2303 assignments).
template <bool CACHED>
__device__ __forceinline__ void group_body(const int32_t* __restrict__ a_expert, const int32_t* __restrict__ a_src,
                           const int32_t* __restrict__ a_dst, const float* __restrict__ a_w, int R,
                           int E, int S, int T, int32_t* __restrict__ expert_offsets,
                           int32_t* __restrict__ row_src, int32_t* __restrict__ row_dst,
                           float* __restrict__ row_w, int32_t* __restrict__ tok_off,
                           int32_t* __restrict__ tok_rows, int32_t* __restrict__ err_word,
                           bool parallel, int* lds, int4* __restrict__ items = nullptr) {
  int* cnt_e = lds;                     // E + 1 (bucket E = dropped assignments)
  int* cnt_t = lds + (E + 1);           // T + 1
  int* hist = lds + (E + 1) + (T + 1);  // kGroupWaves x (max(E, T) + 1) when parallel
  int* c_key = hist + (parallel ? kGroupWaves * ((E > T ? E : T) + 1) : 0);  // CACHED: R each
  int* c_src = c_key + R;
  int* c_dst = c_src + R;
  float* c_w = (float*)(c_dst + R);
  int* g_dst = c_dst + 2 * R;  // output row of grouped row i (-1: dropped)
  int* g_src = g_dst + R;      // its source row (-1: dropped)
  float* g_w = (float*)(g_src + R);  // its router weight
  int* t_rows = c_key;         // token lists, once the keys are no longer read
  // CACHED: the per-wave key masks of the ranking, after the cache (8-byte aligned)
  const size_t mo = (size_t)(g_dst + 3 * R - lds);
  unsigned long long* masks =
      CACHED ? (unsigned long long*)(lds + ((mo + 1) & ~(size_t)1)) : nullptr;
  const int nkmax = (E > T ? E : T) + 1;
  __shared__ int s_part[kGroupWaves];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  const int nw = parallel ? kGroupWaves : 1;
  for (int k = tid; k < E + 1; k += kGroupThreads) cnt_e[k] = 0;
  for (int k = tid; k < T + 1; k += kGroupThreads) cnt_t[k] = 0;
  if (CACHED)
    for (int k = tid; k < nw * nkmax; k += kGroupThreads) masks[k] = 0ull;
  if (parallel)  // the expert placement's per-wave histograms (stable_place, hist_zeroed)
    for (int k = tid; k < nw * (E + 1); k += kGroupThreads) hist[k] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();
  // 1. validate and count (four assignments' loads in flight per thread)
  int err = 0;
  for (int base = 0; base < R; base += 4 * kGroupThreads) {
    int ev[4], sv[4], dv[4];
    float wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = base + u * kGroupThreads + tid;
      ev[u] = sv[u] = dv[u] = 0;
      wv[u] = 0.f;
      if (j < R) {
        ev[u] = a_expert[j];
        sv[u] = a_src[j];
        dv[u] = a_dst[j];
        if (CACHED) wv[u] = a_w[j];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = base + u * kGroupThreads + tid;
      if (j >= R) break;
      const int e = ev[u], sr = sv[u], d = dv[u];
      int bad = 0;
      if (e < 0 || e >= E) bad |= MOE_ERR_EXPERT;
      if (sr < 0 || sr >= S) bad |= MOE_ERR_SRC;
      if (d < 0 || d >= T) bad |= MOE_ERR_DST;
      err |= bad;
      atomicAdd(&cnt_e[bad ? E : e], 1);
      if (!bad) atomicAdd(&cnt_t[d], 1);
      if (CACHED) {
        c_key[j] = bad ? E : e;
        c_src[j] = sr;
        c_dst[j] = d;
        c_w[j] = wv[u];
      }
    }
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  // 2. bucket starts: one exclusive scan over both histograms (cnt_t follows cnt_e in LDS);
  // the token part then starts at R (every assignment is counted once in cnt_e), taken off
  block_exclusive_scan(cnt_e, (E + 1) + (T + 1), s_part);
  for (int k = tid; k < E + 1; k += kGroupThreads) expert_offsets[k] = cnt_e[k];
  for (int k = tid; k < T + 1; k += kGroupThreads) {
    const int v = cnt_t[k] - R;
    cnt_t[k] = v;
    tok_off[k] = v;
  }
  if (tid == 0) *err_word = s_err;
  const int Rv = cnt_e[E];
  // 2b. the GEMMs' work list (when asked for): the non-empty groups in the order the grouped
  // GEMM takes them, groups of more than kWorkListMultiRows rows first, each set in ascending
  // expert id; items[0] = {groups, groups of the first set}, items[1 + a] = {expert, first
  // row, rows, a} of group a.  With it a GEMM workgroup finds its group with one load
  // instead of a scan of the offsets.  From the offsets in LDS, by all waves: unit u of the
  // list is 64 experts of one set (u < nb: the first set, experts 64 u ..; then the second),
  // wave w takes units w, w + 16, ...: one ballot counts a unit's groups, a barrier, then
  // each wave places its units' groups after the counts of the units before them.
  if (items) {  // uniform
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int nb = (E + 63) / 64, nu = 2 * nb;  // nu <= kWorkListUnits (E <= 8192)
    __shared__ int s_cnt[kWorkListUnits];
    auto unit_sel = [&](int u, int& e) {
      const int set = u / nb;
      e = (u - set * nb) * 64 + lane;
      const int G = e < E ? cnt_e[e + 1] - cnt_e[e] : 0;
      return set == 0 ? G > kWorkListMultiRows : (G > 0 && G <= kWorkListMultiRows);
    };
    for (int u = wave; u < nu; u += kGroupWaves) {
      int e;
      const int c = __popcll(__ballot(unit_sel(u, e)));
      if (lane == 0) s_cnt[u] = c;
    }
    __syncthreads();
    // the units' exclusive prefix: one scan over the wave when there are at most 64 units
    // (E <= 2048), else sums of the counts read from LDS
    int incl = 0, total = 0, n_multi = 0;
    if (nu <= 64) {  // uniform
      incl = wave_scan_incl(lane < nu ? s_cnt[lane] : 0);
      total = __builtin_amdgcn_readlane(incl, 63);
      n_multi = __builtin_amdgcn_readlane(incl, nb - 1);
    } else {
      for (int u = 0; u < nu; ++u) {
        total += s_cnt[u];
        if (u == nb - 1) n_multi = total;
      }
    }
    for (int u = wave; u < nu; u += kGroupWaves) {
      int before;
      if (nu <= 64) {
        before = __builtin_amdgcn_readlane(incl, u) - s_cnt[u];
      } else {
        before = 0;
        for (int v = 0; v < u; ++v) before += s_cnt[v];
      }
      int e;
      const bool sel = unit_sel(u, e);
      const uint64_t m = __ballot(sel);
      const int a = before + __popcll(m & below);
      if (sel) items[1 + a] = int4{e, cnt_e[e], cnt_e[e + 1] - cnt_e[e], a};
    }
    if (tid == 0) items[0] = int4{total, n_multi, 0, 0};
  }
  __syncthreads();
  // 3. grouped rows in (expert, assignment) order; dropped assignments last
  if constexpr (CACHED) {
    stable_place(R, E + 1, cnt_e, hist, nw, [&](int j) -> int { return c_key[j]; },
                 [&](int j, int pos) {
                   const bool ok = pos < Rv;
                   g_src[pos] = ok ? c_src[j] : -1;
                   g_dst[pos] = ok ? c_dst[j] : -1;
                   g_w[pos] = ok ? c_w[j] : 0.f;
                 }, masks, parallel);
    for (int i = tid; i < R; i += kGroupThreads) {  // (after stable_place's barrier)
      row_src[i] = g_src[i];
      row_dst[i] = g_dst[i];
      row_w[i] = g_w[i];
    }
  } else {
    auto key_e = [&](int j) -> int {
      const int e = a_expert[j], sr = a_src[j], d = a_dst[j];
      const bool ok = e >= 0 && e < E && sr >= 0 && sr < S && d >= 0 && d < T;
      return ok ? e : E;
    };
    stable_place(R, E + 1, cnt_e, hist, nw, key_e, [&](int j, int pos) {
      const bool ok = pos < Rv;
      row_src[pos] = ok ? a_src[j] : -1;
      row_dst[pos] = ok ? a_dst[j] : -1;
      row_w[pos] = ok ? a_w[j] : 0.f;
    }, nullptr, parallel);
  }
  // 4. token lists, ascending grouped row (the grouped rows' outputs are visible after
  // stable_place's barrier)
  if constexpr (CACHED) {
    stable_place(Rv, T, cnt_t, hist, nw, [&](int i) -> int { return g_dst[i]; },
                 [&](int i, int pos) { t_rows[pos] = i; }, masks);
    for (int i = tid; i < Rv; i += kGroupThreads) tok_rows[i] = t_rows[i];
  } else {
    stable_place(Rv, T, cnt_t, hist, nw, [&](int i) -> int { return row_dst[i]; },
                 [&](int i, int pos) { tok_rows[pos] = i; });
  }
}

__global__ __launch_bounds__(kGroupThreads) void k_group(
    const int32_t* __restrict__ a_expert, const int32_t* __restrict__ a_src,
    const int32_t* __restrict__ a_dst, const float* __restrict__ a_w, int R, int E, int S, int T,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_src, int32_t* __restrict__ row_dst,
    float* __restrict__ row_w, int32_t* __restrict__ tok_off, int32_t* __restrict__ tok_rows,
    int32_t* __restrict__ err_word, bool parallel, bool cached, int4* __restrict__ items) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  if (R <= kSmallGroupRows)
    group_small(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst, row_w,
                tok_off, tok_rows, err_word, items);
  else if (cached)
    group_body<true>(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst,
                     row_w, tok_off, tok_rows, err_word, parallel, lds, items);
  else
    group_body<false>(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst,
                      row_w, tok_off, tok_rows, err_word, parallel, lds, items);
}

// Grouping (block 0) and NVFP4 quantization of the S source rows of x (the other blocks,
// 1024 / nthreads rows each) in one launch: the two are independent, since a row's codes
// depend only on the row.  Block 0 also clears zero[0 .. nzero) (the next launch's
// counters).
template <int BPT>
__global__ __launch_bounds__(kGroupThreads) void k_group_quantize(
    const int32_t* __restrict__ a_expert, const int32_t* __restrict__ a_src,
    const int32_t* __restrict__ a_dst, const float* __restrict__ a_w, int R, int E, int S, int T,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_src, int32_t* __restrict__ row_dst,
    float* __restrict__ row_w, int32_t* __restrict__ tok_off, int32_t* __restrict__ tok_rows,
    int32_t* __restrict__ err_word, bool parallel, bool cached,
    const uint16_t* __restrict__ x, int H, int nthreads, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs, float* __restrict__ xgs, int4* __restrict__ items,
    int* __restrict__ zero, int nzero) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  __shared__ float s_red[kGroupWaves];
  if (blockIdx.x == 0) {
    for (int k = threadIdx.x; k < nzero; k += kGroupThreads) zero[k] = 0;
    if (R <= kSmallGroupRows)  // (no work list: the GEMMs scan the offsets)
      group_small(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst,
                  row_w, tok_off, tok_rows, err_word);
    else if (cached)
      group_body<true>(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst,
                       row_w, tok_off, tok_rows, err_word, parallel, lds, items);
    else
      group_body<false>(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst,
                        row_w, tok_off, tok_rows, err_word, parallel, lds, items);
    return;
  }
  const int rows_per_block = kGroupThreads / nthreads;
  const int slot = threadIdx.x / nthreads, t = threadIdx.x % nthreads;
  const int row = (blockIdx.x - 1) * rows_per_block + slot;
  const bool active = row < S;
  const int NB = H / 16;
  float v[BPT][16];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int b = t + nthreads * k;
    u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
    if (active && b < NB) {
      const u32x4* p = (const u32x4*)(x + (size_t)row * H + 16 * b);
      w0 = p[0];
      w1 = p[1];
    }
    bf16x16_to_f32(w0, w1, v[k]);
  }
  // every thread takes part in the row-max barrier; only the slots of real rows store
  const float amax = row_amax_threads<BPT>(v, t, nthreads, s_red + slot * (nthreads / 64));
  if (active)
    quantize_row_store<BPT>(v, NB, t, nthreads, amax, xq + (size_t)row * (H / 2),
                            xs + (size_t)row * NB, xgs + row);
}

// LDS of the grouping workgroup: per-wave histograms when they fit in 64 KiB; the cached
// assignments on top when the total fits in the CU's 160 KiB.
constexpr size_t kGroupLdsMax = 158 * 1024;  // the CU's 160 KiB less the static LDS

static bool group_parallel(int E, int T) {
  return group_lds_ints(E, T, true, 0, false) * sizeof(int) <= 65536;
}

static bool group_cached(int E, int T, int R) {
  return group_lds_ints(E, T, group_parallel(E, T), R, true) * sizeof(int) <= kGroupLdsMax;
}

template <class Kern>
static hipError_t set_lds(Kern kern, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

hipError_t launch_group(const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                        const float* a_w, int R, int E, int S, int T, int32_t* expert_offsets,
                        int32_t* row_src, int32_t* row_dst, float* row_w, int32_t* tok_off,
                        int32_t* tok_rows, int32_t* err_word, hipStream_t s, int4* items) {
  const bool par = group_parallel(E, T), cached = group_cached(E, T, R);
  const size_t lds = R <= kSmallGroupRows ? 0 : group_lds_ints(E, T, par, R, cached) * sizeof(int);
  const hipError_t e = set_lds(k_group, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupThreads), lds, s, a_expert, a_src, a_dst, a_w, R,
                     E, S, T, expert_offsets, row_src, row_dst, row_w, tok_off, tok_rows, err_word,
                     par, cached, items);
  return hipGetLastError();
}

hipError_t launch_group_quantize(const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                                 const float* a_w, int R, int E, int S, int T,
                                 int32_t* expert_offsets, int32_t* row_src, int32_t* row_dst,
                                 float* row_w, int32_t* tok_off, int32_t* tok_rows,
                                 int32_t* err_word, const uint16_t* x, int H, uint8_t* xq,
                                 uint8_t* xs, float* xgs, int4* items, hipStream_t s, int* zero,
                                 int nzero) {
  const bool par = group_parallel(E, T), cached = group_cached(E, T, R);
  const int NB = H / 16, nt = row_threads(NB);
  const int rows_per_block = kGroupThreads / nt;
  const dim3 grid(1 + (S + rows_per_block - 1) / rows_per_block);
  const size_t lds = R <= kSmallGroupRows ? 0 : group_lds_ints(E, T, par, R, cached) * sizeof(int);
  if (NB <= 256) {
    const hipError_t e = set_lds(k_group_quantize<1>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_group_quantize<1>, grid, dim3(kGroupThreads), lds, s, a_expert, a_src,
                       a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst, row_w, tok_off,
                       tok_rows, err_word, par, cached, x, H, nt, xq, xs, xgs, items, zero,
                       nzero);
  } else {
    const hipError_t e = set_lds(k_group_quantize<2>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_group_quantize<2>, grid, dim3(kGroupThreads), lds, s, a_expert, a_src,
                       a_dst, a_w, R, E, S, T, expert_offsets, row_src, row_dst, row_w, tok_off,
                       tok_rows, err_word, par, cached, x, H, nt, xq, xs, xgs, items, zero,
                       nzero);
  }
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
