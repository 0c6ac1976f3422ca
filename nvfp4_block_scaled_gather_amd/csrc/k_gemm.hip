// Grouped NVFP4 GEMM: out[i, n] = sum_k a(i, k) * w_e(n, k) for every row i of every
// non-empty expert group e (alpha = 1; the globals are applied by the next kernel).
//
// The GEMM is weight-stream bound: every active expert's packed weights are read from HBM
// exactly once.  Per 16-row tile, a wave reads each 128-column chunk with one 16-byte load
// per lane and the scales of a group of up to 8 chunks with one load of up to 16 bytes per
// lane (layout in common.h), keeping a ring of D chunks in flight.
//
// Work decomposition: a work item is (expert, 4 * NS consecutive 16-row tiles) and one
// workgroup runs one item; each of its 4 waves streams NS tiles over all of K.  The
// group's activation rows are staged once per workgroup in LDS (direct buffer-to-LDS
// loads, up to 16 rows per pass), so the four waves share them and the vector-memory path
// carries only the weight stream.
//
// Two kernels, each over the groups its path owns (chosen per group on the device, so
// the host never needs the group sizes):
//  * k_gemm_mfma: the weight tile is the A operand of v_mfma_f32_16x16x32_f16 (16 weight
//    rows x 32 k), the pass's activation rows the B operand (16 columns).  Lane l holds
//    weight row l & 15 and the 32 k of quarter l >> 4 of each 128-column chunk; MFMA j of
//    the chunk takes word j (8 k) of that quarter, and the B operand uses the same k
//    assignment.  A B column beyond the pass's rows only feeds an output row that is not
//    stored, so those lanes simply re-read row 0.
//  * k_gemm_gemv (groups of at most 4 rows per pass): each lane dots its weight row
//    segment with each activation row's matching segment, 16 elements (one scale block)
//    at a time with v_dot2_f32_f16, then multiplies by the weight block scale; the four
//    k-quarters are summed across lanes at the end in a fixed tree.
// Both dequantize exactly (dequant8 in common.h) and accumulate in fp32 in an order that
// depends only on (N, K) and the path, never on the other rows of the group.
// Two more kernels serve the layer's decode-sized batches (at most 32 assignments) on the
// MFMA path with k_gemm_mfma's passes and arithmetic: k_gemm_swiglu_grouping (w13 with the
// SwiGLU epilogue, each workgroup grouping the assignments and quantizing its group's
// source rows itself) and k_gemm_quantizing (w2, each workgroup quantizing its rows of h).
// k_gemm_layer runs the layer's two GEMMs and the quantization of h between them as one
// launch for batches of more than 32 assignments (k_gemm_mfma's items, flags between them).
//
// Outputs are written as whole rows of the workgroup's block (store_out): measured on
// MI355X, write-back stores that are later evicted from L2 in the middle of the weight
// stream cost 4-5% of a GEMM at these sizes (one to two microseconds per MB written),
// non-temporal stores less than half of that, full-line stores less again, and with NVFP4
// activations full-line stores written through at device scope less still.
#include "common.h"

#ifndef MOE_GEMM_NS
#define MOE_GEMM_NS 2  // 16-row tiles per wave, MFMA kernel
#endif
#ifndef MOE_GEMM_D
#define MOE_GEMM_D 4   // chunks in flight per wave, MFMA kernel
#endif
#ifndef MOE_GEMV_NS
#define MOE_GEMV_NS 2  // 16-row tiles per wave, GEMV kernel
#endif
#ifndef MOE_GEMV_D
#define MOE_GEMV_D 2
#endif
#ifndef MOE_W_CPOL
#define MOE_W_CPOL 2  // cache policy of the weight-stream loads: non-temporal (read once)
#endif
// Weight loads of a group that takes several passes (more than 16 rows): through the
// caches (SC0), so that its later passes find the item's weights in the MALL instead of
// HBM.  Measured on MI355X against non-temporal loads: the Zipf decode batch (six groups of
// 21-57 rows) 2.9% faster; caching every item's weights instead was 11% slower on ragged570.
constexpr int kMultiPassWCpol = 1;


namespace moe {

constexpr int kGemmWaves = 4;
// s_waitcnt operand that waits for LDS (lgkmcnt 0) and leaves vector-memory loads and
// exports in flight (vmcnt 63, expcnt 7: the largest counts, i.e. no wait).
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int kPassRows = 16;  // activation rows per MFMA pass (the B operand's columns)
constexpr int kGemvRows = 4;   // activation rows per GEMV pass

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
  // SwiGLU epilogue (w13 with N = 2I): h [rows, I] bf16 instead of out
  const float* g_gate;
  const float* g_up;
  const float* row_gs;
  const int32_t* gs_map;  // grouped row i uses row_gs[gs_map[i]]; nullptr: row_gs[i]
  uint16_t* h;
  int I;
  // Scatter-ready output (w2 of the layer; c_w != nullptr): grouped row i is multiplied by
  // c_w[i] * c_g[e] * c_gs[i] (router weight, the expert's down global, the row's
  // activation global), the term the scatter-add sums.
  const float* c_w;
  const float* c_g;
  const float* c_gs;       // nullptr: 1 (bf16 activations carry no row global)
  // W4A16: bf16 activation rows [a_rows, K] (through amap) in place of aq / as
  const uint16_t* ab;
  // The grouping's work list (kWorkListMultiRows), or nullptr: workgroups then scan the
  // offsets.  Only for launches that own every group (gmin <= 1, no upper bound).
  const int4* items;
};

// ------------------------------------------------------------------------- LDS layout
// [rows x q_stride nibbles][rows x s_stride scales] (or [rows x b_stride bf16]).  The row
// strides are padded so that the 16 rows a wave reads at once fall in
// distinct banks (a nibble row stride of 16 mod 256 bytes, a scale row stride of 8 mod 256).
__host__ __device__ __forceinline__ int q_stride(int K) { return K / 2 + 16; }
__host__ __device__ __forceinline__ int s_stride(int K) { return K / 16 + 8; }
// bf16 activation rows (W4A16): 2K bytes, padded the same way.
__host__ __device__ __forceinline__ int b_stride(int K) { return 2 * K + 16; }
// The staging area also holds the MFMA epilogue's output block (16 rows x the workgroup's
// columns plus padding), which for small K is larger than the staged rows; 256 bytes of
// slack keep the B-operand prefetch past the last chunk inside the allocation.
static size_t out_block_bytes(int NS, int waves, int rows = kPassRows) {
  return (size_t)rows * (16 * NS * waves + 4) * 4;
}
// A double pass (mfma_dpass) stages kDPassRows rows over half of K at a time.
constexpr int kDPassRows = 2 * kPassRows;
static size_t gemm_lds_bytes(int K, int rows, bool abf = false, int NS = 2,
                             int waves = kGemmWaves) {
  size_t stage = (size_t)rows * (abf ? b_stride(K) : q_stride(K) + s_stride(K));
  size_t outb = out_block_bytes(NS, waves);
  if (!abf && rows == kPassRows) {  // the instances that run double passes
    const size_t dstage = (size_t)kDPassRows * (q_stride(K / 2) + s_stride(K / 2));
    const size_t dout = out_block_bytes(NS, waves, kDPassRows);
    stage = stage > dstage ? stage : dstage;
    outb = outb > dout ? outb : dout;
  }
  return (stage > outb ? stage : outb) + 256;
}

// The group of a workgroup's item.  Active groups are the experts whose group size is in
// [gmin, gmax], in ascending expert id; item it of a launch belongs to active group
// it / items_per_e.  When some group needs two or more passes over its weights (more than
// PR rows), the groups of more than PR rows come first instead (each set in ascending
// expert id), so that their long items start first rather than forming the kernel's tail.
// Wave 0 scans the offsets (512 experts per round, all loads of a round in flight
// together) for group ai in plain order, counting the multi-pass groups on the way, and
// scans again only when there are any.  The lane that holds
// the group publishes (expert, first row, size) through LDS.  Returns false if there are at
// most ai active groups (the workgroup has no item).  The order changes which workgroup
// computes an output, never how.
struct ItemGroup {
  int e, r0, G;
};

template <int PR>
__device__ __forceinline__ bool find_group(const GemmArgs& p, int ai, int* s_grp, ItemGroup& g) {
  if (PR == kWorkListMultiRows && p.items) {
    // the grouping's work list has the groups in this order: one load (ai < min(E, R) <= E,
    // so the entry is inside the list even when it is past the last group)
    const int4 h = p.items[0];
    const int4 it = p.items[1 + ai];
    g.e = __builtin_amdgcn_readfirstlane(it.x);
    g.r0 = __builtin_amdgcn_readfirstlane(it.y);
    g.G = __builtin_amdgcn_readfirstlane(it.z);
    return ai < __builtin_amdgcn_readfirstlane(h.x);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    // Group number `target` among the active groups of the set `sel` (0: all; 1: more than
    // PR rows; 2: at most PR rows), in ascending expert id.  `count`: scan every expert and
    // count the multi-pass groups.
    int n_multi = 0;
    auto scan = [&](int sel, int target, bool count) {
      int n = 0, nm = 0;
      bool found = false;
      for (int base = 0; base < p.E && (count || !found); base += 512) {  // uniform
        int lo[8], hi[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = base + 64 * u + lane;
          lo[u] = e < p.E ? p.off[e] : 0;
          hi[u] = e < p.E ? p.off[e + 1] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = base + 64 * u + lane;
          const int sz = hi[u] - lo[u];
          const bool act = e < p.E && sz >= p.gmin && sz <= p.gmax;
          const bool mp = act && sz > PR;
          if (count) nm += __popcll(__ballot(mp));
          const bool a = act && (sel == 0 || mp == (sel == 1));
          const uint64_t m = __ballot(a);
          const int c = __popcll(m);
          if (!found && target < n + c) {  // uniform
            if (a && n + __popcll(m & below) == target) {
              s_grp[0] = e;
              s_grp[1] = lo[u];
              s_grp[2] = sz;
            }
            found = true;
          }
          n += c;
        }
      }
      if (count) n_multi = nm;
      return found;
    };
    bool found = scan(0, ai, true);
    if (n_multi > 0)  // the multi-pass groups first
      found = ai < n_multi ? scan(1, ai, false) : scan(2, ai - n_multi, false);
    if (lane == 0) s_grp[3] = found ? 1 : 0;
  }
  __syncthreads();
  g.e = __builtin_amdgcn_readfirstlane(s_grp[0]);
  g.r0 = __builtin_amdgcn_readfirstlane(s_grp[1]);
  g.G = __builtin_amdgcn_readfirstlane(s_grp[2]);
  return __builtin_amdgcn_readfirstlane(s_grp[3]) != 0;
}

// Buffer resource over [base, base + bytes): loads at offsets beyond the range return 0
// and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// GEMM output stores: 16 bytes at byte offset off of a pass's output rows.  With NVFP4
// activations they are written through the L2 at device scope (cache policy SC1), not
// marked non-temporal; measured on MI355X against non-temporal stores: the ragged2303 layer
// 0.9% faster, ragged570 0.6%, single-token decode 2% (the outputs are written in the middle
// of the weight stream and read by the next kernel).  The W4A16 instances (fewer, larger
// workgroups) measured 1% slower with them, so they keep non-temporal stores.  Write-back
// stores were 1.8-2.6% slower than non-temporal ones.
template <bool ABF>
__device__ __forceinline__ void store_out(const u32x4& v, __amdgpu_buffer_rsrc_t r, int off) {
  constexpr int kSC1 = 16, kNT = 2;
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, ABF ? kNT : kSC1);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Cache policy SC1 of a buffer access: device scope.  A store is written through this
// XCD's L2, and a load does not take a line that this L2 may hold from before another XCD
// wrote it; with these, data passes between workgroups of one launch without cache
// maintenance (the writer waits for its stores to complete before it signals).
constexpr int kDeviceScope = 16;

// Activation global of pass row r (< nrows) of rows arow0 ..: read at device scope when
// APOL says so (the rows' globals were written earlier in the same launch).
template <int APOL>
__device__ __forceinline__ float pass_row_global(const float* gs, int arow0, int nrows, int r) {
  if constexpr (APOL == 0) {
    return gs[arow0 + r];
  } else {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(gs + arow0, nrows * 4);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * r, 0, APOL));
  }
}

// Stage activation rows arow0 .. arow0 + nrows - 1 (through amap) into LDS with
// buffer-to-LDS loads: wave w copies rows w, w + WAVES, ...; an NVFP4 row is K/2 nibble
// bytes in 1 KiB pieces (16 bytes per lane) and K/16 scale bytes in 256-byte pieces (4
// bytes per lane); a bf16 row (ABF) is 2K bytes in 1 KiB pieces.  The caller waits for the
// loads and synchronizes before reading.  APOL: the loads' cache policy (kDeviceScope for
// rows written earlier in the same launch by other workgroups).
template <bool ABF, int WAVES, int APOL = 0>
__device__ __forceinline__ void stage_rows(const GemmArgs& p, int arow0, int nrows, uint8_t* s_q,
                                           uint8_t* s_s) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (ABF) {
    const int rb = 2 * p.K;
    const __amdgpu_buffer_rsrc_t br = make_rsrc(p.ab, p.a_rows * rb);
    for (int row = wave; row < nrows; row += WAVES) {
      const int i = arow0 + row;
      const int src = __builtin_amdgcn_readfirstlane(p.amap ? p.amap[i] : i);
      uint8_t* db = s_q + row * b_stride(p.K);
      for (int o = 0; o < rb; o += 1024) {
        if (o + 16 * lane < rb)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_ptr_t)(db + o), 16, 16 * lane,
                                                   src * rb + o, 0, APOL);
      }
    }
  } else {
    const int qb = p.K / 2, sb = p.K / 16;
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.aq, p.a_rows * qb);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.as, p.a_rows * sb);
    for (int row = wave; row < nrows; row += WAVES) {
      const int i = arow0 + row;
      const int src = __builtin_amdgcn_readfirstlane(p.amap ? p.amap[i] : i);
      uint8_t* dq = s_q + row * q_stride(p.K);
      uint8_t* ds = s_s + row * s_stride(p.K);
      for (int o = 0; o < qb; o += 1024) {
        if (o + 16 * lane < qb)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_ptr_t)(dq + o), 16, 16 * lane,
                                                   src * qb + o, 0, APOL);
      }
      for (int o = 0; o < sb; o += 256) {
        if (o + 4 * lane < sb)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_t)(ds + o), 4, 4 * lane,
                                                   src * sb + o, 0, APOL);
      }
    }
  }
}

// The 2S scale bytes of one scale group for this lane (voff: its byte offset in the group).
template <int S, int WC = MOE_W_CPOL>
__device__ __forceinline__ u32x4 load_scale_group(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if constexpr (S == 8) {
    v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, WC);
  } else if constexpr (S == 4) {
    const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, WC);
    v[0] = t[0];
    v[1] = t[1];
  } else if constexpr (S == 2) {
    v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, WC);
  } else {
    v[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, WC);
  }
  return v;
}

// The two scale bytes of chunk j of a group (low byte: the first 16 of the 32 columns).
__device__ __forceinline__ uint32_t chunk_scales(const u32x4& g, int j) {
  return (g[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
}

// ------------------------------------------------------------------------- weight ring
// Streams NS tiles (buffer wr, tiles sstride bytes apart) over all of K in scale groups of
// S chunks with a ring of D chunks (D <= S, both powers of two, S divides NC = K / 128).
// consume(c, j, wn, sg) uses chunk c (chunk j of its group): wn[s] holds its nibbles for
// tile s and sg[s] the group's scales.  Loads in the main loop are unconditional and
// pinned right after the use of their slot, so every wait is a counted one and the
// prefetch distance stays D chunks.
// The ring's registers: D chunks of NS tiles in flight, and the current scale group.
template <int NS, int D>
struct Ring {
  u32x4 wn[D][NS];
  u32x4 cur[NS];
};

template <int NS, int S, int WC>
__device__ __forceinline__ void ring_load_nib(u32x4 (&dst)[NS], __amdgpu_buffer_rsrc_t wr,
                                              int sstride, int vw, int c) {
  const int g = c / S, j = c - g * S;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    dst[s] = __builtin_amdgcn_raw_buffer_load_b128(wr, vw, s * sstride + g * S * kChunkBytes +
                                                               j * 1024, WC);
}

template <int NS, int S, int WC>
__device__ __forceinline__ void ring_load_scales(u32x4 (&dst)[NS], __amdgpu_buffer_rsrc_t wr,
                                                 int sstride, int vs, int g) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
    dst[s] = load_scale_group<S, WC>(wr, vs, s * sstride + g * S * kChunkBytes);
}

// The ring's first loads: scale group 0 (unless P0 > 0) and chunks P0 .. P-1.
template <int NS, int D, int S, int WC, int P = D, int P0 = 0>
__device__ __forceinline__ void ring_prime(Ring<NS, D>& rg, __amdgpu_buffer_rsrc_t wr,
                                           int sstride, int vw, int vs) {
  static_assert(0 <= P0 && P0 <= P && P <= D, "chunks P0 .. P-1 of the ring");
  if constexpr (P0 == 0) ring_load_scales<NS, S, WC>(rg.cur, wr, sstride, vs, 0);
#pragma unroll
  for (int d = P0; d < P; ++d) {
    ring_load_nib<NS, S, WC>(rg.wn[d], wr, sstride, vw, d);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Streams NS tiles (buffer wr, tiles sstride bytes apart) over all of K in scale groups of
// S chunks with a ring of D chunks (D <= S, both powers of two, S divides NC = K / 128).
// consume(c, j, wn, sg) uses chunk c (chunk j of its group): wn[s] holds its nibbles for
// tile s and sg[s] the group's scales.  Loads in the main loop are unconditional and
// pinned right after the use of their slot, so every wait is a counted one and the
// prefetch distance stays D chunks.  PRIMED > 0: the caller has issued the scale group and
// the first PRIMED chunks of the ring (ring_prime<..., PRIMED>) into rg already, earlier,
// so that their latency overlaps its own work; the rest are issued here.
template <int NS, int D, int S, class Consume, int WC = MOE_W_CPOL, int PRIMED = 0>
__device__ __forceinline__ void stream_weights(__amdgpu_buffer_rsrc_t wr, int NC, int sstride,
                                               int vw, int vs, Consume consume,
                                               Ring<NS, D>& rg) {
  u32x4 nxt[NS];
  const int NG = NC / S;
  if constexpr (PRIMED == 0) ring_prime<NS, D, S, WC>(rg, wr, sstride, vw, vs);
  else ring_prime<NS, D, S, WC, D, PRIMED>(rg, wr, sstride, vw, vs);
  int g = 0;
  for (; g + 1 < NG; ++g) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      consume(g * S + j, j, rg.wn[j % D], rg.cur);
      __builtin_amdgcn_sched_barrier(0);
      if (j == S - D) ring_load_scales<NS, S, WC>(nxt, wr, sstride, vs, g + 1);  // with the
                                                                              // first refill
      ring_load_nib<NS, S, WC>(rg.wn[j % D], wr, sstride, vw, g * S + j + D);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) rg.cur[s] = nxt[s];
  }
#pragma unroll
  for (int j = 0; j < S; ++j) {  // last group: refill only inside it
    consume(g * S + j, j, rg.wn[j % D], rg.cur);
    if (j + D < S) {
      __builtin_amdgcn_sched_barrier(0);
      ring_load_nib<NS, S, WC>(rg.wn[j % D], wr, sstride, vw, g * S + j + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int NS, int D, int S, int WC, int PRIMED = 0, class Consume>
__device__ __forceinline__ void stream_weights_c(__amdgpu_buffer_rsrc_t wr, int NC, int sstride,
                                                 int vw, int vs, Consume consume,
                                                 Ring<NS, D>& rg) {
  stream_weights<NS, D, S, Consume, WC, PRIMED>(wr, NC, sstride, vw, vs, consume, rg);
}

// The weight buffer of a pass's NS tiles (wt: the first, uniform; nsv: tiles this wave
// has, <= 0 for none: an empty range, so its loads return zeros and touch nothing) and the
// distance between its tiles (SWI: a gate tile and the up tile I/16 tiles after it).
template <bool SWI>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pass_weights(const GemmArgs& p,
                                                               const uint8_t* wt, int nsv,
                                                               int& sstride) {
  const int tstride = (p.K / 128) * kChunkBytes;
  sstride = SWI ? (p.I / 16) * tstride : tstride;
  const int range = nsv <= 0 ? 0 : SWI ? sstride + tstride : nsv * tstride;
  // (readfirstlane: the clamp may be computed on the vector unit, and a descriptor the
  // compiler believes divergent turns every load into a loop over lanes)
  return make_rsrc(wt, __builtin_amdgcn_readfirstlane(range));
}

// The pass's epilogue.  Lane l holds output rows r + 16 hr (hr < HR) x weight rows
// 4 kq .. 4 kq + 3 of each tile in acc[hr].  The workgroup's output block (its rows x
// 16 NS WAVES columns, or x 16 WAVES h columns) is assembled in LDS over the staged rows and
// written as whole rows, so every store covers full 128-byte lines (written from the lanes
// directly, each line arrived in 32- or 64-byte pieces from several waves).  ow / ogs:
// lane row r + 16 hr's router weight and activation global (scatter-ready epilogue); FQ:
// the row globals are s_rgs[row] instead.
template <int NS, int HR, bool SWI, bool ABF, int WAVES, bool FQ>
__device__ __forceinline__ void pass_epilogue(const GemmArgs& p, const f32x4 (&acc)[HR][NS],
                                              int nsv, int arow0, int nrows, int col0,
                                              uint8_t* s_q, float ggate, float gup,
                                              const float* s_rgs, const float (&ow)[HR],
                                              const float (&ogs)[HR]) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, r = lane & 15;
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // every wave is done with the staged rows: reuse them for the output
  if (SWI) {
    constexpr int WCH = 16 * WAVES;            // h columns of the workgroup
    constexpr int LPR = WCH / 8;               // 16-byte pieces per row
    uint16_t* so = (uint16_t*)s_q;             // [rows][WCH + 8] bf16 (the output block)
#pragma unroll
    for (int hr = 0; hr < HR; ++hr) {
      const int rr = r + kPassRows * hr;
      if (rr < nrows && nsv > 0) {
        const int i = arow0 + rr;
        const float gs = FQ ? s_rgs[rr] : p.row_gs ? p.row_gs[p.gs_map ? p.gs_map[i] : i] : 1.0f;
        const float cg = gs * ggate, cu = gs * gup;
        uint32_t hb[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) hb[x] = swiglu_bf16(cg, acc[hr][0][x], cu, acc[hr][1][x]);
        const u32x2 v = {hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        *(u32x2*)(so + rr * (WCH + 8) + wave * 16 + 4 * kq) = v;
      }
    }
    __syncthreads();
    const int colW = col0 - 16 * wave;
    const __amdgpu_buffer_rsrc_t ho = make_rsrc(p.h + (size_t)arow0 * p.I, nrows * p.I * 2);
    for (int u = threadIdx.x; u < nrows * LPR; u += 64 * WAVES) {
      const int row = u / LPR, c = (u % LPR) * 8;
      if (colW + c < p.I) {
        const u32x4 v = *(const u32x4*)(so + row * (WCH + 8) + c);
        store_out<ABF>(v, ho, (row * p.I + colW + c) * 2);
      }
    }
  } else {
    constexpr int WC = 16 * NS * WAVES;        // the workgroup's output columns
    constexpr int LPR = WC / 4;                // 16-byte pieces per row
    float* so = (float*)s_q;                   // [rows][WC + 4] floats (the output block)
#pragma unroll
    for (int hr = 0; hr < HR; ++hr) {
      const int rr = r + kPassRows * hr;
      if (rr < nrows) {
        // ggate: the expert's down global here; FQ: the row global just computed
        const float cf = ow[hr] * ggate * (FQ ? s_rgs[rr] : ogs[hr]);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          f32x4 v = acc[hr][s];
          if (p.c_w) {
            v[0] = v[0] * cf;
            v[1] = v[1] * cf;
            v[2] = v[2] * cf;
            v[3] = v[3] * cf;
          }
          if (s < nsv) *(f32x4*)(so + rr * (WC + 4) + wave * 16 * NS + 16 * s + 4 * kq) = v;
        }
      }
    }
    __syncthreads();
    const int colW = col0 - 16 * NS * wave;
    const __amdgpu_buffer_rsrc_t oo = make_rsrc(p.out + (size_t)arow0 * p.N, nrows * p.N * 4);
    for (int u = threadIdx.x; u < nrows * LPR; u += 64 * WAVES) {
      const int row = u / LPR, c = (u % LPR) * 4;
      if (colW + c < p.N) {
        const f32x4 v = *(const f32x4*)(so + row * (WC + 4) + c);
        store_out<ABF>(__builtin_bit_cast(u32x4, v), oo, (row * p.N + colW + c) * 4);
      }
    }
  }
}

// ------------------------------------------------------------------------- MFMA path
// The NVFP4 MFMA loop of a pass, for kernels whose waves run passes of their own (the
// decode-sized w2 launch that also sums the tokens): streams the NS weight tiles of wr
// against staged activation row rl (this lane's B column; K columns, staging area s_q /
// s_s), accumulating into acc, with the instructions of mfma_pass's NVFP4 loop (kept inline
// there: calling this from mfma_pass changed its address arithmetic and measured 0.6 us
// slower at one decode token).  The B operand of chunk c is read from LDS while chunk c - 1
// is computed (reads one chunk past the end land in the row padding, the next region or
// the slack: never used).
template <int NS, int D, int S, int WPOL, int PRIMED>
__device__ __forceinline__ void nvfp4_stream_mfma(__amdgpu_buffer_rsrc_t wr, int K, int sstride,
                                                  const uint8_t* s_q, const uint8_t* s_s, int rl,
                                                  f32x4 (&acc)[NS], Ring<NS, D>& rg) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, NC = K / 128;
  const uint8_t* aq_l = s_q + rl * q_stride(K) + 16 * kq;
  const uint8_t* as_l = s_s + rl * s_stride(K) + 2 * kq;
  u32x4 an_next = *(const u32x4*)aq_l;
  uint32_t asc_next = *(const uint16_t*)as_l;
  stream_weights_c<NS, D, S, WPOL, PRIMED>(wr, NC, sstride, 16 * lane, S * 1024 + 2 * S * lane,
                           [&](int c, int j, const u32x4 (&wn)[NS], const u32x4 (&sg)[NS]) {
    const u32x4 an = an_next;
    const uint32_t asc = asc_next;
    an_next = *(const u32x4*)(aq_l + 64 * (c + 1));
    asc_next = *(const uint16_t*)(as_l + 8 * (c + 1));
    __builtin_amdgcn_sched_barrier(0);  // issue the reads before this chunk's work
    const uint32_t sa = scale_pair_signed(asc);
    f16x8 bop[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bop[q] = dequant8(an[q], sa, q >= 2);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t sw = scale_pair_pos(sg[s][j >> 1], (j & 1) ? 0x0c030c02u : 0x0c010c00u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x8 aop = dequant8(wn[s][q], sw, q >= 2);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[q], acc[s], 0, 0, 0);
      }
    }
  }, rg);
}

// The W4A16 MFMA loop of a pass, for kernels whose waves run passes of their own (the
// decode-sized W4A16 w2 launch that also sums the tokens): streams the NS weight tiles of wr
// against staged bf16 activation row rl (K columns, staging area s_b), with the instructions
// of mfma_pass's W4A16 loop (kept inline there, as its NVFP4 loop is).
template <int NS, int D, int S, int WPOL, int PRIMED>
__device__ __forceinline__ void bf16_stream_mfma(__amdgpu_buffer_rsrc_t wr, int K, int sstride,
                                                 const uint8_t* s_b, int rl, f32x4 (&acc)[NS],
                                                 Ring<NS, D>& rg) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, NC = K / 128;
  const uint8_t* ab_l = s_b + rl * b_stride(K) + 64 * kq;
  u32x4 b_next[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) b_next[q] = *(const u32x4*)(ab_l + 16 * q);
  stream_weights_c<NS, D, S, WPOL, PRIMED>(wr, NC, sstride, 16 * lane, S * 1024 + 2 * S * lane,
                           [&](int c, int j, const u32x4 (&wn)[NS], const u32x4 (&sg)[NS]) {
    u32x4 bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bq[q] = b_next[q];
      b_next[q] = *(const u32x4*)(ab_l + 256 * (c + 1) + 16 * q);
    }
    __builtin_amdgcn_sched_barrier(0);  // issue the reads before this chunk's work
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f16x2 hs = __builtin_bit_cast(
          f16x2, scale_pair_pos(sg[s][j >> 1], (j & 1) ? 0x0c030c02u : 0x0c010c00u));
      const float f0 = (float)hs[0], f1 = (float)hs[1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 aop = dequant8_bf16(wn[s][q], q >= 2 ? f1 : f0);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, __builtin_bit_cast(bf16x8, bq[q]),
                                                         acc[s], 0, 0, 0);
      }
    }
  }, rg);
}

// One pass: stage the pass's rows, then stream NS weight tiles (wt: first tile, uniform)
// against them.  Every wave of the workgroup calls this together (it synchronizes); a
// wave with no tile in this item (nsv <= 0) loads nothing (empty buffer range) and stores
// nothing.
//
// SWI (NS == 2): the two tiles are a gate tile and the up tile I/16 tiles after it, and
// the epilogue writes h = SwiGLU(gate, up) as bf16 (ggate, gup: the expert's gate / up
// weight globals) instead of the fp32 products.  Otherwise, with p.c_w, ggate is the
// expert's down global of the scatter-ready epilogue.
//
// FQ: the pass's rows are already quantized into the staging area and their row globals
// are in s_rgs (the decode-sized GEMMs below); nothing is staged from global memory.
// PRIMED > 0 (with FQ): the caller issued the scale group and the first PRIMED chunks of
// this pass's weight ring into *ext before it quantized the rows (ring_prime<..., PRIMED>
// on pass_weights<SWI>(p, wt, nsv, .)), so that their latency overlapped the quantization.
// With FQ the barrier below waits for LDS only, leaving weight loads in flight.
template <int NS, int D, int S, bool SWI, bool ABF, int WAVES, bool FQ = false,
          int WPOL = MOE_W_CPOL, int PRIMED = 0, int APOL = 0>
__device__ __forceinline__ void mfma_pass(const GemmArgs& p, const uint8_t* __restrict__ wt,
                                          int nsv, int arow0, int nrows, int col0,
                                          uint8_t* s_q, uint8_t* s_s, float ggate, float gup,
                                          const float* s_rgs = nullptr,
                                          Ring<NS, D>* ext = nullptr) {
  static_assert(!SWI || NS == 2, "the SwiGLU epilogue pairs one gate and one up tile");
  static_assert(PRIMED == 0 || FQ, "only rows quantized in place overlap the first loads");
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, r = lane & 15;
  const int K = p.K, NC = K / 128;
  // Passes of one item load the same weight chunks; keep the compiler from hoisting those
  // loads out of the pass loop (it would hold a second copy of the ring in registers).
  if constexpr (PRIMED == 0) asm volatile("" ::: "memory");
  int sstride;
  const __amdgpu_buffer_rsrc_t wr = pass_weights<SWI>(p, wt, nsv, sstride);
  Ring<NS, D> own;
  Ring<NS, D>& rg = PRIMED > 0 ? *ext : own;
  // scatter-ready epilogue: this lane's coefficient inputs, loaded now so the epilogue
  // does not wait on them
  float ow = 0.f, ogs = 1.f;
  if (!SWI && p.c_w && r < nrows) {
    ow = p.c_w[arow0 + r];
    if (!FQ && p.c_gs) ogs = pass_row_global<APOL>(p.c_gs, arow0, nrows, r);
  }

  if constexpr (FQ) {
    // the rows were written to LDS by this workgroup's threads: wait for those writes
    // only (the primed weight loads stay in flight), then meet at the barrier; the
    // compiler barriers keep LDS accesses on their side of it
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  } else {
    stage_rows<ABF, WAVES, APOL>(p, arow0, nrows, s_q, s_s);
    __builtin_amdgcn_s_waitcnt(0);  // the staged rows have landed in LDS
    __syncthreads();
  }

  const int rl = r < nrows ? r : 0;
  f32x4 acc[1][NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) acc[0][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (ABF) {
    // W4A16: the B operand is the staged bf16 row as it is, with the weights' k
    // assignment (lane: row r; MFMA q of a chunk takes the 8 k at 32 kq + 8 q), the A
    // operand the weights dequantized exactly to bf16.
    const uint8_t* ab_l = s_q + rl * b_stride(K) + 64 * kq;
    u32x4 b_next[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) b_next[q] = *(const u32x4*)(ab_l + 16 * q);
    stream_weights_c<NS, D, S, WPOL, PRIMED>(wr, NC, sstride, 16 * lane, S * 1024 + 2 * S * lane,
                             [&](int c, int j, const u32x4 (&wn)[NS], const u32x4 (&sg)[NS]) {
      u32x4 bq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bq[q] = b_next[q];
        b_next[q] = *(const u32x4*)(ab_l + 256 * (c + 1) + 16 * q);
      }
      __builtin_amdgcn_sched_barrier(0);  // issue the reads before this chunk's work
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // the chunk's two block scales times 2^-8 (exact f16, widened exactly)
        const f16x2 hs = __builtin_bit_cast(
            f16x2, scale_pair_pos(sg[s][j >> 1], (j & 1) ? 0x0c030c02u : 0x0c010c00u));
        const float f0 = (float)hs[0], f1 = (float)hs[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x8 aop = dequant8_bf16(wn[s][q], q >= 2 ? f1 : f0);
          acc[0][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              aop, __builtin_bit_cast(bf16x8, bq[q]), acc[0][s], 0, 0, 0);
        }
      }
    }, rg);
  } else {
    const uint8_t* aq_l = s_q + rl * q_stride(K) + 16 * kq;
    const uint8_t* as_l = s_s + rl * s_stride(K) + 2 * kq;
    // The B operand of chunk c is read from LDS while chunk c - 1 is computed (reads one
    // chunk past the end land in the row padding, the next region or the slack: never used).
    u32x4 an_next = *(const u32x4*)aq_l;
    uint32_t asc_next = *(const uint16_t*)as_l;
    stream_weights_c<NS, D, S, WPOL, PRIMED>(wr, NC, sstride, 16 * lane, S * 1024 + 2 * S * lane,
                             [&](int c, int j, const u32x4 (&wn)[NS], const u32x4 (&sg)[NS]) {
      const u32x4 an = an_next;
      const uint32_t asc = asc_next;
      an_next = *(const u32x4*)(aq_l + 64 * (c + 1));
      asc_next = *(const uint16_t*)(as_l + 8 * (c + 1));
      __builtin_amdgcn_sched_barrier(0);  // issue the reads before this chunk's work
      const uint32_t sa = scale_pair_signed(asc);
      f16x8 bop[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bop[q] = dequant8(an[q], sa, q >= 2);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint32_t sw = scale_pair_pos(sg[s][j >> 1], (j & 1) ? 0x0c030c02u : 0x0c010c00u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x8 aop = dequant8(wn[s][q], sw, q >= 2);
          acc[0][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[q], acc[0][s], 0, 0, 0);
        }
      }
    }, rg);
  }

  const float ow1[1] = {ow}, ogs1[1] = {ogs};
  pass_epilogue<NS, 1, SWI, ABF, WAVES, FQ>(p, acc, nsv, arow0, nrows, col0, s_q, ggate, gup, s_rgs,
                                           ow1, ogs1);
}

// Stage K-half hf (columns [hf K/2, (hf + 1) K/2)) of NVFP4 rows arow0 .. arow0 + nrows - 1
// into LDS as rows of K/2 columns (row strides q_stride(K/2) and s_stride(K/2)).
template <int WAVES, int APOL = 0>
__device__ __forceinline__ void stage_rows_half(const GemmArgs& p, int arow0, int nrows, int hf,
                                                uint8_t* s_q, uint8_t* s_s) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qb = p.K / 2, sb = p.K / 16, hq = qb / 2, hs = sb / 2, K2 = p.K / 2;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.aq, p.a_rows * qb);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.as, p.a_rows * sb);
  for (int row = wave; row < nrows; row += WAVES) {
    const int i = arow0 + row;
    const int src = __builtin_amdgcn_readfirstlane(p.amap ? p.amap[i] : i);
    uint8_t* dq = s_q + row * q_stride(K2);
    uint8_t* ds = s_s + row * s_stride(K2);
    for (int o = 0; o < hq; o += 1024) {
      if (o + 16 * lane < hq)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_ptr_t)(dq + o), 16, 16 * lane,
                                                 src * qb + hf * hq + o, 0, APOL);
    }
    for (int o = 0; o < hs; o += 256) {
      if (o + 4 * lane < hs)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_t)(ds + o), 4, 4 * lane,
                                                 src * sb + hf * hs + o, 0, APOL);
    }
  }
}

// A double pass (NVFP4 activations, groups of more than kPassRows rows): up to kDPassRows
// rows against one stream of the NS weight tiles, the rows staged over one half of K at a
// time (the LDS of one pass of kPassRows rows over all of K), lane row r taking rows r and
// r + 16 as two B operands, each MFMA of a chunk issued once per operand.  Every output
// accumulates over the chunks in mfma_pass's order with the same instructions, so the
// results are the bits of two single passes, with the weights streamed once instead of
// twice.  Needs an even number of scale groups (K / 128 a multiple of 2 S), so that each
// half starts a scale group.  The B operands are read from LDS in the chunk that uses them
// (no read-ahead): the two operands' registers keep the instance within 128 registers per
// lane, four waves per SIMD.
template <int NS, int D, int S, bool SWI, int WAVES, int WPOL, int APOL = 0>
__device__ __forceinline__ void mfma_dpass(const GemmArgs& p, const uint8_t* __restrict__ wt,
                                           int nsv, int arow0, int nrows, int col0,
                                           uint8_t* s_q, float ggate, float gup) {
  static_assert(!SWI || NS == 2, "the SwiGLU epilogue pairs one gate and one up tile");
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, r = lane & 15;
  const int K2 = p.K / 2, NC2 = p.K / 256;
  uint8_t* s_s = s_q + kDPassRows * q_stride(K2);
  asm volatile("" ::: "memory");  // (as in mfma_pass: no loads hoisted across passes)
  int sstride;
  const int tstride = (p.K / 128) * kChunkBytes;
  sstride = SWI ? (p.I / 16) * tstride : tstride;
  const int range = nsv <= 0 ? 0 : SWI ? sstride + tstride : nsv * tstride;
  const int hoff = (NC2 / S) * S * kChunkBytes;  // the second half: its first scale group
  float ow[2] = {0.f, 0.f}, ogs[2] = {1.f, 1.f};
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
    const int rr = r + kPassRows * hr;
    if (!SWI && p.c_w && rr < nrows) {
      ow[hr] = p.c_w[arow0 + rr];
      if (p.c_gs) ogs[hr] = pass_row_global<APOL>(p.c_gs, arow0, nrows, rr);
    }
  }
  // lanes past the pass's rows read row 0: their B columns only feed rows not stored
  const int rl0 = r < nrows ? r : 0;
  const int rl1 = r + kPassRows < nrows ? r + kPassRows : 0;
  f32x4 acc[2][NS];
#pragma unroll
  for (int hr = 0; hr < 2; ++hr)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[hr][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int hf = 0; hf < 2; ++hf) {
    if (hf) __syncthreads();  // every wave is done with the first half's rows
    stage_rows_half<WAVES, APOL>(p, arow0, nrows, hf, s_q, s_s);
    __builtin_amdgcn_s_waitcnt(0);  // the staged rows have landed in LDS
    __syncthreads();
    const int hrange = range == 0 ? 0 : hf ? range - hoff : range;
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(wt + (hf ? hoff : 0), __builtin_amdgcn_readfirstlane(hrange));
    Ring<NS, D> rg;
    const uint8_t* aq0 = s_q + rl0 * q_stride(K2) + 16 * kq;
    const uint8_t* aq1 = s_q + rl1 * q_stride(K2) + 16 * kq;
    const uint8_t* as0 = s_s + rl0 * s_stride(K2) + 2 * kq;
    const uint8_t* as1 = s_s + rl1 * s_stride(K2) + 2 * kq;
    stream_weights_c<NS, D, S, WPOL>(wr, NC2, sstride, 16 * lane, S * 1024 + 2 * S * lane,
                             [&](int c, int j, const u32x4 (&wn)[NS], const u32x4 (&sg)[NS]) {
      const u32x4 an0 = *(const u32x4*)(aq0 + 64 * c), an1 = *(const u32x4*)(aq1 + 64 * c);
      const uint32_t sa0 = scale_pair_signed(*(const uint16_t*)(as0 + 8 * c));
      const uint32_t sa1 = scale_pair_signed(*(const uint16_t*)(as1 + 8 * c));
      uint32_t sw[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        sw[s] = scale_pair_pos(sg[s][j >> 1], (j & 1) ? 0x0c030c02u : 0x0c010c00u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x8 b0 = dequant8(an0[q], sa0, q >= 2);
        const f16x8 b1 = dequant8(an1[q], sa1, q >= 2);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f16x8 aop = dequant8(wn[s][q], sw[s], q >= 2);
          acc[0][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, b0, acc[0][s], 0, 0, 0);
          acc[1][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, b1, acc[1][s], 0, 0, 0);
        }
      }
    }, rg);
  }
  pass_epilogue<NS, 2, SWI, false, WAVES, false>(p, acc, nsv, arow0, nrows, col0, s_q, ggate,
                                                 gup, nullptr, ow, ogs);
}

// Item ii (of items_per_item(p)) of group g: the tiles [ii * per_item, (ii + 1) * per_item)
// of the group's weights against all of its rows.  PR: activation rows staged per pass (at
// most the B operand's 16 columns).  Groups of more than PR rows take double passes where
// they can (mfma_dpass).  APOL: cache policy of the activation loads.
template <bool SWI, int NS, int WAVES>
__host__ __device__ __forceinline__ int item_tiles(const GemmArgs& p) {
  return SWI ? p.I / 16 : p.N / 16;  // SWI: a wave owns one gate tile (and its up tile)
}
template <bool SWI, int NS, int WAVES>
__host__ __device__ __forceinline__ int items_per_group(const GemmArgs& p) {
  constexpr int per_item = SWI ? WAVES : WAVES * NS;
  return (item_tiles<SWI, NS, WAVES>(p) + per_item - 1) / per_item;
}

template <int NS, int D, int S, bool SWI, bool ABF, int WAVES, int PR, int APOL = 0>
__device__ __forceinline__ void run_item(const GemmArgs& p, int ii, const ItemGroup& g,
                                         uint8_t* smem) {
  uint8_t* s_q = smem;
  uint8_t* s_s = s_q + PR * q_stride(p.K);  // NVFP4 scales (unused with ABF)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles = item_tiles<SWI, NS, WAVES>(p);
  constexpr int per_item = SWI ? WAVES : WAVES * NS;
  const int t0 = ii * per_item + wave * (SWI ? 1 : NS);
  const int nsv = SWI ? (t0 < tiles ? 2 : 0) : min(NS, tiles - t0);
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  const uint8_t* wt = p.w + (size_t)g.e * expert_bytes + (size_t)(nsv > 0 ? t0 : 0) * tile_bytes;
  const float ggate = SWI ? p.g_gate[g.e] : p.c_w ? p.c_g[g.e] : 0.f;
  const float gup = SWI ? p.g_up[g.e] : 0.f;
  if (g.G > PR) {  // uniform: several passes over the same weights
    int b = 0;
    if constexpr (!ABF && PR == kPassRows) {
      // double passes while more than one pass's rows remain (an even number of scale
      // groups; uniform)
      if ((p.K / 128) % (2 * S) == 0) {
        for (; g.G - b > PR; b += kDPassRows) {
          if (b) __syncthreads();  // the previous pass is done with the staged rows
          mfma_dpass<NS, D, S, SWI, WAVES, kMultiPassWCpol, APOL>(
              p, wt, nsv, g.r0 + b, min(kDPassRows, g.G - b), 16 * t0, s_q, ggate, gup);
        }
      }
    }
    for (; b < g.G; b += PR) {
      if (b) __syncthreads();  // the previous pass is done with the staged rows
      mfma_pass<NS, D, S, SWI, ABF, WAVES, false, kMultiPassWCpol, 0, APOL>(
          p, wt, nsv, g.r0 + b, min(PR, g.G - b), 16 * t0, s_q, s_s, ggate, gup);
    }
    return;
  }
  for (int b = 0; b < g.G; b += PR) {
    if (b) __syncthreads();  // the previous pass is done with the staged rows
    mfma_pass<NS, D, S, SWI, ABF, WAVES, false, MOE_W_CPOL, 0, APOL>(
        p, wt, nsv, g.r0 + b, min(PR, g.G - b), 16 * t0, s_q, s_s, ggate, gup);
  }
}

// One workgroup per item: item it is item it % items_per_e of active group it / items_per_e.
// The grid has one item slot per group that can be non-empty, so every item has a
// workgroup and no workgroup has two.  The waves-per-SIMD hint keeps the 4-chunk-ring
// NVFP4 instances at four waves per SIMD with the double pass's registers (without it they
// compile to three).
template <int NS, int D, int S, bool SWI, bool ABF, int WAVES, int PR>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(ABF || D > 4 ? 1 : 4)))
void k_gemm_mfma(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_grp[4];
  const int items_per_e = items_per_group<SWI, NS, WAVES>(p);
  const int item = blockIdx.x;
  ItemGroup g;
  if (!find_group<PR>(p, item / items_per_e, s_grp, g)) return;  // uniform
  run_item<NS, D, S, SWI, ABF, WAVES, PR>(p, item % items_per_e, g, smem);
}

// ------------------------------------------------------------------------- fused layer
// The layer's w13 GEMM (SwiGLU epilogue), the NVFP4 quantization of h and the w2 GEMM
// (scatter-ready epilogue) in one launch, for batches of more than 32 assignments.  The grid
// is three ranges, each in the work list's order: [0, n13) the w13 items, then one
// quantization workgroup per group, then the w2 items.  A w13 item raises its own flag once
// its part of h is written; a group's quantization workgroup waits for the flags of the
// group's w13 items, quantizes the group's rows of h and raises the group's flag; a w2
// item waits for that flag.  So the w2 items fill the slots that the w13 GEMM's last round
// leaves free, and the quantization runs in that round too, instead of as a launch of its
// own between the two GEMMs.
//
// Why it cannot deadlock: workgroups are dispatched in index order (per XCD), so a waiting
// workgroup was dispatched after every workgroup it waits for (all earlier in the grid), and
// the w13 items wait for nothing; every wait is bounded regardless (kSyncSpinMax polls, then
// the error bit MOE_ERR_SYNC and no further waiting).
//
// Visibility without cache maintenance: h, hq, hs, hgs and the flags are written with
// device-scope stores (through the L2) and read with device-scope loads, and a writer waits
// for its stores to complete before it raises its flag (one thread, after a barrier).
// Plain flag stores, one word per item: measured on MI355X, one device-scope atomic add
// per w13 item (a counter per group, the last item quantizing) made the layer 12-14%
// slower, with or without using the returned value, while the wait for the stores costs
// nothing measurable.  The arithmetic of every output is k_gemm_mfma's and k_quantize's, so
// the results are the bits of the separate launches.
struct LayerSync {
  int n13;         // workgroups of the w13 GEMM: `groups` slots of n13 / groups items each
  int groups;      // group slots (min(E, R)); kQuantParts quantization workgroups each
                   // follow the w13 range, then the w2 GEMM's workgroups
  int* done13;     // [n13] nonzero once w13 item slot b has written its part of h
  int* ready;      // [kQuantParts x groups]: entry kQuantParts a + j nonzero once part j
                   // of group a is quantized
  int32_t* err;    // device error word
  uint8_t* hq;     // NVFP4 h: codes [R, I/2], scales [R, I/16], row globals [R]
  uint8_t* hs;
  float* hgs;
};
constexpr int kSyncSpinMax = 1 << 19;

// Lane l < n of wave 0: flags[l], read at device scope (1 elsewhere).  Issued at the start
// of a workgroup, so that its latency overlaps the work list lookup.
__device__ __forceinline__ int load_flags(const int* flags, int n) {
  const int lane = threadIdx.x & 63;
  return threadIdx.x < 64 && lane < n
             ? __hip_atomic_load(flags + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
}

// Wave 0 waits until the n flags at flags[0 .. n) (n <= 64; v: load_flags's first read)
// are all nonzero, polling with device-scope loads; gives up after kSyncSpinMax polls and
// sets MOE_ERR_SYNC.  The workgroup meets at a barrier afterwards.
__device__ __forceinline__ void wait_flags(int v, const int* flags, int n, int32_t* err) {
  if (threadIdx.x < 64) {
    bool done = __ballot(v == 0) == 0ull;
    for (int k = 0; !done && k < kSyncSpinMax; ++k) {
      __builtin_amdgcn_s_sleep(8);
      done = __ballot(load_flags(flags, n) == 0) == 0ull;
    }
    if (!done && threadIdx.x == 0)
      __hip_atomic_fetch_or(err, MOE_ERR_SYNC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  asm volatile("" ::: "memory");
}

// Once every store of this workgroup has completed: flag = 1 (device scope).
__device__ __forceinline__ void raise_flag(int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct RowStoreDevice {
  __amdgpu_buffer_rsrc_t q, sc, gs;
  __device__ __forceinline__ void codes(int b, const u32x2& v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, q, 8 * b, 0, kDeviceScope);
  }
  __device__ __forceinline__ void scale(int b, uint32_t sb) {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, sc, b, 0, kDeviceScope);
  }
  __device__ __forceinline__ void global(float g) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, g), gs, 0, 0, kDeviceScope);
  }
};

// Part j of the quantization of a group's rows r0 .. r0 + G - 1 of h (bf16, I columns) to
// NVFP4: the 16-row blocks j, j + kQuantParts, ... of the group, one row per wave at a time
// (lane l: scale blocks l + 64 k, k < BPT), with k_quantize's arithmetic.
constexpr int kQuantParts = 4;
template <int BPT>
__device__ __forceinline__ void quantize_h_rows(const uint16_t* h, int I, int r0, int G, int j,
                                                const LayerSync& f) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NB = I / 16;
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(h + (size_t)r0 * I, G * I * 2);
  for (int b0 = 16 * j; b0 < G; b0 += 16 * kQuantParts)
  for (int row = b0 + wave; row < min(G, b0 + 16); row += kGemmWaves) {
    float v[BPT][16];
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int blk = lane + 64 * k;
      u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
      if (blk < NB) {
        w0 = __builtin_amdgcn_raw_buffer_load_b128(hr, (row * I + 16 * blk) * 2, 0, kDeviceScope);
        w1 = __builtin_amdgcn_raw_buffer_load_b128(hr, (row * I + 16 * blk) * 2 + 16, 0,
                                                   kDeviceScope);
      }
      bf16x16_to_f32(w0, w1, v[k]);
    }
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < BPT; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, __builtin_fabsf(v[k][e]));
    const float amax = wave_max(m);
    const int i = r0 + row;
    RowStoreDevice st{make_rsrc(f.hq + (size_t)i * (I / 2), I / 2),
                      make_rsrc(f.hs + (size_t)i * NB, NB), make_rsrc(f.hgs + i, 4)};
    quantize_row_emit<BPT>(v, NB, lane, 64, amax, st);
  }
}

// D13, NS2, D2: the w13 GEMM's ring depth and the w2 GEMM's tiles per wave and ring depth,
// those of the separate launches' instances for the same grid (large: 4, 2, 4; small:
// 8, 1, 8).
template <int D13, int NS2, int D2, int S, int BPT>
__global__ __launch_bounds__(64 * kGemmWaves)
__attribute__((amdgpu_waves_per_eu(D13 > 4 ? 1 : 4)))
void k_gemm_layer(GemmArgs p13, GemmArgs p2, LayerSync f) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_grp[4];
  ItemGroup g;
  const int b = blockIdx.x;
  const int ipe13 = items_per_group<true, 2, kGemmWaves>(p13);
  if (b < f.n13) {  // uniform: a w13 item
    if (!find_group<kPassRows>(p13, b / ipe13, s_grp, g)) return;  // uniform
    run_item<2, D13, S, true, false, kGemmWaves, kPassRows>(p13, b % ipe13, g, smem);
    raise_flag(f.done13 + b);
    return;
  }
  if (b < f.n13 + kQuantParts * f.groups) {  // uniform: part j of group a's quantization
    const int a = (b - f.n13) / kQuantParts, j = (b - f.n13) % kQuantParts;
    const int v = load_flags(f.done13 + a * ipe13, ipe13);
    if (!find_group<kPassRows>(p13, a, s_grp, g)) return;  // uniform
    if (16 * j < g.G) {  // uniform
      wait_flags(v, f.done13 + a * ipe13, ipe13, f.err);
      quantize_h_rows<BPT>(p13.h, p13.I, g.r0, g.G, j, f);
    }
    raise_flag(f.ready + b - f.n13);
    return;
  }
  // a w2 item
  const int ipe2 = items_per_group<false, NS2, kGemmWaves>(p2);
  const int item = b - f.n13 - kQuantParts * f.groups;
  const int* ready = f.ready + kQuantParts * (item / ipe2);
  const int v = load_flags(ready, kQuantParts);
  if (!find_group<kPassRows>(p2, item / ipe2, s_grp, g)) return;  // uniform
  wait_flags(v, ready, kQuantParts, f.err);
  run_item<NS2, D2, S, false, false, kGemmWaves, kPassRows, kDeviceScope>(p2, item % ipe2, g,
                                                                          smem);
}

// ------------------------------------------------------------------------- decode w13
// A batch of at most kSmallGroupRows expert-rows (decode): the w13 GEMM with the SwiGLU
// epilogue, every workgroup grouping the assignments itself with one wave (the one-wave
// grouping's order) and quantizing its group's source rows straight into its staging area
// with the grouping launch's quantizer, so the layer needs no grouping launch before this
// one.  One extra workgroup writes the grouping's outputs for the later kernels.  The items,
// passes and arithmetic are those of k_gemm_mfma's small-batch SwiGLU instance, so the
// results are the same bits.  Workgroup ai / items_per_e takes the ai-th expert with rows
// in ascending id (no multi-pass-first order: that only changes which workgroup computes
// what).
constexpr int kSmallGroupRows = 32;

// Quantize nrows bf16 rows of K columns (K <= 4096 BPT, BPT 16-element blocks per thread;
// RPS rows' loads in flight at a time; row_ptr(r): row r's first element, nullptr: an
// all-zero row) into the staging area, row r at s_q + r q_stride(K) / s_s + r s_stride(K)
// and its row global at s_rgs[r], with the quantizer of the row kernels (every thread of
// the workgroup takes part).  after_first_loads() runs
// once, after the first rows' loads are issued and before they are waited for (the caller
// issues its first weight loads there, so that their latency overlaps the quantization;
// loads complete in order, so they must come after the rows' loads).  PRE: pre holds this
// thread's BPT blocks of a row the caller loaded already, used for every row (all rows the
// same source row; otherwise pre is not read).  The caller synchronizes before the staged
// rows are read.
template <int BPT, int RPS, bool PRE = false, class RowPtr, class AfterLoads>
__device__ __forceinline__ void quantize_rows_to_lds(RowPtr row_ptr, int nrows, int K,
                                                     uint8_t* s_q, uint8_t* s_s, float* s_rgs,
                                                     float* s_red, AfterLoads after_first_loads,
                                                     const u32x4 (&pre)[BPT][2]) {
  constexpr int NT = 64 * kGemmWaves;  // threads per row: block b = t + NT k of each row
  const int NB = K / 16, t = threadIdx.x;
  for (int r = 0; r < nrows; r += RPS) {
    u32x4 w[RPS][BPT][2];
#pragma unroll
    for (int rr = 0; rr < RPS; ++rr) {
      const uint16_t* src = r + rr < nrows ? row_ptr(r + rr) : nullptr;
#pragma unroll
      for (int k = 0; k < BPT; ++k) {
        const int blk = t + NT * k;
        w[rr][k][0] = w[rr][k][1] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (PRE) {  // every row is the one whose blocks the caller loaded
          w[rr][k][0] = pre[k][0];
          w[rr][k][1] = pre[k][1];
        } else if (src && blk < NB) {
          const u32x4* px = (const u32x4*)(src + 16 * blk);
          w[rr][k][0] = px[0];
          w[rr][k][1] = px[1];
        }
      }
    }
    if (r == 0) {  // uniform: after the first rows' loads, before they are waited for
      __builtin_amdgcn_sched_barrier(0);
      after_first_loads();
      __builtin_amdgcn_sched_barrier(0);
    }
    float v[RPS][BPT][16];
#pragma unroll
    for (int rr = 0; rr < RPS; ++rr)
#pragma unroll
      for (int k = 0; k < BPT; ++k) bf16x16_to_f32(w[rr][k][0], w[rr][k][1], v[rr][k]);
#pragma unroll
    for (int rr = 0; rr < RPS; ++rr) {
      // every thread joins the row-max barrier; only real rows store
      // (consecutive rows alternate between two slots of s_red: a slot is rewritten only
      // after the barrier of the next row, which every wave reaches after its reads)
      const float amax = row_amax_threads<BPT>(v[rr], t, NT, s_red + ((r + rr) & 1) * kGemmWaves);
      if (r + rr < nrows)
        quantize_row_store<BPT>(v[rr], NB, t, NT, amax, s_q + (r + rr) * q_stride(K),
                                s_s + (r + rr) * s_stride(K), s_rgs + r + rr);
    }
  }
}

template <int BPT, int RPS, class RowPtr, class AfterLoads>
__device__ __forceinline__ void quantize_rows_to_lds(RowPtr row_ptr, int nrows, int K,
                                                     uint8_t* s_q, uint8_t* s_s, float* s_rgs,
                                                     float* s_red, AfterLoads after_first_loads) {
  const u32x4 none[BPT][2] = {};
  quantize_rows_to_lds<BPT, RPS, false>(row_ptr, nrows, K, s_q, s_s, s_rgs, s_red,
                                        after_first_loads, none);
}

struct GroupArgs {
  const int32_t* a_expert;
  const int32_t* a_src;
  const int32_t* a_dst;
  const float* a_w;
  int R, S, T;
  const uint16_t* x;  // source rows [S, K] bf16
  int32_t* offsets;
  int32_t* row_src;
  int32_t* row_dst;
  float* row_w;
  int32_t* tok_off;
  int32_t* tok_rows;
  int32_t* err;
  int4* items;  // the grouped GEMMs' work list for the later launches (or nullptr)
};

// ABF (W4A16): the source rows are bf16 activations used as they are (copied into the
// staging area, row global 1), in passes of 4 rows like the small-batch W4A16 instance.
template <int D, int S, bool ABF, int BPT, bool PRE = false>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm_swiglu_grouping(GemmArgs p, GroupArgs q) {
  constexpr int PR = ABF ? 4 : kPassRows;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_grp[4];
  __shared__ int s_src[kSmallGroupRows];    // source rows of the group's grouped rows
  __shared__ float s_rgs[kPassRows];        // row globals of the pass's rows
  __shared__ float s_red[2 * kGemmWaves];   // row-max partials of two rows
  uint8_t* s_q = smem;
  uint8_t* s_s = s_q + PR * q_stride(p.K);  // NVFP4 scales (unused with ABF)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles = p.I / 16, per_item = kGemmWaves;
  const int items_per_e = (tiles + per_item - 1) / per_item;
  const int ai = blockIdx.x / items_per_e;
  // PRE (one source row, a single decode token; NVFP4): every grouped row is that row, so
  // its blocks are loaded now and arrive while wave 0 groups.  A separate instance: the
  // registers they hold would cost the general one a wave per SIMD.
  static_assert(!PRE || !ABF, "the prefetch feeds the NVFP4 quantization");
  u32x4 xpre[BPT][2];
  if constexpr (PRE) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int blk = threadIdx.x + 64 * kGemmWaves * k;
      xpre[k][0] = xpre[k][1] = u32x4{0u, 0u, 0u, 0u};
      if (blk < p.K / 16) {
        const u32x4* px = (const u32x4*)(q.x + 16 * blk);
        xpre[k][0] = px[0];
        xpre[k][1] = px[1];
      }
    }
  }
  if (blockIdx.x == gridDim.x - 1) {
    // the launch's extra workgroup: the grouping's outputs for the later launches (the
    // offsets, row maps and token lists, and the work list), off the items' path (measured
    // on MI355X: a workgroup that also did this ended about 1 us after the others)
    group_small(q.a_expert, q.a_src, q.a_dst, q.a_w, q.R, p.E, q.S, q.T, q.offsets, q.row_src,
                q.row_dst, q.row_w, q.tok_off, q.tok_rows, q.err, q.items);
    return;
  }
  if (wave == 0) {
    // grouped position of lane j's assignment: the number of (key, index) pairs below its
    // own (the counting loop with every lane active, as in group_small)
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const bool act = lane < q.R;
    int e = 0, sr = 0, d = 0;
    if (act) {
      e = q.a_expert[lane];
      sr = q.a_src[lane];
      d = q.a_dst[lane];
    }
    const bool valid = act && e >= 0 && e < p.E && sr >= 0 && sr < q.S && d >= 0 && d < q.T;
    const int key = act ? (valid ? e : p.E) : 0x7FFFFFFF;
    int rank = 0;
    for (int k = 0; k < q.R; ++k) {
      const int kk = __builtin_amdgcn_readlane(key, k);
      rank += (kk < key || (kk == key && k < lane)) ? 1 : 0;
    }
    const int pos = act ? rank : lane;
    const int skey = __builtin_amdgcn_ds_permute(4 * pos, key);  // lane p: key at position p
    const int ssrc = __builtin_amdgcn_ds_permute(4 * pos, sr);
    const int prev = __shfl_up(skey, 1, 64);
    const bool first = skey < p.E && (lane == 0 || prev != skey);  // a group starts at lane
    const uint64_t m = __ballot(first);
    const uint64_t sel = __ballot(first && __popcll(m & below) == ai);
    const bool found = sel != 0ull;  // uniform
    if (found) {
      const int r0 = __builtin_ctzll(sel);
      const int eg = __builtin_amdgcn_readlane(skey, r0);
      const int G = __popcll(__ballot(skey == eg));
      if (lane >= r0 && lane < r0 + G) s_src[lane - r0] = ssrc;
      if (lane == 0) {
        s_grp[0] = eg;
        s_grp[1] = r0;
        s_grp[2] = G;
      }
    }
    if (lane == 0) s_grp[3] = found ? 1 : 0;
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(s_grp[3]) == 0) return;  // uniform
  const int eg = __builtin_amdgcn_readfirstlane(s_grp[0]);
  const int r0 = __builtin_amdgcn_readfirstlane(s_grp[1]);
  const int G = __builtin_amdgcn_readfirstlane(s_grp[2]);
  const int t0 = (blockIdx.x % items_per_e) * per_item + wave;
  const int nsv = t0 < tiles ? 2 : 0;
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  const uint8_t* wt = p.w + (size_t)eg * expert_bytes + (size_t)(nsv > 0 ? t0 : 0) * tile_bytes;
  const float ggate = p.g_gate[eg], gup = p.g_up[eg];
  // NVFP4: the first pass's weight loads go out while its rows are being quantized
  Ring<2, D> rg;
  int sstride;
  const __amdgpu_buffer_rsrc_t wr = pass_weights<true>(p, wt, nsv, sstride);
  for (int b = 0; b < G; b += PR) {
    if (b) __syncthreads();  // the previous pass is done with the staged rows
    const int nrows = min(PR, G - b);
    if constexpr (ABF) {
      const int pieces = p.K / 8;  // 16-byte pieces of a bf16 row
      for (int u = threadIdx.x; u < nrows * pieces; u += 64 * kGemmWaves) {
        const int r = u / pieces, c = u - r * pieces;
        const u32x4 v = *(const u32x4*)(q.x + (size_t)s_src[b + r] * p.K + 8 * c);
        *(u32x4*)(s_q + r * b_stride(p.K) + 16 * c) = v;
      }
      if (threadIdx.x < nrows) s_rgs[threadIdx.x] = 1.0f;
      mfma_pass<2, D, S, true, ABF, kGemmWaves, true>(p, wt, nsv, r0 + b, nrows, 16 * t0, s_q,
                                                      s_s, ggate, gup, s_rgs);
    } else {
      auto rows = [&](int r) { return q.x + (size_t)s_src[b + r] * p.K; };
      if (b == 0) {  // one row at a time here: the ring's registers are live
        // (half the ring; issuing all of it here measured 0.9 us slower at one token)
        constexpr int P = D / 2 > 0 ? D / 2 : 1;
        auto prime = [&] {
          ring_prime<2, D, S, MOE_W_CPOL, P>(rg, wr, sstride, 16 * lane, S * 1024 + 2 * S * lane);
        };
        if constexpr (PRE)
          quantize_rows_to_lds<BPT, 1, true>(rows, nrows, p.K, s_q, s_s, s_rgs, s_red, prime, xpre);
        else
          quantize_rows_to_lds<BPT, 1>(rows, nrows, p.K, s_q, s_s, s_rgs, s_red, prime);
        mfma_pass<2, D, S, true, false, kGemmWaves, true, MOE_W_CPOL, P>(
            p, wt, nsv, r0 + b, nrows, 16 * t0, s_q, s_s, ggate, gup, s_rgs, &rg);
      } else {
        quantize_rows_to_lds<BPT, 2>(rows, nrows, p.K, s_q, s_s, s_rgs, s_red, [] {});
        mfma_pass<2, D, S, true, false, kGemmWaves, true>(p, wt, nsv, r0 + b, nrows, 16 * t0,
                                                          s_q, s_s, ggate, gup, s_rgs);
      }
    }
  }
}

// A batch of at most kSmallGroupRows expert-rows: the w2 GEMM with the scatter-ready
// epilogue, each workgroup quantizing its group's rows of h (bf16, grouped order) straight
// into its staging area with the quantizer of the row kernels, so the layer needs no
// quantization launch between the two GEMMs; the scatter coefficient takes the row global
// it has just computed.  Items, passes and arithmetic are those of k_gemm_mfma's
// small-batch instance: the same bits.
template <int D, int S, int BPT, bool PRE = false>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm_quantizing(GemmArgs p,
                                                                     const uint16_t* __restrict__ h) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_grp[4];
  __shared__ float s_rgs[kPassRows];
  __shared__ float s_red[2 * kGemmWaves];
  uint8_t* s_q = smem;
  uint8_t* s_s = s_q + kPassRows * q_stride(p.K);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles = p.N / 16, per_item = kGemmWaves;  // one tile per wave
  const int items_per_e = (tiles + per_item - 1) / per_item;
  const int ai = blockIdx.x / items_per_e;
  // PRE (one source row, a single decode token): its experts are distinct as a rule, so
  // every group is one row and group ai is grouped row ai; that row's blocks are loaded
  // before the group is known and used if the group proves to be that row.  A separate
  // instance, for the registers they hold (as in k_gemm_swiglu_grouping).
  u32x4 hpre[BPT][2];
  if constexpr (PRE) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int blk = threadIdx.x + 64 * kGemmWaves * k;
      hpre[k][0] = hpre[k][1] = u32x4{0u, 0u, 0u, 0u};
      if (ai < p.a_rows && blk < p.K / 16) {
        const u32x4* px = (const u32x4*)(h + (size_t)ai * p.K + 16 * blk);
        hpre[k][0] = px[0];
        hpre[k][1] = px[1];
      }
    }
  }
  ItemGroup g;
  if (!find_group<kPassRows>(p, ai, s_grp, g)) return;  // uniform
  const int t0 = (blockIdx.x % items_per_e) * per_item + wave;
  const int nsv = min(1, tiles - t0);
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  const uint8_t* wt = p.w + (size_t)g.e * expert_bytes + (size_t)(nsv > 0 ? t0 : 0) * tile_bytes;
  const float gdown = p.c_g[g.e];
  // the first pass's weight loads go out while its rows of h are being quantized
  const int lane = threadIdx.x & 63;
  Ring<1, D> rg;
  int sstride;
  const __amdgpu_buffer_rsrc_t wr = pass_weights<false>(p, wt, nsv, sstride);
  for (int b = 0; b < g.G; b += kPassRows) {
    if (b) __syncthreads();  // the previous pass is done with the staged rows
    const int nrows = min(kPassRows, g.G - b);
    const int row0 = g.r0 + b;
    auto rows = [&](int r) { return h + (size_t)(row0 + r) * p.K; };
    if (b == 0) {  // one row at a time here: the ring's registers are live
      auto prime = [&] {
        ring_prime<1, D, S, MOE_W_CPOL>(rg, wr, sstride, 16 * lane, S * 1024 + 2 * S * lane);
      };
      if (PRE && g.G == 1 && g.r0 == ai)  // uniform: the row loaded at entry is the group's
        quantize_rows_to_lds<BPT, 1, true>(rows, nrows, p.K, s_q, s_s, s_rgs, s_red, prime, hpre);
      else
        quantize_rows_to_lds<BPT, 1>(rows, nrows, p.K, s_q, s_s, s_rgs, s_red, prime);
      mfma_pass<1, D, S, false, false, kGemmWaves, true, MOE_W_CPOL, D>(
          p, wt, nsv, row0, nrows, 16 * t0, s_q, s_s, gdown, 0.f, s_rgs, &rg);
    } else {
      quantize_rows_to_lds<BPT, 2>(rows, nrows, p.K, s_q, s_s, s_rgs, s_red, [] {});
      mfma_pass<1, D, S, false, false, kGemmWaves, true>(p, wt, nsv, row0, nrows, 16 * t0, s_q,
                                                         s_s, gdown, 0.f, s_rgs);
    }
  }
}

// A batch of at most WV expert-rows (one or two decode tokens): the w2 GEMM and the per-token
// sum in one launch.  Workgroup c owns output columns 16 c .. 16 c + 15 of every token:
// wave w takes group w of the work list (one 16-row tile of that expert's w2 weights,
// streamed over all of K), quantizes the group's rows of h into the staging area itself,
// and puts each row's scatter term (the product times row_w[i] * g_down[e] * hgs[i], in
// the order of the scatter-ready epilogue) into LDS; after one barrier the workgroup sums
// each token's terms as the per-token sum does (eight interleaved partial sums over the
// token's list, added in order 0..7) and writes the token's 16 bf16 outputs.  No term
// goes through global memory and there is no third launch.  A wave quantizes its rows
// alone (the row maximum by a wave reduction); every product, term and sum is the
// operation the separate launches perform, so the output has the same bits.
struct TokenSumArgs {
  const int32_t* tok_off;   // [T + 1]
  const int32_t* tok_rows;  // grouped rows of token t: tok_rows[tok_off[t] .. tok_off[t + 1])
  int T;
  uint16_t* out;            // [T, N] bf16
};
constexpr int kSumTokLds = 64;  // tokens whose list offsets are read into LDS at entry

template <int WV, int D, int S, int BPT>
__global__ __launch_bounds__(64 * WV) void k_gemm_quantizing_sum(GemmArgs p,
                                                                 const uint16_t* __restrict__ h,
                                                                 TokenSumArgs ts) {
  static_assert(WV == 8 || WV == 16, "a power of two of at most 16 waves");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float s_rgs[WV];       // row globals of the grouped rows
  __shared__ f32x4 s_term[WV][4];   // scatter terms: [grouped row][4 columns x 4]
  __shared__ int s_rows[WV];        // the token lists
  __shared__ int s_off[kSumTokLds + 1];
  const int K = p.K, R = p.a_rows, NB = K / 16;
  uint8_t* s_q = smem;                      // [WV rows][q_stride(K)]
  uint8_t* s_s = s_q + WV * q_stride(K);    // [WV rows][s_stride(K)], then 256 bytes of slack
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x;
  // grouped row `wave` of h, loaded before the work list arrives: when every group is one
  // row (distinct experts, the rule for one token), group `wave` is that row
  u32x4 hpre[BPT][2];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int blk = lane + 64 * k;
    hpre[k][0] = hpre[k][1] = u32x4{0u, 0u, 0u, 0u};
    if (wave < R && blk < NB) {
      const u32x4* px = (const u32x4*)(h + (size_t)wave * K + 16 * blk);
      hpre[k][0] = px[0];
      hpre[k][1] = px[1];
    }
  }
  // the token lists, for the sum at the end (put into LDS after the GEMM, so that no wave
  // waits for them before its weight loads)
  const int tr = threadIdx.x < R ? ts.tok_rows[threadIdx.x] : 0;
  const int to = threadIdx.x <= min(ts.T, kSumTokLds) ? ts.tok_off[threadIdx.x] : 0;
  // this wave's group: work list entry `wave` (ascending expert id; R <= WV <= 16 rows, so
  // no group takes a second pass)
  int4 it = int4{0, 0, 0, 0};
  if (wave < R && wave < p.E) it = p.items[1 + wave];
  const int ng = __builtin_amdgcn_readfirstlane(p.items[0].x);
  const bool has = wave < ng;  // uniform
  const int e = has ? __builtin_amdgcn_readfirstlane(it.x) : 0;
  const int r0 = has ? __builtin_amdgcn_readfirstlane(it.y) : 0;
  const int G = has ? __builtin_amdgcn_readfirstlane(it.z) : 0;
  const size_t expert_bytes = (size_t)p.N * K / 16 * 9;
  const uint8_t* wt = p.w + (size_t)e * expert_bytes + (size_t)tile * 9 * K;
  int sstride;
  const __amdgpu_buffer_rsrc_t wr = pass_weights<false>(p, wt, has ? 1 : 0, sstride);
  Ring<1, D> rg;
  float ow = 0.f, gdown = 0.f;
  const int kq = lane >> 4, rr = lane & 15;
  if (has) {
    ring_prime<1, D, S, MOE_W_CPOL>(rg, wr, sstride, 16 * lane, S * 1024 + 2 * S * lane);
    gdown = p.c_g[e];
    if (rr < G) ow = p.c_w[r0 + rr];
    // the group's rows of h, quantized by this wave alone
    for (int r = 0; r < G; ++r) {
      const int i = r0 + r;
      u32x4 w[BPT][2];
      const bool pre = G == 1 && r0 == wave;  // uniform: the row loaded at entry
#pragma unroll
      for (int k = 0; k < BPT; ++k) {
        const int blk = lane + 64 * k;
        w[k][0] = hpre[k][0];
        w[k][1] = hpre[k][1];
        if (!pre) {
          w[k][0] = w[k][1] = u32x4{0u, 0u, 0u, 0u};
          if (blk < NB) {
            const u32x4* px = (const u32x4*)(h + (size_t)i * K + 16 * blk);
            w[k][0] = px[0];
            w[k][1] = px[1];
          }
        }
      }
      float v[BPT][16];
#pragma unroll
      for (int k = 0; k < BPT; ++k) bf16x16_to_f32(w[k][0], w[k][1], v[k]);
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < BPT; ++k)
#pragma unroll
        for (int x = 0; x < 16; ++x) m = fmaxf(m, __builtin_fabsf(v[k][x]));
      const float amax = wave_max(m);
      quantize_row_store<BPT>(v, NB, lane, 64, amax, s_q + i * q_stride(K), s_s + i * s_stride(K),
                              s_rgs + i);
    }
    // this wave's LDS writes have landed (its weight loads stay in flight)
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
    // lanes past the group's rows read its first row: their B columns feed no term
    const int rl = r0 + (rr < G ? rr : 0);
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    nvfp4_stream_mfma<1, D, S, MOE_W_CPOL, D>(wr, K, sstride, s_q, s_s, rl, acc, rg);
    if (rr < G) {
      const int i = r0 + rr;
      const float cf = ow * gdown * s_rgs[i];
      f32x4 v = acc[0];
      v[0] = v[0] * cf;
      v[1] = v[1] * cf;
      v[2] = v[2] * cf;
      v[3] = v[3] * cf;
      s_term[i][kq] = v;
    }
  }
  if (threadIdx.x < R) s_rows[threadIdx.x] = tr;
  if (threadIdx.x <= min(ts.T, kSumTokLds)) s_off[threadIdx.x] = to;
  __syncthreads();
  // the per-token sum of the tile's 16 columns: thread u takes token u / 4, columns
  // 4 (u % 4) .. 4 (u % 4) + 3
  for (int u = threadIdx.x; u < 4 * ts.T; u += 64 * WV) {
    const int t = u >> 2, c4 = u & 3;
    const int p0 = t < kSumTokLds ? s_off[t] : ts.tok_off[t];
    const int p1 = t < kSumTokLds ? s_off[t + 1] : ts.tok_off[t + 1];
    f32x4 part[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int base = p0; base < p1; base += 8) {
      // the eight rows' indices, then their terms, each read as one batch (entries past the
      // token's list are read in range and not added)
      int ix[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ix[j] = s_rows[min(base + j, WV - 1)] & (WV - 1);
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = s_term[ix[j]][c4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (base + j < p1) {
          part[j][0] += v[j][0];
          part[j][1] += v[j][1];
          part[j][2] += v[j][2];
          part[j][3] += v[j][3];
        }
      }
    }
    f32x4 sum = part[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      sum[0] += part[j][0];
      sum[1] += part[j][1];
      sum[2] += part[j][2];
      sum[3] += part[j][3];
    }
    u32x2 ov;
    ov[0] = f32_to_bf16_rne(sum[0]) | (f32_to_bf16_rne(sum[1]) << 16);
    ov[1] = f32_to_bf16_rne(sum[2]) | (f32_to_bf16_rne(sum[3]) << 16);
    *(u32x2*)(ts.out + (size_t)t * p.N + 16 * tile + 4 * c4) = ov;
  }
}

// The W4A16 counterpart of k_gemm_quantizing_sum: a batch of at most WV expert-rows, the
// w2 GEMM over bf16 rows of h (each wave copies its group's rows into the staging area as
// they are: bf16 activations carry no row global) and the per-token sum in one launch; the
// terms are the W4A16 scatter-ready products acc * (row_w[i] * g_down[e]).
template <int WV, int D, int S>
__global__ __launch_bounds__(64 * WV) void k_gemm_w4a16_sum(GemmArgs p,
                                                            const uint16_t* __restrict__ h,
                                                            TokenSumArgs ts) {
  static_assert(WV == 8 || WV == 16, "a power of two of at most 16 waves");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ f32x4 s_term[WV][4];   // scatter terms: [grouped row][4 columns x 4]
  __shared__ int s_rows[WV];        // the token lists
  __shared__ int s_off[kSumTokLds + 1];
  const int K = p.K, R = p.a_rows;
  uint8_t* s_b = smem;  // [WV rows][b_stride(K)], then 256 bytes of slack
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x;
  const int tr = threadIdx.x < R ? ts.tok_rows[threadIdx.x] : 0;
  const int to = threadIdx.x <= min(ts.T, kSumTokLds) ? ts.tok_off[threadIdx.x] : 0;
  int4 it = int4{0, 0, 0, 0};
  if (wave < R && wave < p.E) it = p.items[1 + wave];
  const int ng = __builtin_amdgcn_readfirstlane(p.items[0].x);
  const bool has = wave < ng;  // uniform
  const int e = has ? __builtin_amdgcn_readfirstlane(it.x) : 0;
  const int r0 = has ? __builtin_amdgcn_readfirstlane(it.y) : 0;
  const int G = has ? __builtin_amdgcn_readfirstlane(it.z) : 0;
  const size_t expert_bytes = (size_t)p.N * K / 16 * 9;
  const uint8_t* wt = p.w + (size_t)e * expert_bytes + (size_t)tile * 9 * K;
  int sstride;
  const __amdgpu_buffer_rsrc_t wr = pass_weights<false>(p, wt, has ? 1 : 0, sstride);
  Ring<1, D> rg;
  float ow = 0.f, gdown = 0.f;
  const int kq = lane >> 4, rr = lane & 15;
  if (has) {
    // the group's rows of h into the staging area: the first row's loads go out before the
    // weight loads (loads complete in order), the rest after
    const int rb = 2 * K;  // bytes of a row (at most 8 KiB: 8 pieces of 16 bytes per lane)
    u32x4 first[8];
    const uint8_t* src0 = (const uint8_t*)(h + (size_t)r0 * K);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (16 * lane + 1024 * k < rb) first[k] = *(const u32x4*)(src0 + 16 * lane + 1024 * k);
    ring_prime<1, D, S, MOE_W_CPOL>(rg, wr, sstride, 16 * lane, S * 1024 + 2 * S * lane);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (16 * lane + 1024 * k < rb)
        *(u32x4*)(s_b + r0 * b_stride(K) + 16 * lane + 1024 * k) = first[k];
    for (int r = 1; r < G; ++r) {
      const uint8_t* src = (const uint8_t*)(h + (size_t)(r0 + r) * K);
      uint8_t* dst = s_b + (r0 + r) * b_stride(K);
      for (int o = 16 * lane; o < rb; o += 1024) *(u32x4*)(dst + o) = *(const u32x4*)(src + o);
    }
    gdown = p.c_g[e];
    if (rr < G) ow = p.c_w[r0 + rr];
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's LDS writes have landed
    asm volatile("" ::: "memory");
    // lanes past the group's rows read its first row: their B columns feed no term
    const int rl = r0 + (rr < G ? rr : 0);
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    bf16_stream_mfma<1, D, S, MOE_W_CPOL, D>(wr, K, sstride, s_b, rl, acc, rg);
    if (rr < G) {
      const int i = r0 + rr;
      const float cf = ow * gdown;
      f32x4 v = acc[0];
      v[0] = v[0] * cf;
      v[1] = v[1] * cf;
      v[2] = v[2] * cf;
      v[3] = v[3] * cf;
      s_term[i][kq] = v;
    }
  }
  if (threadIdx.x < R) s_rows[threadIdx.x] = tr;
  if (threadIdx.x <= min(ts.T, kSumTokLds)) s_off[threadIdx.x] = to;
  __syncthreads();
  // the per-token sum, as in k_gemm_quantizing_sum.  The two copies stay inline: one shared
  // device function, force-inlined, still changed both kernels' code (the W4A16 one with
  // eight waves grew by a third, in register moves).
  for (int u = threadIdx.x; u < 4 * ts.T; u += 64 * WV) {
    const int t = u >> 2, c4 = u & 3;
    const int p0 = t < kSumTokLds ? s_off[t] : ts.tok_off[t];
    const int p1 = t < kSumTokLds ? s_off[t + 1] : ts.tok_off[t + 1];
    f32x4 part[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int base = p0; base < p1; base += 8) {
      int ix[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ix[j] = s_rows[min(base + j, WV - 1)] & (WV - 1);
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = s_term[ix[j]][c4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (base + j < p1) {
          part[j][0] += v[j][0];
          part[j][1] += v[j][1];
          part[j][2] += v[j][2];
          part[j][3] += v[j][3];
        }
      }
    }
    f32x4 sum = part[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      sum[0] += part[j][0];
      sum[1] += part[j][1];
      sum[2] += part[j][2];
      sum[3] += part[j][3];
    }
    u32x2 ov;
    ov[0] = f32_to_bf16_rne(sum[0]) | (f32_to_bf16_rne(sum[1]) << 16);
    ov[1] = f32_to_bf16_rne(sum[2]) | (f32_to_bf16_rne(sum[3]) << 16);
    *(u32x2*)(ts.out + (size_t)t * p.N + 16 * tile + 4 * c4) = ov;
  }
}

// ------------------------------------------------------------------------- GEMV path
template <int NS, int D, int S>
__device__ __forceinline__ void gemv_pass(const GemmArgs& p, const uint8_t* __restrict__ wt,
                                          int nsv, int arow0, int nrows, int col0,
                                          uint8_t* s_q, uint8_t* s_s, float gdown) {
  constexpr int NR = kGemvRows;
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4;
  const int K = p.K, NC = K / 128;
  asm volatile("" ::: "memory");  // no hoisting of this pass's weight loads (see mfma_pass)
  const int tstride = NC * kChunkBytes;
  // (readfirstlane: the clamp may be computed on the vector unit, and a descriptor the
  // compiler believes divergent turns every load into a loop over lanes)
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(wt, __builtin_amdgcn_readfirstlane((nsv > 0 ? nsv : 0) * tstride));

  stage_rows<false, kGemmWaves>(p, arow0, nrows, s_q, s_s);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  float acc[NS][NR];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int a = 0; a < NR; ++a) acc[s][a] = 0.f;

  Ring<NS, D> rg;
  stream_weights<NS, D, S>(wr, NC, tstride, 16 * lane, S * 1024 + 2 * S * lane,
                           [&](int c, int j, const u32x4 (&wn)[NS], const u32x4 (&sg)[NS]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t ws = chunk_scales(sg[s], j);
      const float sw0 = e4m3_to_f32(ws & 0xFFu), sw1 = e4m3_to_f32(ws >> 8);
      f16x2 wv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) e2m1x8_to_f16(wn[s][q], &wv[4 * q]);
#pragma unroll
      for (int a = 0; a < NR; ++a) {
        if (a >= nrows) break;  // uniform
        const u32x4 an = *(const u32x4*)(s_q + a * q_stride(K) + 16 * kq + 64 * c);
        const uint32_t asc = *(const uint16_t*)(s_s + a * s_stride(K) + 2 * kq + 8 * c);
        const uint32_t sa = scale_pair_signed(asc);
        float b0 = 0.f, b1 = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x8 v = dequant8(an[q], sa, q >= 2);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f16x2 x2 = f16x2{v[2 * m], v[2 * m + 1]};
            if (q < 2) b0 = __builtin_amdgcn_fdot2(wv[4 * q + m], x2, b0, false);
            else b1 = __builtin_amdgcn_fdot2(wv[4 * q + m], x2, b1, false);
          }
        }
        acc[s][a] = fmaf(sw0, b0, acc[s][a]);
        acc[s][a] = fmaf(sw1, b1, acc[s][a]);
      }
    }
  }, rg);

#pragma unroll
  for (int a = 0; a < NR; ++a) {
    if (a >= nrows) break;  // uniform
    const size_t orow = arow0 + a;
    float cf = 1.0f;
    if (p.c_w) cf = p.c_w[arow0 + a] * gdown * p.c_gs[arow0 + a];  // scatter-ready output
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float v = acc[s][a];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (p.c_w) v = v * cf;
      if (s < nsv && lane < 16) __builtin_nontemporal_store(v, p.out + orow * p.N + col0 + 16 * s + lane);
    }
  }
}

template <int NS, int D, int S>
__global__ __launch_bounds__(256) void k_gemm_gemv(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_grp[4];
  uint8_t* s_q = smem;
  uint8_t* s_s = s_q + kGemvRows * q_stride(p.K);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles = p.N / 16, per_item = kGemmWaves * NS;
  const int items_per_e = (tiles + per_item - 1) / per_item;
  ItemGroup g;
  if (!find_group<kGemvRows>(p, blockIdx.x / items_per_e, s_grp, g)) return;  // uniform
  const int t0 = (blockIdx.x % items_per_e) * per_item + wave * NS;
  const int nsv = min(NS, tiles - t0);
  const size_t expert_bytes = (size_t)p.N * p.K / 16 * 9;
  const size_t tile_bytes = (size_t)9 * p.K;
  const uint8_t* wt = p.w + (size_t)g.e * expert_bytes + (size_t)(nsv > 0 ? t0 : 0) * tile_bytes;
  const float gdown = p.c_w ? p.c_g[g.e] : 0.f;
  for (int b = 0; b < g.G; b += kGemvRows) {
    if (b) __syncthreads();
    gemv_pass<NS, D, S>(p, wt, nsv, g.r0 + b, min(kGemvRows, g.G - b), 16 * t0, s_q, s_s, gdown);
  }
}

// ------------------------------------------------------------------------- launch
// Grid: one workgroup per item that can have work.  At most min(E, R) groups are non-empty
// (R grouped rows), so the grid is min(E, R) x items per expert; workgroups past the active
// items exit once they have scanned the offsets.
static int items_per_expert(int per_item, const GemmArgs& a) {
  return (a.N / 16 + per_item - 1) / per_item;
}

static int gemm_grid(int per_item, const GemmArgs& a, int R) {
  const long groups = R < a.E ? (R > 0 ? R : 1) : a.E;
  return (int)(items_per_expert(per_item, a) * groups);
}

// A small batch (decode) fills few workgroups: at most this many items of 8 tiles.  Its
// GEMMs then run the instance with a deeper weight ring (more bytes in flight per wave) and,
// outside the SwiGLU epilogue, one tile per wave (twice the waves).  Both choices change
// only which wave computes an output and how far ahead it loads, never the order of an
// output's accumulation, so results do not depend on the batch.
constexpr int kSmallGridItems = 2048;

template <class Kern>
static hipError_t launch_one(Kern kern, int per_item, const GemmArgs& a, size_t lds, int threads,
                             int R, hipStream_t s) {
  if (lds > 65536) {
    const hipError_t err = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(gemm_grid(per_item, a, R)), dim3(threads), lds, s, a);
  return hipGetLastError();
}

// The packed layout's scale group S fixes the kernel instance; the ring depth D is capped
// at S.
template <int NS, int D, bool SWI, bool ABF = false, int WAVES = kGemmWaves, int PR = kPassRows>
static hipError_t launch_mfma_t(const GemmArgs& a, int per, int R, hipStream_t s) {
  static_assert(PR >= 1 && PR <= kPassRows, "a pass feeds at most the B operand's 16 columns");
  const size_t lds = gemm_lds_bytes(a.K, PR, ABF, NS, WAVES);
  const int th = 64 * WAVES;
  switch (scale_group(a.K / 128)) {
    case 8: return launch_one(k_gemm_mfma<NS, (D < 8 ? D : 8), 8, SWI, ABF, WAVES, PR>, per, a, lds, th, R, s);
    case 4: return launch_one(k_gemm_mfma<NS, (D < 4 ? D : 4), 4, SWI, ABF, WAVES, PR>, per, a, lds, th, R, s);
    case 2: return launch_one(k_gemm_mfma<NS, (D < 2 ? D : 2), 2, SWI, ABF, WAVES, PR>, per, a, lds, th, R, s);
    default: return launch_one(k_gemm_mfma<NS, 1, 1, SWI, ABF, WAVES, PR>, per, a, lds, th, R, s);
  }
}

static bool small_grid(const GemmArgs& a, int R) {
  return gemm_grid(kGemmWaves * 2, a, R) <= kSmallGridItems;
}

static hipError_t launch_mfma(const GemmArgs& a, int R, hipStream_t s) {
  if (small_grid(a, R)) return launch_mfma_t<1, 8, false>(a, kGemmWaves, R, s);
  return launch_mfma_t<MOE_GEMM_NS, MOE_GEMM_D, false>(a, kGemmWaves * MOE_GEMM_NS, R, s);
}

static hipError_t launch_gemv(const GemmArgs& a, int R, hipStream_t s) {
  const int per = kGemmWaves * MOE_GEMV_NS;
  constexpr int D = MOE_GEMV_D;
  const size_t lds = gemm_lds_bytes(a.K, kGemvRows);
  switch (scale_group(a.K / 128)) {
    case 8: return launch_one(k_gemm_gemv<MOE_GEMV_NS, (D < 8 ? D : 8), 8>, per, a, lds, 256, R, s);
    case 4: return launch_one(k_gemm_gemv<MOE_GEMV_NS, (D < 4 ? D : 4), 4>, per, a, lds, 256, R, s);
    case 2: return launch_one(k_gemm_gemv<MOE_GEMV_NS, (D < 2 ? D : 2), 2>, per, a, lds, 256, R, s);
    default: return launch_one(k_gemm_gemv<MOE_GEMV_NS, 1, 1>, per, a, lds, 256, R, s);
  }
}

hipError_t launch_grouped_gemm_swiglu(const uint8_t* aq, const uint8_t* as, const int32_t* amap,
                                      int a_rows, const int32_t* off, int E, int R,
                                      const uint8_t* w13, int I, int K, const float* g_gate,
                                      const float* g_up, const float* row_gs,
                                      const int32_t* gs_map, uint16_t* h, hipStream_t s,
                                      const int4* items) {
  GemmArgs a{aq, as, amap, a_rows, off, E, w13, 2 * I, K, nullptr, 1, 0x7FFFFFFF,
             g_gate, g_up, row_gs, gs_map, h, I};
  a.items = items;
  // one gate tile per wave: (I/16)/4 items per expert, the grid of N = 2I with 8 per item
  if (small_grid(a, R)) return launch_mfma_t<2, 8, true>(a, 2 * kGemmWaves, R, s);
  return launch_mfma_t<2, MOE_GEMM_D, true>(a, 2 * kGemmWaves, R, s);
}

hipError_t launch_grouped_gemm(const uint8_t* aq, const uint8_t* as, const int32_t* amap,
                               int a_rows, const int32_t* off, int E, int R, const uint8_t* w,
                               int N, int K, float* out, int flags, int gemv_max_rows,
                               hipStream_t s, const float* c_w, const float* c_g,
                               const float* c_gs, const int4* items) {
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
    GemmArgs a{aq, as, amap, a_rows, off, E, w, N, K, out, gemv_lo, gemv_hi};
    a.c_w = c_w;
    a.c_g = c_g;
    a.c_gs = c_gs;
    const hipError_t err = launch_gemv(a, R, s);
    if (err != hipSuccess) return err;
  }
  if (mfma_lo < big) {
    GemmArgs a{aq, as, amap, a_rows, off, E, w, N, K, out, mfma_lo < 1 ? 1 : mfma_lo, big};
    a.c_w = c_w;
    a.c_g = c_g;
    a.c_gs = c_gs;
    if (mfma_lo <= 1) a.items = items;  // the work list covers every group
    const hipError_t err = launch_mfma(a, R, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

bool grouped_gemm_layer_fits(int E, int R, int H, int I) {
  // both GEMMs on their large-grid instances with the 8-chunk scale group, and rows of h
  // that one wave quantizes with at most two scale blocks per lane
  if (R < 1 || H % 1024 || I % 1024 || I > 2048) return false;
  GemmArgs a13{};
  a13.E = E;
  a13.N = 2 * I;
  a13.K = H;
  GemmArgs a2{};
  a2.E = E;
  a2.N = H;
  a2.K = I;
  // (the two GEMMs on the same kind of grid, so that one instance serves both)
  return small_grid(a13, R) == small_grid(a2, R);
}

int grouped_gemm_layer_sync_ints(int E, int R, int H, int I) {
  if (!grouped_gemm_layer_fits(E, R, H, I)) return 0;
  GemmArgs a13{};
  a13.E = E;
  a13.N = 2 * I;
  a13.K = H;
  a13.I = I;
  const int n13 = gemm_grid(2 * kGemmWaves, a13, R);
  return n13 + kQuantParts * (n13 / items_per_group<true, 2, kGemmWaves>(a13));
}

hipError_t launch_grouped_gemm_layer(const uint8_t* xq, const uint8_t* xs, const int32_t* row_src,
                                     int S, const int32_t* off, int E, int R, const uint8_t* w13,
                                     const uint8_t* w2, int I, int H, const float* g_gate,
                                     const float* g_up, const float* xgs, uint16_t* h,
                                     uint8_t* hq, uint8_t* hs, float* hgs, const float* row_w,
                                     const float* g_down, float* terms, const int4* items,
                                     int* sync, int32_t* err, hipStream_t s) {
  const int big = 0x7FFFFFFF;
  GemmArgs a13{xq, xs, row_src, S, off, E, w13, 2 * I, H, nullptr, 1, big,
               g_gate, g_up, xgs, row_src, h, I};
  a13.items = items;
  GemmArgs a2{hq, hs, nullptr, R, off, E, w2, H, I, terms, 1, big};
  a2.c_w = row_w;
  a2.c_g = g_down;
  a2.c_gs = hgs;
  a2.items = items;
  // the separate launches' instances: a small grid (decode batches of 33 to 64 rows at
  // 288 experts) takes the deeper ring and, in w2, one tile per wave
  const bool small = small_grid(a13, R);
  const int n13 = gemm_grid(2 * kGemmWaves, a13, R);
  const int n2 = gemm_grid((small ? 1 : 2) * kGemmWaves, a2, R);
  const int groups = n13 / items_per_group<true, 2, kGemmWaves>(a13);
  const LayerSync f{n13, groups, sync, sync + n13, err, hq, hs, hgs};
  const size_t l13 = gemm_lds_bytes(H, kPassRows),
               l2 = gemm_lds_bytes(I, kPassRows, false, small ? 1 : 2);
  const size_t lds = l13 > l2 ? l13 : l2;
  auto kern = small ? (I <= 1024 ? k_gemm_layer<8, 1, 8, 8, 1> : k_gemm_layer<8, 1, 8, 8, 2>)
                    : (I <= 1024 ? k_gemm_layer<MOE_GEMM_D, 2, MOE_GEMM_D, 8, 1>
                                 : k_gemm_layer<MOE_GEMM_D, 2, MOE_GEMM_D, 8, 2>);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(n13 + kQuantParts * groups + n2), dim3(64 * kGemmWaves), lds, s,
                     a13, a2, f);
  return hipGetLastError();
}

// ------------------------------------------------------------------------- W4A16
// bf16 activations take 2K bytes per staged row (128 KiB for 16 rows at K = 4096), which
// leaves room for one workgroup per CU: the general W4A16 instance runs 16 waves per
// workgroup, the same 16 waves per CU streaming weights against one shared copy of the
// staged rows.  Batch shapes that allow it take smaller workgroups (below).
constexpr int kW4A16Waves = 16;
// A small batch would leave most CUs idle with such workgroups (at one row per group, 8
// items per expert at N = 4096), so it runs the small-grid shape of the NVFP4 instances
// (4 waves, deep ring) staging 4 rows per pass: 32 KiB at K = 4096, four workgroups per
// CU.  It is taken only when there are at most as many rows as experts, so that passes of
// 4 rows rarely repeat a group's weight stream (a decode step of up to 4 tokens, top-k,
// never does: no group has more rows than tokens).
constexpr int kSmallW4A16PassRows = 4;
constexpr int kW4A16PassRows8 = 8;

static bool small_w4a16(const GemmArgs& a, int R) { return small_grid(a, R) && R <= a.E; }

hipError_t launch_grouped_gemm_w4a16(const uint16_t* ab, const int32_t* amap, int a_rows,
                                     const int32_t* off, int E, int R, const uint8_t* w, int N,
                                     int K, float* out, hipStream_t s, const float* c_w,
                                     const float* c_g, const int4* items) {
  GemmArgs a{nullptr, nullptr, amap, a_rows, off, E, w, N, K, out, 1, 0x7FFFFFFF};
  a.c_w = c_w;
  a.c_g = c_g;
  a.ab = ab;
  a.items = items;  // (read only by the instances that stage kWorkListMultiRows rows a pass)
  if (small_w4a16(a, R))
    return launch_mfma_t<1, 8, false, true, kGemmWaves, kSmallW4A16PassRows>(a, kGemmWaves, R, s);
  // Up to K = 2048 the 16 staged rows take at most 64 KiB: two workgroups of 8 waves per CU,
  // so one workgroup's ramp and tail overlap the other's stream (with the w2 GEMM on this
  // instance the W4A16 layer measured 2-3% faster on MI355X than with 16-wave workgroups).
  if (K <= 2048) return launch_mfma_t<2, MOE_GEMM_D, false, true, 8>(a, 2 * 8, R, s);
  return launch_mfma_t<2, MOE_GEMM_D, false, true, kW4A16Waves>(a, 2 * kW4A16Waves, R, s);
}

hipError_t launch_grouped_gemm_swiglu_w4a16(const uint16_t* ab, const int32_t* amap, int a_rows,
                                            const int32_t* off, int E, int R, const uint8_t* w13,
                                            int I, int K, const float* g_gate, const float* g_up,
                                            uint16_t* h, hipStream_t s, const int4* items) {
  GemmArgs a{nullptr, nullptr, amap, a_rows, off, E, w13, 2 * I, K, nullptr, 1, 0x7FFFFFFF,
             g_gate, g_up, nullptr, nullptr, h, I};
  a.ab = ab;
  a.items = items;  // (as above)
  // one gate tile per wave: (I/WAVES)/16 items per expert, the grid of N = 2I with 2 WAVES
  // tiles per item
  if (small_w4a16(a, R))
    return launch_mfma_t<2, 8, true, true, kGemmWaves, kSmallW4A16PassRows>(a, 2 * kGemmWaves, R, s);
  // At most 4 rows per expert on average, groups rarely exceed 8 rows: staging 8 rows per
  // pass (64 KiB at K = 4096) fits two 8-wave workgroups per CU (the W4A16 layer measured
  // 3.7% faster on ragged570 than with one 16-wave workgroup staging 16 rows).
  if (R <= 4 * E)
    return launch_mfma_t<2, MOE_GEMM_D, true, true, 8, kW4A16PassRows8>(a, 2 * 8, R, s);
  return launch_mfma_t<2, MOE_GEMM_D, true, true, kW4A16Waves>(a, 2 * kW4A16Waves, R, s);
}

template <bool ABF>
static hipError_t launch_swiglu_grouping_t(const int32_t* a_expert, const int32_t* a_src,
                                           const int32_t* a_dst, const float* a_w, int R, int E,
                                           int S, int T, const uint16_t* x,
                                           int32_t* expert_offsets, int32_t* row_src,
                                           int32_t* row_dst, float* row_w, int32_t* tok_off,
                                           int32_t* tok_rows, int32_t* err_word,
                                           const uint8_t* w13, int I, int K, const float* g_gate,
                                           const float* g_up, uint16_t* h, hipStream_t s,
                                           int4* items) {
  if (R < 1 || R > kSmallGroupRows) return hipErrorInvalidValue;
  GemmArgs a{nullptr, nullptr, nullptr, S, expert_offsets, E, w13, 2 * I, K, nullptr, 1,
             0x7FFFFFFF, g_gate, g_up, nullptr, nullptr, h, I};
  const GroupArgs g{a_expert, a_src, a_dst, a_w, R, S, T, x, expert_offsets, row_src,
                    row_dst, row_w, tok_off, tok_rows, err_word, items};
  const size_t lds = gemm_lds_bytes(K, ABF ? 4 : kPassRows, ABF);
  // one workgroup per item slot, plus the one that writes the grouping's outputs
  const dim3 grid(gemm_grid(2 * kGemmWaves, a, R) + 1), block(64 * kGemmWaves);
  auto go = [&](auto kern) {
    if (lds > 65536) {
      const hipError_t err = hipFuncSetAttribute((const void*)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(kern, grid, block, lds, s, a, g);
    return hipGetLastError();
  };
  // (a thread quantizes one 16-element block of each row up to K = 4096, two above)
  if (K <= 64 * kGemmWaves * 16 && !ABF && S == 1) {  // one source row: its prefetching instance
    switch (scale_group(K / 128)) {
      case 8: return go(k_gemm_swiglu_grouping<8, 8, false, 1, true>);
      case 4: return go(k_gemm_swiglu_grouping<4, 4, false, 1, true>);
      case 2: return go(k_gemm_swiglu_grouping<2, 2, false, 1, true>);
      default: return go(k_gemm_swiglu_grouping<1, 1, false, 1, true>);
    }
  }
  // Two to four tokens (several workgroups per CU): a 4-chunk ring over the 8-chunk scale
  // groups measured faster than the 8-chunk one (M = 2 54.4 -> 50.5 us, M = 4 87.4 -> 84.3
  // with the w2 launch's likewise, MI355X A/B); one token keeps the deeper ring.
  if (K <= 64 * kGemmWaves * 16 && !ABF && scale_group(K / 128) == 8)
    return go(k_gemm_swiglu_grouping<4, 8, false, 1>);
  if (K <= 64 * kGemmWaves * 16) {
    switch (scale_group(K / 128)) {
      case 8: return go(k_gemm_swiglu_grouping<8, 8, ABF, 1>);
      case 4: return go(k_gemm_swiglu_grouping<4, 4, ABF, 1>);
      case 2: return go(k_gemm_swiglu_grouping<2, 2, ABF, 1>);
      default: return go(k_gemm_swiglu_grouping<1, 1, ABF, 1>);
    }
  }
  switch (scale_group(K / 128)) {
    case 8: return go(k_gemm_swiglu_grouping<8, 8, ABF, 2>);
    case 4: return go(k_gemm_swiglu_grouping<4, 4, ABF, 2>);
    case 2: return go(k_gemm_swiglu_grouping<2, 2, ABF, 2>);
    default: return go(k_gemm_swiglu_grouping<1, 1, ABF, 2>);
  }
}

hipError_t launch_grouped_gemm_swiglu_grouping(const int32_t* a_expert, const int32_t* a_src,
                                               const int32_t* a_dst, const float* a_w, int R,
                                               int E, int S, int T, const uint16_t* x,
                                               int32_t* expert_offsets, int32_t* row_src,
                                               int32_t* row_dst, float* row_w, int32_t* tok_off,
                                               int32_t* tok_rows, int32_t* err_word,
                                               const uint8_t* w13, int I, int K,
                                               const float* g_gate, const float* g_up,
                                               uint16_t* h, hipStream_t s, bool bf16_acts,
                                               int4* items) {
  auto f = bf16_acts ? launch_swiglu_grouping_t<true> : launch_swiglu_grouping_t<false>;
  return f(a_expert, a_src, a_dst, a_w, R, E, S, T, x, expert_offsets, row_src, row_dst, row_w,
           tok_off, tok_rows, err_word, w13, I, K, g_gate, g_up, h, s, items);
}

hipError_t launch_grouped_gemm_quantizing(const uint16_t* h, const int32_t* expert_offsets,
                                          int E, int R, const uint8_t* w2, int N, int K,
                                          float* out, const float* row_w, const float* g_down,
                                          hipStream_t s, const int4* items, bool one_source) {
  if (R < 1 || R > kSmallGroupRows) return hipErrorInvalidValue;
  GemmArgs a{nullptr, nullptr, nullptr, R, expert_offsets, E, w2, N, K, out, 1, 0x7FFFFFFF};
  a.c_w = row_w;
  a.c_g = g_down;
  a.items = items;
  const size_t lds = gemm_lds_bytes(K, kPassRows, false, 1);
  const dim3 grid(gemm_grid(kGemmWaves, a, R)), block(64 * kGemmWaves);
  auto go = [&](auto kern) {
    if (lds > 65536) {
      const hipError_t err = hipFuncSetAttribute((const void*)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(kern, grid, block, lds, s, a, h);
    return hipGetLastError();
  };
  if (K <= 64 * kGemmWaves * 16 && one_source) {  // its prefetching instance
    switch (scale_group(K / 128)) {
      case 8: return go(k_gemm_quantizing<8, 8, 1, true>);
      case 4: return go(k_gemm_quantizing<4, 4, 1, true>);
      case 2: return go(k_gemm_quantizing<2, 2, 1, true>);
      default: return go(k_gemm_quantizing<1, 1, 1, true>);
    }
  }
  // (two to four tokens: a 4-chunk ring, as in launch_swiglu_grouping_t)
  if (K <= 64 * kGemmWaves * 16 && scale_group(K / 128) == 8) return go(k_gemm_quantizing<4, 8, 1>);
  if (K <= 64 * kGemmWaves * 16) {
    switch (scale_group(K / 128)) {
      case 8: return go(k_gemm_quantizing<8, 8, 1>);
      case 4: return go(k_gemm_quantizing<4, 4, 1>);
      case 2: return go(k_gemm_quantizing<2, 2, 1>);
      default: return go(k_gemm_quantizing<1, 1, 1>);
    }
  }
  switch (scale_group(K / 128)) {
    case 8: return go(k_gemm_quantizing<8, 8, 2>);
    case 4: return go(k_gemm_quantizing<4, 4, 2>);
    case 2: return go(k_gemm_quantizing<2, 2, 2>);
    default: return go(k_gemm_quantizing<1, 1, 2>);
  }
}

// (K above 2048 with 16 waves would spill: four blocks of h per lane and the ring)
bool grouped_gemm_quantizing_sum_fits(int R, int K) {
  return R >= 1 && R <= 16 && K <= (R <= 8 ? 4096 : 2048) &&
         (K <= 1024 || scale_group(K / 128) == 8);
}

hipError_t launch_grouped_gemm_quantizing_sum(const uint16_t* h, int E, int R, const uint8_t* w2,
                                              int N, int K, const float* row_w,
                                              const float* g_down, const int4* items,
                                              const int32_t* tok_off, const int32_t* tok_rows,
                                              int T, uint16_t* out, hipStream_t s) {
  if (!grouped_gemm_quantizing_sum_fits(R, K) || N % 16 != 0 || !items) return hipErrorInvalidValue;
  GemmArgs a{nullptr, nullptr, nullptr, R, nullptr, E, w2, N, K, nullptr, 1, 0x7FFFFFFF};
  a.c_w = row_w;
  a.c_g = g_down;
  a.items = items;
  const TokenSumArgs ts{tok_off, tok_rows, T, out};
  const int WV = R <= 8 ? 8 : 16;
  const size_t lds = (size_t)WV * (q_stride(K) + s_stride(K)) + 256;
  auto go = [&](auto kern) {
    if (lds > 65536) {
      const hipError_t err = hipFuncSetAttribute((const void*)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(kern, dim3(N / 16), dim3(64 * WV), lds, s, a, h, ts);
    return hipGetLastError();
  };
  // (one token: an 8-chunk weight ring; two: a 4-chunk ring, as in the three-launch path)
  if (K > 2048) return go(k_gemm_quantizing_sum<8, 8, 8, 4>);
  if (K > 1024) return WV == 8 ? go(k_gemm_quantizing_sum<8, 8, 8, 2>) : go(k_gemm_quantizing_sum<16, 4, 8, 2>);
  switch (scale_group(K / 128)) {
    case 8: return WV == 8 ? go(k_gemm_quantizing_sum<8, 8, 8, 1>) : go(k_gemm_quantizing_sum<16, 4, 8, 1>);
    case 4: return WV == 8 ? go(k_gemm_quantizing_sum<8, 4, 4, 1>) : go(k_gemm_quantizing_sum<16, 4, 4, 1>);
    case 2: return WV == 8 ? go(k_gemm_quantizing_sum<8, 2, 2, 1>) : go(k_gemm_quantizing_sum<16, 2, 2, 1>);
    default: return WV == 8 ? go(k_gemm_quantizing_sum<8, 1, 1, 1>) : go(k_gemm_quantizing_sum<16, 1, 1, 1>);
  }
}

// (the bf16 rows of 16 waves' groups fill 66 KiB of LDS at K = 2048)
bool grouped_gemm_w4a16_sum_fits(int R, int K) {
  return R >= 1 && R <= 16 && K <= (R <= 8 ? 4096 : 2048);
}

hipError_t launch_grouped_gemm_w4a16_sum(const uint16_t* h, int E, int R, const uint8_t* w2,
                                         int N, int K, const float* row_w, const float* g_down,
                                         const int4* items, const int32_t* tok_off,
                                         const int32_t* tok_rows, int T, uint16_t* out,
                                         hipStream_t s) {
  if (!grouped_gemm_w4a16_sum_fits(R, K) || N % 16 != 0 || !items) return hipErrorInvalidValue;
  GemmArgs a{nullptr, nullptr, nullptr, R, nullptr, E, w2, N, K, nullptr, 1, 0x7FFFFFFF};
  a.c_w = row_w;
  a.c_g = g_down;
  a.items = items;
  const TokenSumArgs ts{tok_off, tok_rows, T, out};
  const int WV = R <= 8 ? 8 : 16;
  const size_t lds = (size_t)WV * b_stride(K) + 256;
  auto go = [&](auto kern) {
    if (lds > 65536) {
      const hipError_t err = hipFuncSetAttribute((const void*)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(kern, dim3(N / 16), dim3(64 * WV), lds, s, a, h, ts);
    return hipGetLastError();
  };
  switch (scale_group(K / 128)) {
    case 8: return WV == 8 ? go(k_gemm_w4a16_sum<8, 8, 8>) : go(k_gemm_w4a16_sum<16, 4, 8>);
    case 4: return WV == 8 ? go(k_gemm_w4a16_sum<8, 4, 4>) : go(k_gemm_w4a16_sum<16, 4, 4>);
    case 2: return WV == 8 ? go(k_gemm_w4a16_sum<8, 2, 2>) : go(k_gemm_w4a16_sum<16, 2, 2>);
    default: return WV == 8 ? go(k_gemm_w4a16_sum<8, 1, 1>) : go(k_gemm_w4a16_sum<16, 1, 1>);
  }
}

}  // namespace moe
