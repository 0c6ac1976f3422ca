// Shared device helpers and internal launch interfaces of the MoE NVFP4 library.
// gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ------------------------------------------------------------------------------ codec
// e4m3fn value of a scale byte, as an exact float.  Normal codes: 2^(e-7) * (1 + m/8),
// built directly as float bits; subnormal codes: m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                      : (float)m * 0.001953125f;
  return (b & 0x80u) ? -mag : mag;
}

// Nearest e4m3fn code of a non-negative float, ties to even, saturating at 448 (0x7E).
// Normal range: round the float32 significand to 3 bits with round-half-even on the bit
// pattern (a carry moves into the exponent); below 2^-6 the grid is uniform with step
// 2^-9, so the code is rint(v * 512) (v * 512 is exact).
__device__ __forceinline__ uint32_t e4m3_encode_pos(float v) {
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);
  const uint32_t b = __float_as_uint(v);
  const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;  // biased exp : 3-bit mantissa
  const uint32_t code = r - (120u << 3);                        // rebias 127 -> 7
  return code > 0x7Eu ? 0x7Eu : code;
}

// Nearest e2m1 codes of eight finite floats, ties to even (code LSB 0), saturating at 6,
// sign kept (-0 and negative values that round to 0 give code 8; grid {0, .5, 1, 1.5, 2,
// 3, 4, 6}), packed as one word with element 2k in the low nibble of byte k.  This is the
// hardware fp32 -> fp4 pack conversion at scale 1 (no scaling): compared on MI355X against
// a software nearest-even encoder over every non-NaN fp32 bit pattern, with no difference.
__device__ __forceinline__ uint32_t e2m1x8_encode(const float* q) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
}

// Eight e2m1 nibbles (one 32-bit word, element 2k in the low nibble of byte k) times a
// non-negative block scale given as a float times 2^-8 (scale_pair_pos's f16 halves,
// widened) -> 8 exact bf16 values in element order (W4A16 weights).  Each nibble pair
// converts to float times 2^8 exactly, the product with the scaled e4m3 value has at most
// 6 significant bits (exact in float), and its upper 16 bits are then the bf16 value itself.
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t w, float scale) {
  const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 0);
  const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 1);
  const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 2);
  const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 3);
  const f32x2 pp[4] = {p0, p1, p2, p3};
  u32x4 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float lo = pp[b][0] * scale, hi = pp[b][1] * scale;
    r[b] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, r);
}

// bf16 <-> float
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------- dequantization
// The gfx950 scaled FP4 conversion applies only the exponent of its fp32 scale operand,
// so it cannot apply an e4m3 block scale (4 significant bits) by itself.  We convert
// with a power-of-two scale of 2^8 and multiply by the block scale expressed as f16
// times 2^-8: an e4m3fn byte s.eeee.mmm placed as f16 bits s.0eeee.mmm0000000 is exactly
// e4m3 * 2^-8, for normal and subnormal codes alike.  Every product e2m1 * e4m3 (6
// significant bits, magnitude in [2^-10, 2688]) is exact in f16, so the dequantized
// operands are exact.
//
// Scales travel in pairs: the two block scales of a lane's 32-element row segment, as the
// f16 values of both in one 32-bit register (first block in the low half); a multiply
// broadcasts the half it needs.

// Scale pair from two e4m3 bytes of `w` (selector: which bytes; 0x0c010c00 takes bytes
// 0 and 1, 0x0c030c02 bytes 2 and 3) whose sign bits are clear: the f16 bits are the byte
// shifted left by 7.  Packed weight scales are always non-negative (the packer moves a
// negative scale's sign into the block's e2m1 codes).
__device__ __forceinline__ uint32_t scale_pair_pos(uint32_t w, uint32_t sel) {
  return __builtin_amdgcn_perm(0u, w, sel) << 7;
}
// Same for bytes 0 and 1 of `w` that may carry a sign: the sign bit moves to bit 15.
__device__ __forceinline__ uint32_t scale_pair_signed(uint32_t w) {
  const uint32_t u = __builtin_amdgcn_perm(0u, w, 0x0c010c00u) << 7;
  return (u & 0x3F803F80u) | ((u << 1) & 0x80008000u);
}

// Eight e2m1 nibbles (one 32-bit word, element 2k in the low nibble of byte k) times
// one scale of a pair (hi: the second block's) -> 8 exact f16 values in element order.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, uint32_t pair, bool hi) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3);
  const f16x2 h = __builtin_bit_cast(f16x2, pair);
  const f16x2 s = hi ? __builtin_shufflevector(h, h, 1, 1) : __builtin_shufflevector(h, h, 0, 0);
  p0 *= s; p1 *= s; p2 *= s; p3 *= s;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight e2m1 nibbles -> 8 exact f16 values of the bare e2m1 codes (no scale).
__device__ __forceinline__ void e2m1x8_to_f16(uint32_t w, f16x2 out[4]) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
}

// ------------------------------------------------------------------------------ SwiGLU
// One SwiGLU output as bf16 bits: zg = cg * ag, zu = cu * au (cg, cu: the row's gate / up
// coefficient, activation global times the expert's weight global), silu(zg) * zu.  Shared
// by the SwiGLU kernel and the fused w13 epilogue so that both give the same bits.
__device__ __forceinline__ uint32_t swiglu_bf16(float cg, float ag, float cu, float au) {
  const float zg = cg * ag, zu = cu * au;
  const float silu = zg / (1.0f + expf(-zg));
  return f32_to_bf16_rne(silu * zu);
}

// ------------------------------------------------------------------ packed weight layout
// A matrix [N, K] is stored as N/16 tiles of 16 rows, an expert as N/16 consecutive tiles,
// with no padding (N * K * 9/16 bytes per expert).  A tile covers K/128 chunks of 128
// columns, taken in scale groups of S consecutive chunks (S = scale_group(K/128): the
// largest of 8, 4, 2, 1 that divides K/128).  A scale group is S * 1152 contiguous bytes:
//   [j * 1024, (j + 1) * 1024), j < S: chunk j of the group; lane l (0..63) owns bytes
//                 [16l, 16l + 16): row (l & 15) of the tile, columns [128c + 32(l >> 4), +32)
//                 of the chunk's 128 columns c — the canonical nibble bytes of that row
//                 segment, in order;
//   [S * 1024 + 2S * l, +2S): lane l's scale bytes for the S chunks of the group, two
//                 per chunk (the two e4m3 scales of its 32-column row segment), chunk by
//                 chunk.
// Block scales are stored non-negative: a block whose scale byte has the sign bit set is
// stored with that bit clear and the sign bits of its 16 e2m1 codes flipped, which gives
// the same 16 values bit for bit (negative zero included).
// So a wave reads a chunk of a tile with one 16-byte load per lane, and the scales of S
// chunks with one 2S-byte load per lane (16 bytes at S = 8), all perfectly coalesced.
constexpr int kChunkBytes = 1152;

__host__ __device__ __forceinline__ int scale_group(int nc) {
  return nc % 8 == 0 ? 8 : nc % 4 == 0 ? 4 : nc % 2 == 0 ? 2 : 1;
}

// ------------------------------------------------------------------ row quantization
__device__ __forceinline__ float wave_max(float v) {
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

// Expand 16 bf16 values (two 16-byte words, element order) to floats.
__device__ __forceinline__ void bf16x16_to_f32(const u32x4& w0, const u32x4& w1, float* v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w0[e] << 16);
    v[2 * e + 1] = __uint_as_float(w0[e] & 0xFFFF0000u);
    v[8 + 2 * e] = __uint_as_float(w1[e] << 16);
    v[8 + 2 * e + 1] = __uint_as_float(w1[e] & 0xFFFF0000u);
  }
}

// NVFP4 row quantization, for a row held by `nthreads` threads of the workgroup (a
// multiple of 64, aligned to a wave): thread t (0 <= t < nthreads) owns scale blocks
// b = t + nthreads * k (k < BPT, b < NB) and holds their 16 values in v[k][.].
// Arithmetic, in float32 with correctly rounded divisions and no contraction, in order:
//   amax = max|x|; gs = amax / 2688 (1 if amax == 0); per block: sf = max|x_b| / (6 gs),
//   sc = e4m3(sf) nearest-even saturating, d = e4m3_value(sc) * gs; per element:
//   code = e2m1(x / d) nearest-even saturating with its sign, 0 if d == 0.
//
// Step 1: the row's amax.  Every thread of the workgroup must call this together (it has a
// workgroup barrier).  s_red: nthreads / 64 floats of LDS private to this row.
template <int BPT>
__device__ __forceinline__ float row_amax_threads(const float (&v)[BPT][16], int t, int nthreads,
                                                  float* s_red) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < BPT; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, __builtin_fabsf(v[k][e]));
  m = wave_max(m);
  if ((t & 63) == 0) s_red[t >> 6] = m;
  __syncthreads();
  float amax = 0.0f;
  for (int w = 0; w < nthreads / 64; ++w) amax = fmaxf(amax, s_red[w]);
  return amax;
}

// Step 2: codes, scale bytes and the row global (no barrier; call only for real rows),
// handed to `st`: st.codes(b, {lo, hi}) for block b's 16 codes (8 bytes, element order),
// st.scale(b, byte) for its scale byte, st.global(gs) (by thread 0).
template <int BPT, class Store>
__device__ __forceinline__ void quantize_row_emit(const float (&v)[BPT][16], int NB, int t,
                                                  int nthreads, float amax, Store& st) {
#pragma clang fp contract(off)
  const float gs = amax > 0.0f ? amax / 2688.0f : 1.0f;
  const float tg = 6.0f * gs;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int b = t + nthreads * k;
    if (b >= NB) continue;
    float bmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, __builtin_fabsf(v[k][e]));
    const float sf = bmax / tg;
    const uint32_t sb = e4m3_encode_pos(sf);
    const float d = e4m3_to_f32(sb) * gs;
    uint32_t lo = 0, hi = 0;
    if (d >= 0x1p-60f && d <= 0x1p60f) {
      // x / d correctly rounded without a division per element: the reciprocal refined by
      // one Newton step, then the quotient x * y corrected twice by its exact residual
      // fma(-d, q, x) (Markstein's method; the same operations as the IEEE division
      // sequence when no operand needs rescaling, which holds for d in this range and
      // every x whose quotient can reach the first decision point 0.25).  The residual
      // steps turn a zero quotient of -0 into +0, so the sign is taken from x (d > 0).
      float y = __builtin_amdgcn_rcpf(d);
      y = fmaf(fmaf(-d, y, 1.0f), y, y);
      auto quot = [&](float x) {
        float q = x * y;
        q = fmaf(fmaf(-d, q, x), y, q);
        q = fmaf(fmaf(-d, q, x), y, q);
        return __builtin_copysignf(q, x);  // a zero quotient keeps x's sign, as x / d does
      };
      float qv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) qv[e] = quot(v[k][e]);
      lo = e2m1x8_encode(qv);
      hi = e2m1x8_encode(qv + 8);
    } else if (d != 0.0f) {
      float qv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) qv[e] = v[k][e] / d;
      lo = e2m1x8_encode(qv);
      hi = e2m1x8_encode(qv + 8);
    }
    st.codes(b, u32x2{lo, hi});
    st.scale(b, sb);
  }
  if (t == 0) st.global(gs);
}

// Plain stores of a quantized row: codes at q (NB x 8 bytes), scale bytes at sc, the
// global at *gs_out.
struct RowStorePlain {
  uint8_t* __restrict__ q;
  uint8_t* __restrict__ sc;
  float* __restrict__ gs_out;
  __device__ __forceinline__ void codes(int b, const u32x2& v) { *(u32x2*)(q + 8 * (size_t)b) = v; }
  __device__ __forceinline__ void scale(int b, uint32_t sb) { sc[b] = (uint8_t)sb; }
  __device__ __forceinline__ void global(float gs) { *gs_out = gs; }
};

template <int BPT>
__device__ __forceinline__ void quantize_row_store(const float (&v)[BPT][16], int NB, int t,
                                                   int nthreads, float amax,
                                                   uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ sc,
                                                   float* __restrict__ gs_out) {
  RowStorePlain st{q, sc, gs_out};
  quantize_row_emit<BPT>(v, NB, t, nthreads, amax, st);
}

// The grouped GEMM's work list, written by the grouping: the non-empty groups in the order
// the GEMM's items take them, groups of more than this many rows (one pass of activation
// rows) first.  items[0] = {groups, groups of more than kWorkListMultiRows rows},
// items[1 + a] = {expert, first grouped row, rows} of group a.
constexpr int kWorkListMultiRows = 16;

// ------------------------------------------------------------------ one-wave grouping
// The grouping of a small batch (at most 64 assignments) by one wave, shared by the
// grouping launch and the decode-sized w13 GEMM, which groups in every workgroup.
// Number of lanes p whose `sorted` value is below x, where `sorted` ascends with the lane
// index (a binary search over the wave with shuffles; every lane of the wave must call it).
__device__ __forceinline__ int wave_count_below(int sorted, int x) {
  int i = 0;
  for (int step = 32; step >= 1; step >>= 1)
    if (__shfl(sorted, i + step - 1, 64) < x) i += step;
  if (i == 63 && __shfl(sorted, 63, 64) < x) i = 64;
  return i;
}

// The grouping of at most 64 assignments by wave 0 (lane j holds assignment j), with the
// results of group_body: grouped position = the number of (key, index) pairs below the
// lane's own (key = expert id, or E for a dropped assignment), by one comparison
// per assignment; the token lists likewise by (output row, grouped position); the offsets
// by binary searches of the sorted keys, which one ds_permute puts in lane order.
__device__ __forceinline__ void group_small(const int32_t* __restrict__ a_expert,
                                            const int32_t* __restrict__ a_src,
                                            const int32_t* __restrict__ a_dst,
                                            const float* __restrict__ a_w, int R, int E, int S,
                                            int T, int32_t* __restrict__ expert_offsets,
                                            int32_t* __restrict__ row_src,
                                            int32_t* __restrict__ row_dst,
                                            float* __restrict__ row_w,
                                            int32_t* __restrict__ tok_off,
                                            int32_t* __restrict__ tok_rows,
                                            int32_t* __restrict__ err_word,
                                            int4* __restrict__ items = nullptr) {
  if (threadIdx.x >= 64) return;  // wave 0 only (no barrier follows)
  const int lane = threadIdx.x;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const bool act = lane < R;
  int e = 0, sr = 0, d = 0;
  float wv = 0.f;
  if (act) {
    e = a_expert[lane];
    sr = a_src[lane];
    d = a_dst[lane];
    wv = a_w[lane];
  }
  int bad = 0;
  if (act) {
    if (e < 0 || e >= E) bad |= MOE_ERR_EXPERT;
    if (sr < 0 || sr >= S) bad |= MOE_ERR_SRC;
    if (d < 0 || d >= T) bad |= MOE_ERR_DST;
  }
  const bool valid = act && !bad;
  const uint64_t vmask = __ballot(valid);
  const int Rv = __popcll(vmask);
  // 1. grouped position: stable order by (key, assignment index).  The counting loops run
  // with every lane active: a lane read by readlane must hold the value computed for it,
  // which the compiler only guarantees outside the branches that exclude that lane.
  const int key = act ? (valid ? e : E) : 0x7FFFFFFF;
  int rank = 0;
  for (int k = 0; k < R; ++k) {
    const int kk = __builtin_amdgcn_readlane(key, k);
    rank += (kk < key || (kk == key && k < lane)) ? 1 : 0;
  }
  const int pos = act ? rank : lane;  // lanes past R keep their own slot: still a permutation
  if (act) {
    row_src[pos] = valid ? sr : -1;
    row_dst[pos] = valid ? d : -1;
    row_w[pos] = valid ? wv : 0.f;
  }
  // 2. expert offsets: grouped rows with a key below e (dropped ones carry key E)
  const int skey = __builtin_amdgcn_ds_permute(4 * pos, key);  // lane p: the key at position p
  for (int base = 0; base <= E; base += 64) {  // uniform: every lane joins the shuffles
    const int c = wave_count_below(skey, base + lane);
    if (base + lane <= E) expert_offsets[base + lane] = c;
  }
  // 2b. the grouped GEMMs' work list (kWorkListMultiRows), when asked for: group sizes from
  // the same counts, groups of more than kWorkListMultiRows rows first
  if (items) {  // uniform
    int n = 0, n_multi = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int base = 0; base < E; base += 64) {  // uniform
        const int e = base + lane;
        const int lo = wave_count_below(skey, e), hi = wave_count_below(skey, e + 1);
        const int G = e < E ? hi - lo : 0;
        const bool sel = pass == 0 ? G > kWorkListMultiRows : (G > 0 && G <= kWorkListMultiRows);
        const uint64_t m = __ballot(sel);
        if (sel) items[1 + n + __popcll(m & below)] = int4{e, lo, G, 0};
        n += __popcll(m);
      }
      if (pass == 0) n_multi = n;
    }
    if (lane == 0) items[0] = int4{n, n_multi, 0, 0};
  }
  // 3. token lists: valid rows in (output row, grouped position) order
  const int tkey = valid ? d * 64 + pos : 0x7FFFFFFF;
  int trank = 0;
  for (int k = 0; k < R; ++k) trank += __builtin_amdgcn_readlane(tkey, k) < tkey ? 1 : 0;
  // the other lanes keep distinct slots past Rv
  const int tpos = valid ? trank : Rv + __popcll(~vmask & below);
  if (valid) tok_rows[tpos] = pos;
  const int sdst = __builtin_amdgcn_ds_permute(4 * tpos, valid ? d : 0x7FFFFFFF);
  for (int base = 0; base <= T; base += 64) {
    const int c = wave_count_below(sdst, base + lane);
    if (base + lane <= T) tok_off[base + lane] = c;
  }
  int err = bad;
  for (int m = 32; m >= 1; m >>= 1) err |= __shfl_xor(err, m, 64);
  if (lane == 0) *err_word = err;
}

// Threads per row for NB scale blocks: a multiple of 64, at most 256.
static inline int row_threads(int NB) {
  const int t = ((NB + 63) / 64) * 64;
  return t < 256 ? t : 256;
}

}  // namespace moe

// ------------------------------------------------------------------ internal launchers
// (host functions defined in the kernel translation units; arguments already validated)
namespace moe {
// Grouping of the assignments (moe_gather_rows without the gather); items (E + 1 entries,
// or nullptr): also the grouped GEMM's work list (kWorkListMultiRows).
hipError_t launch_pack(const uint8_t* nib, const uint8_t* scl, int E, int N, int K, uint8_t* packed,
                       bool unpack, uint8_t* nib_out, uint8_t* scl_out, hipStream_t s);
hipError_t launch_group(const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                        const float* a_w, int R, int E, int S, int T, int32_t* expert_offsets,
                        int32_t* row_src, int32_t* row_dst, float* row_w, int32_t* tok_off,
                        int32_t* tok_rows, int32_t* err_word, hipStream_t s,
                        int4* items = nullptr);
hipError_t launch_gather(const uint16_t* x, int H, const int32_t* row_src, int R, uint16_t* xg,
                         hipStream_t s);
// Output row i quantizes input row row_map[i] (row_map == nullptr: row i); rows at or past
// *row_limit (row_limit != nullptr) and rows mapped to a negative index are all-zero rows.
hipError_t launch_quantize(const uint16_t* in, const int32_t* row_map, const int32_t* row_limit,
                           int R, int K, uint8_t* q, uint8_t* sc, float* row_gs, hipStream_t s);
// row_gs of grouped row i is row_gs[gs_map[i]] (gs_map == nullptr: row_gs[i]).
hipError_t launch_swiglu(const float* acc13, int R, int I, const int32_t* expert_offsets, int E,
                         const float* g_gate, const float* g_up, const float* row_gs,
                         const int32_t* gs_map, uint16_t* h, uint8_t* q, uint8_t* sc,
                         float* h_gs, hipStream_t s);
// Activation row of grouped row i is amap[i] (amap == nullptr: row i) of a_rows rows.
// With c_w: grouped row i of expert e is multiplied by the fp32 product
// c_w[i] * c_g[e] * c_gs[i] (each term of the scatter-add).
// R: the grouped rows (expert_offsets[E] <= R), which bounds the non-empty groups.
// items: the grouping's work list (kWorkListMultiRows) for this batch, or nullptr.
hipError_t launch_grouped_gemm(const uint8_t* aq, const uint8_t* as, const int32_t* amap,
                               int a_rows, const int32_t* expert_offsets, int E, int R,
                               const uint8_t* w, int N, int K, float* out, int flags,
                               int gemv_max_rows, hipStream_t s, const float* c_w = nullptr,
                               const float* c_g = nullptr, const float* c_gs = nullptr,
                               const int4* items = nullptr);
// The layer's w13 GEMM with the SwiGLU epilogue, the NVFP4 quantization of h and the w2
// GEMM with the scatter-ready epilogue in one launch (MFMA path for every group, the
// grouping's work list `items`): h [R, I] bf16, hq / hs / hgs and the terms [R, H] are the
// bits of launch_grouped_gemm_swiglu + launch_quantize + launch_grouped_gemm.  sync:
// grouped_gemm_layer_sync_ints(E, R, H, I) ints, zero on entry (launch_group_quantize
// clears them); err: the device error word (MOE_ERR_SYNC is ORed in if a bounded wait gave
// up).  Only where grouped_gemm_layer_fits(E, R, H, I).
bool grouped_gemm_layer_fits(int E, int R, int H, int I);
int grouped_gemm_layer_sync_ints(int E, int R, int H, int I);  // 0 where it does not fit
hipError_t launch_grouped_gemm_layer(const uint8_t* xq, const uint8_t* xs, const int32_t* row_src,
                                     int S, const int32_t* off, int E, int R, const uint8_t* w13,
                                     const uint8_t* w2, int I, int H, const float* g_gate,
                                     const float* g_up, const float* xgs, uint16_t* h,
                                     uint8_t* hq, uint8_t* hs, float* hgs, const float* row_w,
                                     const float* g_down, float* terms, const int4* items,
                                     int* sync, int32_t* err, hipStream_t s);
// The w13 GEMM with SwiGLU applied in its epilogue (MFMA path for every group): the
// fused [2I, K] gate|up weights give h [R, I] bf16 for the grouped rows, equal bit for bit
// to launch_grouped_gemm followed by launch_swiglu.  Rows outside every group are not
// written.
hipError_t launch_grouped_gemm_swiglu(const uint8_t* aq, const uint8_t* as, const int32_t* amap,
                                      int a_rows, const int32_t* expert_offsets, int E, int R,
                                      const uint8_t* w13, int I, int K, const float* g_gate,
                                      const float* g_up, const float* row_gs,
                                      const int32_t* gs_map, uint16_t* h, hipStream_t s,
                                      const int4* items = nullptr);
// The same for a batch of 1..32 assignments, with the grouping of launch_group and the
// quantization of the source rows x [S, K] done inside the launch (the grouping outputs are
// written as launch_group writes them, with the work list in items (E + 1 entries, or
// nullptr); the quantized rows stay in LDS).  bf16_acts: the W4A16 arithmetic
// (launch_grouped_gemm_swiglu_w4a16), the rows used as bf16.
hipError_t launch_grouped_gemm_swiglu_grouping(const int32_t* a_expert, const int32_t* a_src,
                                               const int32_t* a_dst, const float* a_w, int R,
                                               int E, int S, int T, const uint16_t* x,
                                               int32_t* expert_offsets, int32_t* row_src,
                                               int32_t* row_dst, float* row_w, int32_t* tok_off,
                                               int32_t* tok_rows, int32_t* err_word,
                                               const uint8_t* w13, int I, int K,
                                               const float* g_gate, const float* g_up,
                                               uint16_t* h, hipStream_t s, bool bf16_acts,
                                               int4* items);
// The w2 GEMM with the scatter-ready epilogue for a batch of 1..32 grouped rows, quantizing
// its rows of h [R, K] (bf16, grouped order) itself: the bits of launch_quantize on h
// followed by launch_grouped_gemm with c_gs = the quantized rows' globals.  items: the
// work list launch_grouped_gemm_swiglu_grouping wrote for this batch, or nullptr;
// one_source: the batch has a single source row (its groups are then one row each as a
// rule, which the launch uses to load rows of h early).
hipError_t launch_grouped_gemm_quantizing(const uint16_t* h, const int32_t* expert_offsets,
                                          int E, int R, const uint8_t* w2, int N, int K,
                                          float* out, const float* row_w, const float* g_down,
                                          hipStream_t s, const int4* items, bool one_source = false);
// A batch of at most 16 expert-rows: the w2 GEMM of launch_grouped_gemm_quantizing and the
// per-token sum of launch_token_sum in one launch (no scatter terms in global memory), the
// same bits; items: the work list launch_grouped_gemm_swiglu_grouping wrote (required).
// grouped_gemm_quantizing_sum_fits: whether the launch takes R rows at this K.
bool grouped_gemm_quantizing_sum_fits(int R, int K);
// The same for the W4A16 layer: the W4A16 w2 GEMM over bf16 rows of h [R, K] and the
// per-token sum in one launch, the bits of launch_grouped_gemm_w4a16 + launch_token_sum.
bool grouped_gemm_w4a16_sum_fits(int R, int K);
hipError_t launch_grouped_gemm_w4a16_sum(const uint16_t* h, int E, int R, const uint8_t* w2,
                                         int N, int K, const float* row_w, const float* g_down,
                                         const int4* items, const int32_t* tok_off,
                                         const int32_t* tok_rows, int T, uint16_t* out,
                                         hipStream_t s);
hipError_t launch_grouped_gemm_quantizing_sum(const uint16_t* h, int E, int R, const uint8_t* w2,
                                              int N, int K, const float* row_w,
                                              const float* g_down, const int4* items,
                                              const int32_t* tok_off, const int32_t* tok_rows,
                                              int T, uint16_t* out, hipStream_t s);
// W4A16 (bf16 activation rows ab [a_rows, K], through amap): the grouped GEMM (with c_w,
// rows multiplied by c_w[i] * c_g[e]) and the w13 GEMM with the SwiGLU epilogue (gate / up
// globals alone).
hipError_t launch_grouped_gemm_w4a16(const uint16_t* ab, const int32_t* amap, int a_rows,
                                     const int32_t* expert_offsets, int E, int R, const uint8_t* w,
                                     int N, int K, float* out, hipStream_t s,
                                     const float* c_w = nullptr, const float* c_g = nullptr,
                                     const int4* items = nullptr);
hipError_t launch_grouped_gemm_swiglu_w4a16(const uint16_t* ab, const int32_t* amap, int a_rows,
                                            const int32_t* expert_offsets, int E, int R,
                                            const uint8_t* w13, int I, int K, const float* g_gate,
                                            const float* g_up, uint16_t* h, hipStream_t s,
                                            const int4* items = nullptr);
// Grouping and NVFP4 quantization of the S source rows of x in one launch (independent
// work: block 0 groups, the other blocks quantize four rows each).  items (E + 1 entries,
// or nullptr): for more than 32 assignments, also the grouped GEMM's work list (see
// kWorkListMultiRows).  zero[0 .. nzero) is cleared (the fused GEMM launch's counters).
hipError_t launch_group_quantize(const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                                 const float* a_w, int R, int E, int S, int T,
                                 int32_t* expert_offsets, int32_t* row_src, int32_t* row_dst,
                                 float* row_w, int32_t* tok_off, int32_t* tok_rows,
                                 int32_t* err_word, const uint16_t* x, int H, uint8_t* xq,
                                 uint8_t* xs, float* xgs, int4* items, hipStream_t s,
                                 int* zero = nullptr, int nzero = 0);
hipError_t launch_scatter(const float* y, int R, int H, const int32_t* expert_offsets, int E,
                          const float* row_w, const float* g_down, const float* row_gs,
                          const int32_t* tok_off, const int32_t* tok_rows, int T, uint16_t* out,
                          hipStream_t s);
// out[t] = bf16(sum of rows yc[tok_rows[p]], p = tok_off[t] .. tok_off[t+1] - 1), in
// launch_scatter's order, for terms already scaled (the scatter-ready GEMM output).
hipError_t launch_token_sum(const float* yc, int R, int H, const int32_t* tok_off,
                            const int32_t* tok_rows, int T, uint16_t* out, hipStream_t s);
}  // namespace moe
