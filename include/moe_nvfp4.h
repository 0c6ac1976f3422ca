/* moe_nvfp4.h — C ABI of the NVFP4 routed-expert MoE layer library for AMD MI355X (gfx950).
 *
 * The library implements the routed-expert loop that the page "The CUTLASS grouped GEMM
 * beats the scalar GEMV loop at every M, M=1 included, so the crossover is 1"
 * (gabewillen.github.io/rocket, posts/runtime; cited below as [GG]) lays out in its
 * section "What changed":
 *
 *   gather -> NVFP4 quantize -> grouped GEMM over the fused gate|up weights (w13)
 *   -> SwiGLU with separate gate / up globals -> NVFP4 quantize -> grouped GEMM over w2
 *   -> scatter-add weighted by router weight * down global.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless the comment says "host".  bf16 values are passed
 *   as their uint16_t bit patterns.  The caller allocates and owns every buffer; the
 *   library allocates nothing and is reentrant.  Its one piece of global state is the
 *   fixed scratch array of moe_layer_forward_noalloc (one per GPU).
 * - Every call is asynchronous on the given stream: it validates its arguments on the
 *   host, enqueues kernels and returns.  Only moe_get_device_error() synchronizes.
 * - Return value: MOE_OK (0) or a negative moe_status.  Argument errors (null pointers
 *   with a non-zero size, unsupported shapes, misalignment, a workspace that is too
 *   small) are detected on the host BEFORE anything is enqueued.  A failed launch returns
 *   MOE_EHIP.  moe_last_error() gives the text of the last failure on the calling thread.
 * - Data errors that only the device can see (an expert id, source row or output row out
 *   of range) never fault: the offending assignment is dropped and a bit is set in a
 *   device error word (MOE_ERR_*), which moe_get_device_error() reads back.
 * - Inputs must be finite; NaN / Inf inputs give unspecified (but deterministic) output.
 * - Results are deterministic: repeated calls with identical inputs give bit-identical
 *   outputs (no floating-point atomics anywhere).
 *
 * NVFP4 (page "Fusing the MoE layer's two grouped GEMMs is worth 4%, and a CUDA graph
 * already collects it", gabewillen.github.io/rocket, posts/kernels, cited below as [MF]; table
 * "Bytes decide it before the kernel runs" and section "Different globals on the two
 * halves"): e2m1 elements, two per byte with the even element in the low nibble; one
 * e4m3fn scale byte per 16 consecutive elements along K; one fp32 global per activation
 * row and per weight projection.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument: null pointer, negative size, misalignment */
  MOE_EUNSUPPORTED = -2,  /* shape this library cannot run (see each call's limits) */
  MOE_EHIP = -3,          /* a HIP launch or runtime call failed */
  MOE_EWORKSPACE = -4     /* workspace smaller than the matching *_workspace_bytes() */
} moe_status;

/* flags of grouped_gemm_nvfp4 / moe_layer_desc: how each expert group is computed */
enum {
  MOE_PATH_AUTO = 0,        /* groups of <= gemv_max_rows rows: GEMV; larger: MFMA */
  MOE_PATH_FORCE_GEMV = 1,  /* every group on the wavefront-reduction GEMV */
  MOE_PATH_FORCE_MFMA = 2   /* every group on the MFMA path */
};

/* bits of the device error word.  MOE_ERR_SYNC: inside moe_layer_forward's one-launch
 * GEMM pair (batches of more than 32 assignments), a workgroup gave up waiting for the
 * work it depends on (its group's part of h, or the group's quantized rows of h: a bounded
 * wait that does not end in a correct run); that call's output is then not valid. */
enum { MOE_ERR_EXPERT = 1, MOE_ERR_SRC = 2, MOE_ERR_DST = 4, MOE_ERR_SYNC = 8 };

/* ----------------------------------------------------------------------------------
 * Weight packing (load time).  The grouped GEMM reads expert weights in a layout of
 * this library's own, written once when the weights are loaded — the counterpart of
 * the expert-cache fill in section "The seam CUTLASS forced open" of [GG], which writes
 * the scale layout its GEMM needs once per projection.
 *
 * nvfp4_packed_weight_bytes: host query, bytes of the packed form of E matrices of
 *   [N, K] (exactly E*N*K*9/16: no padding).  Returns 0 if the shape is unsupported.
 *
 * nvfp4_pack_weights: nib [E, N, K/2] canonical e2m1 bytes (row-major, even element in
 *   the low nibble), scl [E, N, K/16] e4m3 scale bytes (row-major) -> packed
 *   [nvfp4_packed_weight_bytes(E, N, K)] bytes, 16-byte aligned.  Values are unchanged:
 *   it is a byte permutation, except that a block whose scale is negative is stored with
 *   the scale's magnitude and the signs of its 16 e2m1 codes flipped (the same 16 values
 *   bit for bit, negative zero included), so that packed scales are never negative.
 *   Because the packed form is a sequence of independent 16-row tiles, packing a fused
 *   [2I, K] gate|up matrix gives the concatenation of the packed gate and up matrices
 *   whenever I % 16 == 0.
 *   Limits: N % 16 == 0, K % 128 == 0, E >= 1.
 *
 * nvfp4_unpack_weights: inverse of nvfp4_pack_weights (same limits): returns the packed
 *   bytes in canonical order — the original bytes when no block scale was negative, else
 *   the value-identical form described above.
 * ---------------------------------------------------------------------------------- */
size_t nvfp4_packed_weight_bytes(int E, int N, int K);
int nvfp4_pack_weights(const uint8_t* nib, const uint8_t* scl, int E, int N, int K,
                       void* packed, hipStream_t stream);
int nvfp4_unpack_weights(const void* packed, int E, int N, int K,
                         uint8_t* nib, uint8_t* scl, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * moe_gather_rows — group assignments by expert and gather their activation rows.
 * Source: [GG], section "What changed": one row per (stream, expert) is
 * gathered, and the batch's rows are grouped per expert in ascending expert id (the
 * pages use an ordered map), so the group order is set by which experts received rows.
 *
 * Inputs:  x [S, H] bf16; assignment j = (a_expert[j], a_src[j], a_dst[j], a_w[j]),
 *          j < R: row a_src[j] of x goes to expert a_expert[j]; its result is added to
 *          output row a_dst[j] (of T) with router weight a_w[j].
 * Outputs: grouped row i (i < R) is the i-th assignment in (expert id, j) order.
 *          expert_offsets [E+1]: rows of expert e are [expert_offsets[e],
 *            expert_offsets[e+1]); expert_offsets[E] = number of valid rows Rv.
 *          row_src, row_dst [R] int32, row_w [R] float: the assignment's fields.
 *          tok_off [T+1], tok_rows [R]: token CSR — tok_rows[tok_off[t] ..
 *            tok_off[t+1]) lists the grouped rows with row_dst == t, ascending.
 *          xg [R, H] bf16: xg[i] = x[row_src[i]].
 *          err_word (one int32): overwritten with the OR of MOE_ERR_* bits found.
 *          Invalid assignments (expert, source or output row out of range) are
 *          dropped: they fill rows [Rv, R) in ascending j with row_src = row_dst = -1,
 *          row_w = 0 and a zero xg row, and are in no token's list.
 * Limits:  R >= 0, S >= 0, 1 <= E <= 8192, 0 <= T, E + T <= 16000, H % 8 == 0.
 * ---------------------------------------------------------------------------------- */
int moe_gather_rows(const uint16_t* x, int S, int H,
                    const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                    const float* a_w, int R, int E, int T,
                    uint16_t* xg, int32_t* expert_offsets, int32_t* row_src,
                    int32_t* row_dst, float* row_w, int32_t* tok_off, int32_t* tok_rows,
                    int32_t* err_word, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * nvfp4_quantize_rows — NVFP4-quantize each bf16 row with its own fp32 global.
 * Source: [GG], section "What changed" (the two quantize steps; the FP4
 * tensor-core GEMM takes FP4 on both operands, section "Numbers").  The pages give no
 * quantizer formula; this one is the two-level NVFP4 reading, in float32, in this order:
 *   amax = max|x|; gs = amax / 2688 (1 if amax == 0)                 [2688 = 6 * 448]
 *   per 16-block b: sf = max|x_b| / (6 * gs); sc[b] = e4m3fn(sf), nearest-even, saturating
 *                   d = value(sc[b]) * gs
 *   per element:    code = e2m1(x / d), nearest-even, saturating, sign kept; 0 if d == 0
 * so that value = e2m1(code) * e4m3(sc[b]) * gs.  Output is bit-exact: every division
 * is the correctly rounded IEEE one.
 *
 * in [R, K] bf16 -> q [R, K/2] (even element in the low nibble), sc [R, K/16],
 * row_gs [R] float.  Limits: K % 16 == 0, 0 < K <= 8192, R >= 0; in 16-byte and q 8-byte
 * aligned.
 * ---------------------------------------------------------------------------------- */
int nvfp4_quantize_rows(const uint16_t* in, int R, int K,
                        uint8_t* q, uint8_t* sc, float* row_gs, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * grouped_gemm_nvfp4 — out[i, n] = sum_k a(i, k) * w_e(n, k) for every row i of every
 * expert group e, with a = e2m1(aq) * e4m3(as) and w = e2m1 * e4m3 of expert e's packed
 * weights; no globals (alpha = 1).
 * Source: [GG], section "What changed": grouped GEMM w13 (N = 2I = 4096,
 * K = H = 4096, fused gate|up) and w2 (N = H, K = I), alpha = 1.
 *
 * aq [R, K/2], as [R, K/16]: NVFP4 activation rows (as written by nvfp4_quantize_rows).
 * expert_offsets [E+1] (device): groups as written by moe_gather_rows.
 * w_packed: E experts of [N, K] packed by nvfp4_pack_weights.  out [R, N] float.
 * Rows outside every group are not written.  Empty experts cost nothing.
 * flags: MOE_PATH_*; gemv_max_rows: largest group taken by the GEMV path under
 *   MOE_PATH_AUTO (0 = never).  Accumulation is fp32 in an order fixed by (N, K) and the
 *   path alone, so a row's output does not depend on the other rows of its group.
 * Limits: N % 16 == 0, K % 128 == 0, E <= 8192, 16-byte aligned pointers.
 * ---------------------------------------------------------------------------------- */
int grouped_gemm_nvfp4(const uint8_t* aq, const uint8_t* as, const int32_t* expert_offsets,
                       int E, int R, const void* w_packed, int N, int K, float* out,
                       int flags, int gemv_max_rows, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * grouped_gemm_w4a16 — out[i, n] = sum_k x(i, k) * w_e(n, k) for every row i of every
 * expert group e, with x the bf16 activation values taken exactly (no quantization) and
 * w = e2m1 * e4m3 of expert e's packed weights; no globals (alpha = 1).
 * Source: [GG], section "Numbers": the dequant-GEMV path computes W4A16, exact BF16
 * activations against an NVFP4 weight; here that arithmetic runs as a grouped GEMM over
 * the same packed weights as grouped_gemm_nvfp4.
 *
 * a [R, K] bf16: the grouped activation rows.  expert_offsets [E+1] (device), w_packed as
 * for grouped_gemm_nvfp4, out [R, N] float.  Rows outside every group are not written.
 * Every group runs on the bf16 matrix cores; the products are exact and accumulate in
 * fp32 in an order fixed by (N, K) alone, so a row's output does not depend on the other
 * rows of its group or batch.
 * Limits: N % 16 == 0, K % 128 == 0, K <= 4096, R * K * 2 < 2^31, E <= 8192, 16-byte
 * aligned pointers.
 * ---------------------------------------------------------------------------------- */
int grouped_gemm_w4a16(const uint16_t* a, const int32_t* expert_offsets, int E, int R,
                       const void* w_packed, int N, int K, float* out, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * swiglu_grouped — h[i, j] = bf16( silu(zg) * zu ), for row i of expert e:
 *   zg = row_gs[i] * g_gate[e] * acc13[i, j],  zu = row_gs[i] * g_up[e] * acc13[i, I + j].
 * Source: [GG], section "What changed" (per-group gate/up weight_scale_2
 * applied in the SwiGLU kernel); [MF], section "Different globals on the two
 * halves", option (a).  row_gs is the activation row global of the w13 GEMM's input.
 *
 * acc13 [R, 2I] float (gate in columns [0, I), up in [I, 2I)), expert_offsets [E+1],
 * g_gate / g_up [E] float, row_gs [R] float -> h [R, I] bf16.  Rows outside every group
 * are written as zeros.  Limits: I % 16 == 0, I <= 8192, E <= 8192.
 * ---------------------------------------------------------------------------------- */
int swiglu_grouped(const float* acc13, int R, int I, const int32_t* expert_offsets, int E,
                   const float* g_gate, const float* g_up, const float* row_gs,
                   uint16_t* h, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * moe_scatter_add — out[t] = bf16( sum over p in [tok_off[t], tok_off[t+1]) of
 *   row_w[i] * g_down[e_i] * row_gs[i] * y[i] ),  i = tok_rows[p].
 * Source: [GG], section "What changed" (scatter-add weighted by router weight
 * * down weight_scale_2) and section "Proof" (shared accumulator row, accumulated in
 * order of i).  row_gs is the activation row global of the w2 GEMM's input.
 *
 * y [R, H] float, expert_offsets [E+1], row_w [R], g_down [E], row_gs [R],
 * tok_off [T+1], tok_rows -> out [T, H] bf16 (every row written; empty tokens are 0).
 * Accumulation is fp32 in a fixed order that depends only on the token's row count
 * (eight interleaved ascending partial sums, added in order), so a token's output does
 * not depend on the rest of the batch.  Limits: H % 4 == 0.
 * ---------------------------------------------------------------------------------- */
int moe_scatter_add(const float* y, int R, int H, const int32_t* expert_offsets, int E,
                    const float* row_w, const float* g_down, const float* row_gs,
                    const int32_t* tok_off, const int32_t* tok_rows, int T,
                    uint16_t* out, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * moe_layer_forward — the whole routed-expert layer: every step above, in order, on
 * one stream, with no host synchronization ([GG], section "What changed").
 * The S source rows are quantized once each, in the same launch as the grouping, and the
 * w13 GEMM reads grouped row i from source row row_src[i] (a row's codes depend only on
 * the row, so this equals gather-then-quantize).  When every group runs on the MFMA path
 * (the default), SwiGLU runs in the w13 GEMM's epilogue and h is quantized by one small
 * launch; with GEMV groups, SwiGLU and the second quantization are one kernel.  A batch
 * of 1 to 32 assignments on the MFMA path has no grouping and no quantization launch: each
 * workgroup of the w13 GEMM groups the assignments and quantizes its group's source rows
 * itself (one more workgroup writes the grouping's outputs to the workspace for the later
 * launches), and each workgroup of the w2 GEMM quantizes its group's rows of h itself.
 * The w2 GEMM writes each row's weighted scatter term, summed per token by the last launch;
 * with at most 16 assignments (and I <= 1024 or I = 2048; also I = 3072 or 4096 with at
 * most 8 assignments) the w2 launch sums each token's terms itself, and the layer is two
 * launches.  A batch of more than 32 assignments on the MFMA path (H and I multiples of
 * 1024, I <= 2048, and H = 2I or else min(E, R)·I/64 and min(E, R)·H/128 on the same side
 * of 2048; otherwise the five launches of the steps) runs the w13 GEMM, the
 * quantization of h and the w2 GEMM as one launch ([MF], the fusion of the two grouped
 * GEMMs): the w2 workgroups start as the w13 GEMM's last workgroups finish, each waiting,
 * with a bounded wait, until its group's rows of h are quantized (MOE_ERR_SYNC if a wait
 * gave up), and the layer is three launches.  The results are bit-identical to calling the
 * separate entry points in sequence.
 *
 * L (host): E, H, I; w13_packed (E x [2I, H], gate rows first) and w2_packed
 *   (E x [H, I]) from nvfp4_pack_weights; per-expert globals g_gate, g_up, g_down [E];
 *   flags / gemv_max_rows as for grouped_gemm_nvfp4.
 * x [S, H] bf16, assignments as for moe_gather_rows, out [T, H] bf16.
 * workspace: >= moe_layer_workspace_bytes(L, S, R, T) bytes, 256-byte aligned.  Its
 *   first int32 is the device error word (pass the workspace to moe_get_device_error).
 * Limits: H % 128 == 0, I % 128 == 0, H and I <= 8192, max(S, R) * H < 2^31 and
 * R * I < 2^31 (the NVFP4 rows a GEMM stages are addressed with 32-bit offsets), plus
 * those of the steps.
 * ---------------------------------------------------------------------------------- */
typedef struct {
  int E, H, I;
  const void* w13_packed;
  const void* w2_packed;
  const float* g_gate;
  const float* g_up;
  const float* g_down;
  int flags;
  int gemv_max_rows;
} moe_layer_desc;

size_t moe_layer_workspace_bytes(const moe_layer_desc* L, int S, int R, int T);
int moe_layer_forward(const moe_layer_desc* L, const uint16_t* x, int S,
                      const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                      const float* a_w, int R, int T, uint16_t* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * moe_layer_forward_noalloc — moe_layer_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same launches and bit-identical results, with the workspace taken from
 * a fixed array the library holds on each GPU (MOE_NOALLOC_SCRATCH_BYTES, allocated with
 * the library's code object on a GPU and held until the process ends) instead of a caller
 * buffer.  It calls no allocating routine; its first call on a device looks up that
 * device's array address once (hipGetSymbolAddress).
 * Same arguments as moe_layer_forward minus the workspace, plus
 * err_word: a device int32 that receives this call's MOE_ERR_* bits (read it with
 *   moe_get_device_error), or NULL to discard them.
 * Returns MOE_EUNSUPPORTED, before any launch, when the call needs more scratch than the
 * array holds (moe_layer_workspace_bytes() > MOE_NOALLOC_SCRATCH_BYTES; at E = 288,
 * H = 4096, I = 2048 and S = R, that is beyond 2,800 rows).  Nothing in the array has to start at any
 * value (every byte a call reads was written earlier in the same call), so nothing is
 * cleared.  Calls on one GPU share its array: calls that can overlap on one GPU (other
 * streams, other threads) race and must be serialized by the caller.
 * ---------------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_layer_desc* L, const uint16_t* x, int S,
                              const int32_t* a_expert, const int32_t* a_src,
                              const int32_t* a_dst, const float* a_w, int R, int T,
                              uint16_t* out, int32_t* err_word, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * moe_layer_forward_w4a16 — the routed-expert layer in W4A16 arithmetic: the steps of
 * moe_layer_forward without the two activation quantizations ([GG], section "Numbers":
 * W4A16 is the arithmetic of the dequant-GEMV path).  Grouping; the w13 GEMM over the
 * bf16 source rows (grouped row i reads source row row_src[i]) with SwiGLU in its
 * epilogue, h = bf16( silu(g_gate[e] * acc_gate) * g_up[e] * acc_up ) (bf16 activations
 * carry no row global); the w2 GEMM over bf16 h; the scatter-add weighted by
 * row_w[i] * g_down[e].  A batch of 1 to 32 assignments has no grouping launch: each
 * workgroup of the w13 GEMM groups the assignments itself (one more workgroup writes the
 * grouping's outputs to the workspace), with the same results.
 * Same descriptor (flags and gemv_max_rows are not used: every group runs on the bf16
 * matrix cores), arguments, workspace (moe_layer_workspace_bytes) and error word as
 * moe_layer_forward.  Limits: those of moe_layer_forward, plus H <= 4096 and I <= 4096.
 * ---------------------------------------------------------------------------------- */
int moe_layer_forward_w4a16(const moe_layer_desc* L, const uint16_t* x, int S,
                            const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                            const float* a_w, int R, int T, uint16_t* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------------------
 * moe_hbm_read_probe — a measurement aid, not a step of the layer: reads `bytes` bytes
 * at `src` once, with non-temporal 16-byte loads per lane, so that the time of the launch
 * gives the HBM read bandwidth this GPU actually reaches — the measured read roofline the
 * weight-streaming GEMMs are judged against ([MF], table "Bytes decide it before the
 * kernel runs": the pages' layer roofline comes from a measured read bandwidth, below the
 * spec; section "Next": profile the w13 GEMM against a raw read of the same access
 * pattern).
 * variant (0 <= variant < moe_hbm_read_probe_variants()): 0, 1, 2: each wave streams a
 *   contiguous run with 8, 16 or 16 KiB of loads in flight, 32, 32 or 16 waves per CU;
 *   3: the w13 GEMM's pattern: one workgroup of 4 waves per 288 KiB item of 8 tiles of
 *   36 KiB, each wave walking two tiles side by side with 4 KiB of each in flight;
 *   4: contiguous runs with 32 KiB in flight per wave, 32 waves per CU.
 * bytes: a positive multiple of 294,912 (one such item); src 16-byte aligned.
 * sink: one device uint32, written only if a lane's XOR of the data it read equals `key`
 *   (it keeps the loads alive; its value means nothing).
 * ---------------------------------------------------------------------------------- */
int moe_hbm_read_probe(const void* src, size_t bytes, int variant, uint32_t key,
                       uint32_t* sink, hipStream_t stream);
int moe_hbm_read_probe_variants(void);

/* Synchronizes `stream`, then returns the device error word at `err_word` (the
 * err_word of moe_gather_rows, or a moe_layer_forward workspace), or a negative
 * moe_status if the read fails. */
int moe_get_device_error(const void* err_word, hipStream_t stream);

/* Text of the last failure on the calling thread ("" if none).  Host pointer, valid
 * until the thread's next call into the library. */
const char* moe_last_error(void);

/* Host string: hash of the sources this library was built from.  Bindings compare it
 * with the sources on disk so that a stale build is refused instead of silently run
 * ([GG], section "A debugging note", lost a day to a stale test binary). */
const char* moe_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
