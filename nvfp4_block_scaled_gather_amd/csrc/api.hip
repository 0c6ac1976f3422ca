// C ABI of the library (declared in include/moe_nvfp4.h): argument validation on the
// host, then kernel launches on the caller's stream.  No allocation, no synchronization
// (except moe_get_device_error); the only state is the per-device address of the fixed
// scratch array of moe_layer_forward_noalloc.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace moe {
// HBM read probe (k_probe.hip): bytes a multiple of 294,912, variant in [0, probe_variants()).
int probe_variants();
hipError_t launch_read_probe(const uint8_t* src, size_t bytes, int variant, uint32_t key,
                             uint32_t* sink, hipStream_t s);
}  // namespace moe

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE(cond, code, ...)                 \
  do {                                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

// Scratch of moe_layer_forward_noalloc: one array per GPU, held by the loaded code object
// until the process ends.  In host code `scratch` only names the symbol; its device address
// comes from hipGetSymbolAddress, once per device, and only that address is ever used.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the first call there).
int scratch_on_current_device(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "layer (no allocation): hipGetDevice");
  REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_EUNSUPPORTED,
          "layer (no allocation): device %d beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "layer (no allocation): hipGetSymbolAddress(scratch)");
    REQUIRE(p && aligned(p, 256), MOE_EHIP, "layer (no allocation): scratch address %p unusable", p);
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

constexpr int kMaxGroupKeys = 16000;  // E + T, LDS histograms of the grouping kernel
constexpr int kMaxRowK = 8192;        // row kernels keep a row in registers
constexpr int kMaxE = 8192;
constexpr int kMaxBf16K = 4096;       // W4A16: 16 staged bf16 rows of K must fit in LDS
constexpr size_t kProbeUnit = 294912; // read probe: one GEMM work item (8 tiles of 36 KiB)

int check_group_args(const void* a_expert, const void* a_src, const void* a_dst, const void* a_w,
                     int R, int E, int S, int T, const void* expert_offsets, const void* row_src,
                     const void* row_dst, const void* row_w, const void* tok_off,
                     const void* tok_rows, const void* err_word) {
  REQUIRE(R >= 0 && S >= 0 && T >= 0, MOE_EINVAL, "negative size (R=%d S=%d T=%d)", R, S, T);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_EUNSUPPORTED, "E=%d outside [1, %d]", E, kMaxE);
  REQUIRE(E + T <= kMaxGroupKeys, MOE_EUNSUPPORTED, "E + T = %d exceeds %d", E + T, kMaxGroupKeys);
  REQUIRE(expert_offsets && tok_off && err_word, MOE_EINVAL, "null offsets / tok_off / err_word");
  if (R > 0) {
    REQUIRE(a_expert && a_src && a_dst && a_w, MOE_EINVAL, "null assignment array");
    REQUIRE(row_src && row_dst && row_w && tok_rows, MOE_EINVAL, "null row array");
  }
  REQUIRE(aligned(expert_offsets, 4) && aligned(row_src, 4) && aligned(row_dst, 4) &&
              aligned(row_w, 4) && aligned(tok_off, 4) && aligned(tok_rows, 4) &&
              aligned(err_word, 4) && aligned(a_expert, 4) && aligned(a_src, 4) &&
              aligned(a_dst, 4) && aligned(a_w, 4),
          MOE_EINVAL, "int32/float arrays must be 4-byte aligned");
  return MOE_OK;
}

int check_gemm_args(const void* aq, const void* as, const void* off, int E, int R, const void* w,
                    int N, int K, const void* out, int flags, int gemv_max_rows) {
  REQUIRE(R >= 0 && N > 0 && K > 0, MOE_EINVAL, "bad sizes (R=%d N=%d K=%d)", R, N, K);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_EUNSUPPORTED, "E=%d outside [1, %d]", E, kMaxE);
  REQUIRE(N % 16 == 0, MOE_EUNSUPPORTED, "N=%d must be a multiple of 16", N);
  REQUIRE(K % 128 == 0, MOE_EUNSUPPORTED, "K=%d must be a multiple of 128", K);
  REQUIRE(flags == MOE_PATH_AUTO || flags == MOE_PATH_FORCE_GEMV || flags == MOE_PATH_FORCE_MFMA,
          MOE_EINVAL, "unknown flags %d", flags);
  REQUIRE(gemv_max_rows >= 0, MOE_EINVAL, "gemv_max_rows=%d < 0", gemv_max_rows);
  REQUIRE(off && w, MOE_EINVAL, "null expert_offsets / weights");
  if (R > 0) REQUIRE(aq && as && out, MOE_EINVAL, "null activation / output");
  REQUIRE(aligned(aq, 16) && aligned(w, 16) && aligned(out, 16) && aligned(as, 2) &&
              aligned(off, 4),
          MOE_EINVAL, "aq, weights and out must be 16-byte aligned");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

#ifndef MOE_SOURCE_HASH
#define MOE_SOURCE_HASH "unknown"
#endif
const char* moe_source_hash(void) { return MOE_SOURCE_HASH; }

size_t nvfp4_packed_weight_bytes(int E, int N, int K) {
  if (E < 1 || N <= 0 || K <= 0 || N % 16 || K % 128) return 0;
  return (size_t)E * N * K / 16 * 9;
}

int nvfp4_pack_weights(const uint8_t* nib, const uint8_t* scl, int E, int N, int K, void* packed,
                       hipStream_t stream) {
  REQUIRE(nvfp4_packed_weight_bytes(E, N, K) > 0, MOE_EUNSUPPORTED,
          "pack: need E >= 1, N %% 16 == 0, K %% 128 == 0 (E=%d N=%d K=%d)", E, N, K);
  REQUIRE(nib && scl && packed, MOE_EINVAL, "pack: null pointer");
  REQUIRE(aligned(nib, 16) && aligned(packed, 16), MOE_EINVAL, "pack: nibbles / packed not 16-byte aligned");
  return hip_status(moe::launch_pack(nib, scl, E, N, K, (uint8_t*)packed, false, nullptr, nullptr, stream),
                    "pack launch");
}

int nvfp4_unpack_weights(const void* packed, int E, int N, int K, uint8_t* nib, uint8_t* scl,
                         hipStream_t stream) {
  REQUIRE(nvfp4_packed_weight_bytes(E, N, K) > 0, MOE_EUNSUPPORTED,
          "unpack: need E >= 1, N %% 16 == 0, K %% 128 == 0 (E=%d N=%d K=%d)", E, N, K);
  REQUIRE(nib && scl && packed, MOE_EINVAL, "unpack: null pointer");
  REQUIRE(aligned(nib, 16) && aligned(packed, 16), MOE_EINVAL, "unpack: nibbles / packed not 16-byte aligned");
  return hip_status(moe::launch_pack(nullptr, nullptr, E, N, K, (uint8_t*)packed, true, nib, scl, stream),
                    "unpack launch");
}

int moe_gather_rows(const uint16_t* x, int S, int H, const int32_t* a_expert, const int32_t* a_src,
                    const int32_t* a_dst, const float* a_w, int R, int E, int T, uint16_t* xg,
                    int32_t* expert_offsets, int32_t* row_src, int32_t* row_dst, float* row_w,
                    int32_t* tok_off, int32_t* tok_rows, int32_t* err_word, hipStream_t stream) {
  int st = check_group_args(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src,
                            row_dst, row_w, tok_off, tok_rows, err_word);
  if (st != MOE_OK) return st;
  REQUIRE(H > 0 && H % 8 == 0, MOE_EUNSUPPORTED, "gather: H=%d must be a positive multiple of 8", H);
  if (R > 0) REQUIRE(xg, MOE_EINVAL, "gather: null xg");
  if (R > 0 && S > 0) REQUIRE(x, MOE_EINVAL, "gather: null x");
  REQUIRE(aligned(x, 16) && aligned(xg, 16), MOE_EINVAL, "gather: x / xg not 16-byte aligned");
  hipError_t e = moe::launch_group(a_expert, a_src, a_dst, a_w, R, E, S, T, expert_offsets, row_src,
                                   row_dst, row_w, tok_off, tok_rows, err_word, stream);
  if (e != hipSuccess) return hip_status(e, "group launch");
  return hip_status(moe::launch_gather(x, H, row_src, R, xg, stream), "gather launch");
}

int nvfp4_quantize_rows(const uint16_t* in, int R, int K, uint8_t* q, uint8_t* sc, float* row_gs,
                        hipStream_t stream) {
  REQUIRE(R >= 0, MOE_EINVAL, "quantize: R=%d < 0", R);
  REQUIRE(K > 0 && K % 16 == 0 && K <= kMaxRowK, MOE_EUNSUPPORTED,
          "quantize: K=%d must be a multiple of 16 in (0, %d]", K, kMaxRowK);
  if (R > 0) REQUIRE(in && q && sc && row_gs, MOE_EINVAL, "quantize: null pointer");
  REQUIRE(aligned(in, 16) && aligned(q, 8) && aligned(row_gs, 4), MOE_EINVAL,
          "quantize: in must be 16-byte and q 8-byte aligned");
  return hip_status(moe::launch_quantize(in, nullptr, nullptr, R, K, q, sc, row_gs, stream), "quantize launch");
}

int grouped_gemm_nvfp4(const uint8_t* aq, const uint8_t* as, const int32_t* expert_offsets, int E,
                       int R, const void* w_packed, int N, int K, float* out, int flags,
                       int gemv_max_rows, hipStream_t stream) {
  int st = check_gemm_args(aq, as, expert_offsets, E, R, w_packed, N, K, out, flags, gemv_max_rows);
  if (st != MOE_OK) return st;
  REQUIRE((long long)R * (K / 2) < (1ll << 31), MOE_EUNSUPPORTED,
          "grouped GEMM: activations of %d rows x %d columns exceed 2 GiB", R, K);
  return hip_status(moe::launch_grouped_gemm(aq, as, nullptr, R, expert_offsets, E, R,
                                             (const uint8_t*)w_packed, N, K, out, flags,
                                             gemv_max_rows, stream),
                    "grouped GEMM launch");
}

int grouped_gemm_w4a16(const uint16_t* a, const int32_t* expert_offsets, int E, int R,
                       const void* w_packed, int N, int K, float* out, hipStream_t stream) {
  int st = check_gemm_args(a, a, expert_offsets, E, R, w_packed, N, K, out, MOE_PATH_FORCE_MFMA, 0);
  if (st != MOE_OK) return st;
  REQUIRE(K <= kMaxBf16K, MOE_EUNSUPPORTED, "W4A16 GEMM: K=%d exceeds %d", K, kMaxBf16K);
  REQUIRE((long long)R * K * 2 < (1ll << 31), MOE_EUNSUPPORTED,
          "W4A16 GEMM: activations of %d rows x %d columns exceed 2 GiB", R, K);
  return hip_status(moe::launch_grouped_gemm_w4a16(a, nullptr, R, expert_offsets, E, R,
                                                   (const uint8_t*)w_packed, N, K, out, stream),
                    "W4A16 grouped GEMM launch");
}

int swiglu_grouped(const float* acc13, int R, int I, const int32_t* expert_offsets, int E,
                   const float* g_gate, const float* g_up, const float* row_gs, uint16_t* h,
                   hipStream_t stream) {
  REQUIRE(R >= 0, MOE_EINVAL, "swiglu: R=%d < 0", R);
  REQUIRE(E >= 1 && E <= kMaxE, MOE_EUNSUPPORTED, "swiglu: E=%d outside [1, %d]", E, kMaxE);
  REQUIRE(I > 0 && I % 16 == 0 && I <= kMaxRowK, MOE_EUNSUPPORTED,
          "swiglu: I=%d must be a multiple of 16 in (0, %d]", I, kMaxRowK);
  REQUIRE(expert_offsets && g_gate && g_up, MOE_EINVAL, "swiglu: null offsets / globals");
  if (R > 0) REQUIRE(acc13 && row_gs && h, MOE_EINVAL, "swiglu: null pointer");
  REQUIRE(aligned(acc13, 16) && aligned(h, 16), MOE_EINVAL, "swiglu: acc13 / h not 16-byte aligned");
  return hip_status(moe::launch_swiglu(acc13, R, I, expert_offsets, E, g_gate, g_up, row_gs, nullptr,
                                       h, nullptr, nullptr, nullptr, stream),
                    "swiglu launch");
}

int moe_scatter_add(const float* y, int R, int H, const int32_t* expert_offsets, int E,
                    const float* row_w, const float* g_down, const float* row_gs,
                    const int32_t* tok_off, const int32_t* tok_rows, int T, uint16_t* out,
                    hipStream_t stream) {
  REQUIRE(R >= 0 && T >= 0, MOE_EINVAL, "scatter: negative size");
  REQUIRE(E >= 1 && E <= kMaxE, MOE_EUNSUPPORTED, "scatter: E=%d outside [1, %d]", E, kMaxE);
  REQUIRE(H > 0 && H % 4 == 0, MOE_EUNSUPPORTED, "scatter: H=%d must be a positive multiple of 4", H);
  REQUIRE(expert_offsets && g_down && tok_off, MOE_EINVAL, "scatter: null offsets / globals / tok_off");
  if (T > 0) REQUIRE(out, MOE_EINVAL, "scatter: null out");
  if (R > 0) REQUIRE(y && row_w && row_gs && tok_rows, MOE_EINVAL, "scatter: null row array");
  REQUIRE(aligned(y, 16) && aligned(out, 8), MOE_EINVAL, "scatter: y must be 16-byte, out 8-byte aligned");
  return hip_status(moe::launch_scatter(y, R, H, expert_offsets, E, row_w, g_down, row_gs, tok_off,
                                        tok_rows, T, out, stream),
                    "scatter launch");
}

// ---------------------------------------------------------------- layer
namespace {
struct LayerWs {
  int32_t* err;
  int32_t* offsets;
  int32_t* row_src;
  int32_t* row_dst;
  float* row_w;
  int32_t* tok_off;
  int32_t* tok_rows;
  uint8_t* xq;
  uint8_t* xs;
  float* xgs;
  float* acc;  // acc13 [R, 2I] (or h [R, I] bf16), later reused for the scatter terms [R, H]
  uint8_t* hq;
  uint8_t* hs;
  float* hgs;
  uint16_t* h16;  // W4A16: h [R, I] bf16 (the w2 GEMM's input while acc takes its output)
  int4* items;    // the grouped GEMMs' work list, E + 1 entries
  int* sync;      // the one-launch GEMM pair's flags (grouped_gemm_layer_sync_ints)
  int nsync;
  size_t bytes;
};

LayerWs carve(const moe_layer_desc* L, int S, int R, int T, uint8_t* base) {
  LayerWs w{};
  size_t o = 0;
  auto take = [&](size_t n) {
    uint8_t* p = base ? base + o : nullptr;
    o = align_up(o + n, 256);
    return p;
  };
  const size_t r = (size_t)R;
  w.err = (int32_t*)take(4);
  w.offsets = (int32_t*)take(4 * ((size_t)L->E + 1));
  w.row_src = (int32_t*)take(4 * r);
  w.row_dst = (int32_t*)take(4 * r);
  w.row_w = (float*)take(4 * r);
  w.tok_off = (int32_t*)take(4 * ((size_t)T + 1));
  w.tok_rows = (int32_t*)take(4 * r);
  const size_t sr = (size_t)S;  // x is quantized once per source row
  w.xq = take(sr * L->H / 2);
  w.xs = take(sr * L->H / 16);
  w.xgs = (float*)take(4 * sr);
  const size_t acc_cols = (size_t)(2 * L->I > L->H ? 2 * L->I : L->H);
  w.acc = (float*)take(4 * r * acc_cols);
  w.hq = take(r * L->I / 2);
  w.hs = take(r * L->I / 16);
  w.hgs = (float*)take(4 * r);
  w.h16 = (uint16_t*)take(2 * r * L->I);
  w.items = (int4*)take(sizeof(int4) * ((size_t)L->E + 1));
  w.nsync = moe::grouped_gemm_layer_sync_ints(L->E, R, L->H, L->I);
  w.sync = (int*)take(4 * (size_t)w.nsync);
  w.bytes = o;
  return w;
}

int check_layer(const moe_layer_desc* L, int S, int R, int T) {
  REQUIRE(L, MOE_EINVAL, "layer: null descriptor");
  REQUIRE(S >= 0 && R >= 0 && T >= 0, MOE_EINVAL, "layer: negative size");
  REQUIRE(L->E >= 1 && L->E <= kMaxE, MOE_EUNSUPPORTED, "layer: E=%d outside [1, %d]", L->E, kMaxE);
  REQUIRE(L->H > 0 && L->H % 128 == 0 && L->H <= kMaxRowK, MOE_EUNSUPPORTED,
          "layer: H=%d must be a multiple of 128 in (0, %d]", L->H, kMaxRowK);
  REQUIRE(L->I > 0 && L->I % 128 == 0 && L->I <= kMaxRowK, MOE_EUNSUPPORTED,
          "layer: I=%d must be a multiple of 128 in (0, %d]", L->I, kMaxRowK);
  REQUIRE(L->E + T <= kMaxGroupKeys, MOE_EUNSUPPORTED, "layer: E + T exceeds %d", kMaxGroupKeys);
  // buffer ranges and offsets of the GEMMs' activation staging are 32-bit: the NVFP4 rows
  // of x (S or R of them, H/2 bytes each) and of h (R rows of I/2 bytes) stay below 2 GiB
  REQUIRE((long long)(S > R ? S : R) * L->H < (1ll << 31), MOE_EUNSUPPORTED,
          "layer: activations exceed 2 GiB of NVFP4 rows");
  REQUIRE((long long)R * L->I < (1ll << 31), MOE_EUNSUPPORTED,
          "layer: %d rows of h (I=%d) exceed 2 GiB of NVFP4 rows", R, L->I);
  return MOE_OK;
}
}  // namespace

size_t moe_layer_workspace_bytes(const moe_layer_desc* L, int S, int R, int T) {
  if (check_layer(L, S, R, T) != MOE_OK) return 0;
  return carve(L, S, R, T, nullptr).bytes;
}

}  // extern "C"

namespace {
// Arguments of moe_layer_forward other than the workspace.
int check_layer_call(const moe_layer_desc* L, const uint16_t* x, int S, const int32_t* a_expert,
                     const int32_t* a_src, const int32_t* a_dst, const float* a_w, int R, int T,
                     const uint16_t* out) {
  int st = check_layer(L, S, R, T);
  if (st != MOE_OK) return st;
  REQUIRE(L->w13_packed && L->w2_packed && L->g_gate && L->g_up && L->g_down, MOE_EINVAL,
          "layer: null weights / globals");
  if (R > 0) REQUIRE(a_expert && a_src && a_dst && a_w, MOE_EINVAL, "layer: null assignment array");
  if (R > 0 && S > 0) REQUIRE(x, MOE_EINVAL, "layer: null x");
  if (T > 0) REQUIRE(out, MOE_EINVAL, "layer: null out");
  REQUIRE(aligned(x, 16) && aligned(out, 8) && aligned(L->w13_packed, 16) && aligned(L->w2_packed, 16),
          MOE_EINVAL, "layer: x / weights must be 16-byte, out 8-byte aligned");
  REQUIRE(L->flags == MOE_PATH_AUTO || L->flags == MOE_PATH_FORCE_GEMV || L->flags == MOE_PATH_FORCE_MFMA,
          MOE_EINVAL, "layer: unknown flags %d", L->flags);
  REQUIRE(L->gemv_max_rows >= 0, MOE_EINVAL, "layer: gemv_max_rows < 0");
  return MOE_OK;
}

// The launches of one layer call over the carved workspace w (arguments already checked).
int run_layer(const moe_layer_desc* L, const uint16_t* x, int S, const int32_t* a_expert,
              const int32_t* a_src, const int32_t* a_dst, const float* a_w, int R, int T,
              uint16_t* out, const LayerWs& w, hipStream_t stream) {
  const int E = L->E, H = L->H, I = L->I;
  hipError_t e;
  const bool all_mfma = L->flags == MOE_PATH_FORCE_MFMA ||
                        (L->flags == MOE_PATH_AUTO && L->gemv_max_rows == 0);
  if (all_mfma && R >= 1 && R <= 32) {
    // A decode-sized batch on the MFMA path, three launches: the w13 GEMM launch groups the
    // assignments and quantizes its rows by itself (writing h to its own buffer, since the
    // w2 launch reads h while writing its terms into acc), the w2 GEMM launch quantizes h
    // by itself, then the per-token sum; up to 16 rows the w2 launch sums the tokens too.
    // Measured on MI355X to save the small launches' time at one to four tokens; the same
    // bits as the sequence below.
    e = moe::launch_grouped_gemm_swiglu_grouping(a_expert, a_src, a_dst, a_w, R, E, S, T, x,
                                                 w.offsets, w.row_src, w.row_dst, w.row_w,
                                                 w.tok_off, w.tok_rows, w.err,
                                                 (const uint8_t*)L->w13_packed, I, H, L->g_gate,
                                                 L->g_up, w.h16, stream, false, w.items);
    if (e != hipSuccess) return hip_status(e, "layer: grouping w13 GEMM + SwiGLU launch");
    if (moe::grouped_gemm_quantizing_sum_fits(R, I)) {
      // at most 16 rows: the w2 launch also sums each token's terms (two launches in all)
      e = moe::launch_grouped_gemm_quantizing_sum(w.h16, E, R, (const uint8_t*)L->w2_packed, H,
                                                  I, w.row_w, L->g_down, w.items, w.tok_off,
                                                  w.tok_rows, T, out, stream);
      return hip_status(e, "layer: quantizing w2 GEMM + per-token sum launch");
    }
    e = moe::launch_grouped_gemm_quantizing(w.h16, w.offsets, E, R, (const uint8_t*)L->w2_packed, H,
                                            I, w.acc, w.row_w, L->g_down, stream, w.items, S == 1);
    if (e != hipSuccess) return hip_status(e, "layer: quantizing w2 GEMM launch");
    e = moe::launch_token_sum(w.acc, R, H, w.tok_off, w.tok_rows, T, out, stream);
    return hip_status(e, "layer: scatter launch");
  }
  // grouping + NVFP4 quantization of the S source rows (one launch); the w13 GEMM reads
  // grouped row i from source row row_src[i], so no gathered copy of x is made
  // (the work list is written and used only when every group is on the MFMA path)
  int4* items = all_mfma && R > 32 ? w.items : nullptr;
  const bool one_launch = all_mfma && R > 32 && moe::grouped_gemm_layer_fits(E, R, H, I);
  e = moe::launch_group_quantize(a_expert, a_src, a_dst, a_w, R, E, S, T, w.offsets, w.row_src,
                                 w.row_dst, w.row_w, w.tok_off, w.tok_rows, w.err, x, H, w.xq,
                                 w.xs, w.xgs, items, stream, one_launch ? w.sync : nullptr,
                                 one_launch ? w.nsync : 0);
  if (e != hipSuccess) return hip_status(e, "layer: group+quantize launch");
  if (one_launch) {
    // more than 32 assignments: w13 + SwiGLU, the quantization of h and w2 in one
    // launch (h in its own buffer, since the w2 items write their terms into acc while
    // other groups' rows of h are still read), then the per-token sum; the same bits
    e = moe::launch_grouped_gemm_layer(w.xq, w.xs, w.row_src, S, w.offsets, E, R,
                                       (const uint8_t*)L->w13_packed,
                                       (const uint8_t*)L->w2_packed, I, H, L->g_gate, L->g_up,
                                       w.xgs, w.h16, w.hq, w.hs, w.hgs, w.row_w, L->g_down, w.acc,
                                       w.items, w.sync, w.err, stream);
    if (e != hipSuccess) return hip_status(e, "layer: fused GEMM launch");
    e = moe::launch_token_sum(w.acc, R, H, w.tok_off, w.tok_rows, T, out, stream);
    return hip_status(e, "layer: scatter launch");
  }
  if (all_mfma) {
    // SwiGLU in the w13 GEMM's epilogue (h in bf16 instead of the fp32 gate|up products),
    // then the NVFP4 quantization of h; the same bits as the unfused sequence below
    uint16_t* h = (uint16_t*)w.acc;
    if (R > 0) {
      e = moe::launch_grouped_gemm_swiglu(w.xq, w.xs, w.row_src, S, w.offsets, E, R,
                                          (const uint8_t*)L->w13_packed, I, H, L->g_gate, L->g_up,
                                          w.xgs, w.row_src, h, stream, items);
      if (e != hipSuccess) return hip_status(e, "layer: w13 GEMM + SwiGLU launch");
    }
    e = moe::launch_quantize(h, nullptr, w.offsets + E, R, I, w.hq, w.hs, w.hgs, stream);
    if (e != hipSuccess) return hip_status(e, "layer: quantize launch");
  } else {
    if (R > 0) {
      e = moe::launch_grouped_gemm(w.xq, w.xs, w.row_src, S, w.offsets, E, R,
                                   (const uint8_t*)L->w13_packed, 2 * I, H, w.acc, L->flags,
                                   L->gemv_max_rows, stream);
      if (e != hipSuccess) return hip_status(e, "layer: w13 GEMM launch");
    }
    e = moe::launch_swiglu(w.acc, R, I, w.offsets, E, L->g_gate, L->g_up, w.xgs, w.row_src, nullptr,
                           w.hq, w.hs, w.hgs, stream);
    if (e != hipSuccess) return hip_status(e, "layer: swiglu+quantize launch");
  }
  // w2 GEMM writing each grouped row's scatter term (row_w * g_down * hgs * y), then a
  // per-token sum over the token lists: the bits of moe_scatter_add on y
  if (R > 0) {
    e = moe::launch_grouped_gemm(w.hq, w.hs, nullptr, R, w.offsets, E, R,
                                 (const uint8_t*)L->w2_packed, H, I, w.acc, L->flags,
                                 L->gemv_max_rows, stream, w.row_w, L->g_down, w.hgs, items);
    if (e != hipSuccess) return hip_status(e, "layer: w2 GEMM launch");
  }
  e = moe::launch_token_sum(w.acc, R, H, w.tok_off, w.tok_rows, T, out, stream);
  return hip_status(e, "layer: scatter launch");
}
}  // namespace

extern "C" {

int moe_layer_forward(const moe_layer_desc* L, const uint16_t* x, int S, const int32_t* a_expert,
                      const int32_t* a_src, const int32_t* a_dst, const float* a_w, int R, int T,
                      uint16_t* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_layer_call(L, x, S, a_expert, a_src, a_dst, a_w, R, T, out);
  if (st != MOE_OK) return st;
  REQUIRE(workspace && aligned(workspace, 256), MOE_EINVAL, "layer: workspace null or not 256-byte aligned");
  const LayerWs w = carve(L, S, R, T, (uint8_t*)workspace);
  REQUIRE(workspace_bytes >= w.bytes, MOE_EWORKSPACE, "layer: workspace %zu bytes < %zu needed",
          workspace_bytes, w.bytes);
  return run_layer(L, x, S, a_expert, a_src, a_dst, a_w, R, T, out, w, stream);
}

int moe_layer_forward_noalloc(const moe_layer_desc* L, const uint16_t* x, int S,
                              const int32_t* a_expert, const int32_t* a_src,
                              const int32_t* a_dst, const float* a_w, int R, int T,
                              uint16_t* out, int32_t* err_word, hipStream_t stream) {
  int st = check_layer_call(L, x, S, a_expert, a_src, a_dst, a_w, R, T, out);
  if (st != MOE_OK) return st;
  REQUIRE(aligned(err_word, 4), MOE_EINVAL, "layer: err_word not 4-byte aligned");
  const size_t need = carve(L, S, R, T, nullptr).bytes;
  REQUIRE(need <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_EUNSUPPORTED,
          "layer (no allocation): this call needs %zu bytes of scratch, more than the library's "
          "fixed %zu-byte array (use moe_layer_forward with a workspace)",
          need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  uint8_t* base = nullptr;
  st = scratch_on_current_device(&base);
  if (st != MOE_OK) return st;
  LayerWs w = carve(L, S, R, T, base);
  if (err_word) w.err = err_word;
  return run_layer(L, x, S, a_expert, a_src, a_dst, a_w, R, T, out, w, stream);
}

int moe_layer_forward_w4a16(const moe_layer_desc* L, const uint16_t* x, int S,
                            const int32_t* a_expert, const int32_t* a_src, const int32_t* a_dst,
                            const float* a_w, int R, int T, uint16_t* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  int st = check_layer(L, S, R, T);
  if (st != MOE_OK) return st;
  REQUIRE(L->H <= kMaxBf16K && L->I <= kMaxBf16K, MOE_EUNSUPPORTED,
          "W4A16 layer: H=%d and I=%d must be <= %d", L->H, L->I, kMaxBf16K);
  REQUIRE((long long)(S > R ? S : R) * (L->H > L->I ? L->H : L->I) * 2 < (1ll << 31),
          MOE_EUNSUPPORTED, "W4A16 layer: bf16 activations exceed 2 GiB");
  REQUIRE(L->w13_packed && L->w2_packed && L->g_gate && L->g_up && L->g_down, MOE_EINVAL,
          "layer: null weights / globals");
  REQUIRE(workspace && aligned(workspace, 256), MOE_EINVAL, "layer: workspace null or not 256-byte aligned");
  const LayerWs w = carve(L, S, R, T, (uint8_t*)workspace);
  REQUIRE(workspace_bytes >= w.bytes, MOE_EWORKSPACE, "layer: workspace %zu bytes < %zu needed",
          workspace_bytes, w.bytes);
  if (R > 0) REQUIRE(a_expert && a_src && a_dst && a_w, MOE_EINVAL, "layer: null assignment array");
  if (R > 0 && S > 0) REQUIRE(x, MOE_EINVAL, "layer: null x");
  if (T > 0) REQUIRE(out, MOE_EINVAL, "layer: null out");
  REQUIRE(aligned(x, 16) && aligned(out, 8) && aligned(L->w13_packed, 16) && aligned(L->w2_packed, 16),
          MOE_EINVAL, "layer: x / weights must be 16-byte, out 8-byte aligned");
  const int E = L->E, H = L->H, I = L->I;
  hipError_t e;
  if (R >= 1 && R <= 32) {
    // a decode-sized batch: the w13 launch groups by itself (no grouping launch); the same
    // bits as the sequence below
    e = moe::launch_grouped_gemm_swiglu_grouping(a_expert, a_src, a_dst, a_w, R, E, S, T, x,
                                                 w.offsets, w.row_src, w.row_dst, w.row_w,
                                                 w.tok_off, w.tok_rows, w.err,
                                                 (const uint8_t*)L->w13_packed, I, H, L->g_gate,
                                                 L->g_up, w.h16, stream, true, w.items);
    if (e != hipSuccess) return hip_status(e, "layer: W4A16 grouping w13 GEMM + SwiGLU launch");
    if (moe::grouped_gemm_w4a16_sum_fits(R, I)) {
      // at most 16 rows: the w2 launch also sums each token's terms (two launches in all)
      e = moe::launch_grouped_gemm_w4a16_sum(w.h16, E, R, (const uint8_t*)L->w2_packed, H, I,
                                             w.row_w, L->g_down, w.items, w.tok_off, w.tok_rows,
                                             T, out, stream);
      return hip_status(e, "layer: W4A16 w2 GEMM + per-token sum launch");
    }
  } else {
    e = moe::launch_group(a_expert, a_src, a_dst, a_w, R, E, S, T, w.offsets, w.row_src,
                          w.row_dst, w.row_w, w.tok_off, w.tok_rows, w.err, stream, w.items);
    if (e != hipSuccess) return hip_status(e, "layer: group launch");
    if (R > 0) {
      e = moe::launch_grouped_gemm_swiglu_w4a16(x, w.row_src, S, w.offsets, E, R,
                                                (const uint8_t*)L->w13_packed, I, H, L->g_gate,
                                                L->g_up, w.h16, stream, w.items);
      if (e != hipSuccess) return hip_status(e, "layer: W4A16 w13 GEMM + SwiGLU launch");
    }
  }
  if (R > 0) {
    e = moe::launch_grouped_gemm_w4a16(w.h16, nullptr, R, w.offsets, E, R,
                                       (const uint8_t*)L->w2_packed, H, I, w.acc, stream, w.row_w,
                                       L->g_down, w.items);
    if (e != hipSuccess) return hip_status(e, "layer: W4A16 w2 GEMM launch");
  }
  e = moe::launch_token_sum(w.acc, R, H, w.tok_off, w.tok_rows, T, out, stream);
  return hip_status(e, "layer: scatter launch");
}

int moe_hbm_read_probe(const void* src, size_t bytes, int variant, uint32_t key, uint32_t* sink,
                       hipStream_t stream) {
  REQUIRE(variant >= 0 && variant < moe::probe_variants(), MOE_EINVAL,
          "read probe: variant %d outside [0, %d)", variant, moe::probe_variants());
  REQUIRE(bytes > 0 && bytes % kProbeUnit == 0, MOE_EUNSUPPORTED,
          "read probe: %zu bytes is not a positive multiple of %zu", bytes, kProbeUnit);
  REQUIRE(bytes / kProbeUnit < (1u << 31), MOE_EUNSUPPORTED, "read probe: %zu bytes is too large",
          bytes);
  REQUIRE(src && sink, MOE_EINVAL, "read probe: null pointer");
  REQUIRE(aligned(src, 16) && aligned(sink, 4), MOE_EINVAL, "read probe: src not 16-byte aligned");
  return hip_status(moe::launch_read_probe((const uint8_t*)src, bytes, variant, key, sink, stream),
                    "read probe launch");
}

int moe_hbm_read_probe_variants(void) { return moe::probe_variants(); }

int moe_get_device_error(const void* err_word, hipStream_t stream) {
  REQUIRE(err_word, MOE_EINVAL, "null error word");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "stream synchronize");
  int32_t v = 0;
  e = hipMemcpy(&v, err_word, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e, "error word read");
  ok();
  return v;
}

}  // extern "C"
