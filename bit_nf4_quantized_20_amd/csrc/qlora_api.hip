// qlora_api.hip -- the C ABI declared in include/qlora.h.
//
// Every entry point validates its arguments on the host before making any
// HIP call (so validation can be exercised on a machine without a GPU),
// then checks once per device that the device is gfx950, then enqueues its
// kernels on the caller's stream.
#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/qlora.h"
#include "common.hpp"
#include "nf4_format.hpp"

using namespace qlora;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QLORA_ERR_DEVICE;
  if (dev >= kMaxDevices) return QLORA_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QLORA_ERR_DEVICE;
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? QLORA_OK : QLORA_ERR_DEVICE;
}

// Scratch of qlora_linear_fwd_noalloc: the library's own device memory,
// sized for the forward's workspace up to kNoAllocScratchBytes.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress (once per
// device, cached below) and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, or nullptr if it cannot be found.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH; }

// ---------------------------------------------------------------------------
// Workspace layout.  Segments are 256-byte aligned; the workspace needs no
// initialisation.
// ---------------------------------------------------------------------------
constexpr size_t kMinWorkspace = 256;

// Largest tensor of the quantize / dequantize calls: 2^36 weights (256 GiB
// as fp32, more than one GPU holds); the dequantize grid runs one thread per
// 32 weights and stays below 2^32 threads.
constexpr int64_t kMaxNumel = int64_t(1) << 36;

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~static_cast<size_t>(255);
    return at;
  }
};

struct FwdLayout {
  size_t u_pad, b_pad, part, w_dq, split, total;
};

// From this many tokens on, the forward dequantizes each weight once into the
// workspace and runs the bf16 GEMM when the workspace holds the expanded
// weight: the fused kernel repeats the dequantization for every token tile,
// which from here on costs more than one extra pass of 2.5 bytes per weight
// (same-box A/B: 8B gate / down / q_proj / k shapes at 512-1792 tokens, the
// expanded route 0.74-1.01x the fused one's time).  With a smaller workspace
// (at least qlora_workspace_bytes_fwd_min) the fused kernel runs at every T.
constexpr int64_t kMaterializeTokens = 512;
struct BwdLayout {
  size_t ut, vt, v_pad, b_t, a_t_pad, w_dq_t, part, grad, uvp, suv, split, total;
};

int64_t padded_rank(int64_t r) { return round_up(r, 64); }

// n projections sharing `in`: outs[i] rows each, N = sum outs[i]
int64_t total_out(const int64_t* outs, int n) {
  int64_t N = 0;
  for (int i = 0; i < n; ++i) N += outs[i];
  return N;
}

// the small-token forward takes the call when every projection fits it; it
// needs a workspace only for the U it computes up front (decode_pre_u)
bool fwd_uses_decode(int64_t T, int64_t in, const int64_t* outs, int n, int64_t r) {
  for (int i = 0; i < n; ++i)
    if (!decode_fits(T, in, outs[i], r)) return false;
  return true;
}

// dropout: the small-token kernel has no mask, so that call always takes the
// general path
// expanded: the forward dequantizes W_hat into the workspace and runs the
// bf16 GEMM (from kMaterializeTokens on when the workspace holds W_hat, and
// always for the 4.5-bit format, whose fp32 block absmax only the standalone
// dequantize reads)
bool fwd_expands(int64_t T, bool absmax_fp32) { return absmax_fp32 || T >= kMaterializeTokens; }

// token-slice partial sums of every dA_i [r][in] (one pass over X for all
// projections) and of one dB_i [out_i][r] at a time (general backward)
size_t grad_part_bytes(int64_t T, int64_t in, const int64_t* outs, int n, int64_t r) {
  int64_t N = 0;
  for (int i = 0; i < n; ++i) N += outs[i];
  size_t b = 0;
  for (int i = 0; i < n; ++i) {
    const size_t bi = static_cast<size_t>(lora_grad_slices(T, outs[i], N) * outs[i] * r) * 4;
    b = bi > b ? bi : b;
  }
  return static_cast<size_t>(lora_grad_slices(T, in, in) * n * r * in) * 4 + b;
}

// split-K partials of a forward GEMM over n projections: one launch over all
// of them, or one per projection where a tile would straddle two
size_t split_bytes(int64_t T, int64_t N, int64_t in, const int64_t* outs, int n) {
  size_t b = gemm_split_bytes(T, N, in);
  for (int i = 0; i < n && n > 1; ++i) {
    const size_t bi = gemm_split_bytes(T, outs[i], in);
    b = bi > b ? bi : b;
  }
  return b;
}

// expand = false: the layout without W_hat (the fused GEMM's), for the
// double-quantized format
FwdLayout fwd_layout(int64_t T, int64_t in, const int64_t* outs, int n, int64_t r, bool dropout,
                     bool absmax_fp32 = false, bool expand = true) {
  FwdLayout l{0, 0, 0, 0, 0, 0};
  Carve c;
  if (!dropout && !absmax_fp32 && fwd_uses_decode(T, in, outs, n, r)) {
    l.u_pad = c.take(decode_u_bytes(n, T, r));  // U [n][T][r] fp32
    l.total = c.off;
    return l;
  }
  const int64_t rp = padded_rank(r), N = total_out(outs, n);
  l.u_pad = c.take(static_cast<size_t>(T * n * rp * 4));  // [T][n 2rp] bf16
  l.b_pad = c.take(static_cast<size_t>(N * n * rp * 4));  // [N][2rp] or [N][n 2rp] bf16
  l.part = c.take(lora_down_part_bytes(T, in, n * rp));
  if (fwd_expands(T, absmax_fp32) && (expand || absmax_fp32))
    l.w_dq = c.take(static_cast<size_t>(N * in * 2));  // [N][in] bf16
  l.split = c.take(split_bytes(T, N, in, outs, n));  // split-K partials of the GEMM
  l.total = c.off;
  return l;
}

int64_t token_pitch(int64_t T) { return round_up(T, 8); }


// Up to kDxSmallMaxT tokens without dropout the backward is the three
// launches of k_dx_small.hip: no W_hat^T, no padded factors; the W_hat^T
// region holds the fp32 row-split partials of dX instead ([splits][T][in],
// at most dx_small_max_splits of them), then the U / V chunk partials and
// sU, sV [n][T][r] fp32.
bool bwd_small(int64_t T, bool dropout) { return T <= kDxSmallMaxT && !dropout; }

// Above that the dX GEMM takes one of two routes (dX bit-identical either
// way): with a workspace that holds W_hat^T (2 * in * sum(out) bytes) it
// expands W_hat^T once and runs the bf16 GEMM, the faster route at every
// measured size; with a smaller one (at least the layout without that region)
// it reads the NF4 codes and dequantizes each weight tile, transposed, while
// staging it into LDS, so the backward needs no memory proportional to the
// weight.  The 4.5-bit format (read by the standalone transposed dequantize
// only) and codes too large for 32-bit offsets always expand.
bool bwd_can_fuse(int64_t in, const int64_t* outs, int n, bool absmax_fp32) {
  if (absmax_fp32) return false;
  for (int i = 0; i < n; ++i)
    if (!nf4t_fits(outs[i], in)) return false;
  return true;
}

// expand: the layout holds W_hat^T (the general path's expanded route)
BwdLayout bwd_layout(int64_t T, int64_t in, const int64_t* outs, int n, int64_t r, bool dropout,
                     bool expand = true) {
  const int64_t rp = padded_rank(r), N = total_out(outs, n);
  const bool small = bwd_small(T, dropout);
  int64_t out_max = 0;
  size_t part = lora_down_part_bytes(T, in, n * rp);
  for (int i = 0; i < n; ++i) {
    out_max = outs[i] > out_max ? outs[i] : out_max;
    const size_t pv = lora_down_part_bytes(T, outs[i], rp);
    part = pv > part ? pv : part;
  }
  Carve c;
  BwdLayout l{};
  if (small) {
    l.w_dq_t = c.take(static_cast<size_t>(dx_small_max_splits(N, in) * T * in * 4));  // dX partials
    l.uvp = c.take(bwd_small_uv_bytes(T, in, outs, n, r));
    l.suv = c.take(static_cast<size_t>(2 * n * T * r * 4));
  } else {
    l.ut = c.take(static_cast<size_t>(n * 2 * rp * token_pitch(T) * 2));  // [n][2rp][T'] bf16
    l.vt = c.take(static_cast<size_t>(n * 2 * rp * token_pitch(T) * 2));
    l.v_pad = c.take(static_cast<size_t>(T * n * rp * 4));                // [T][n 2rp] bf16
    l.b_t = c.take(static_cast<size_t>(r * out_max * 2));                 // one B^T at a time
    l.a_t_pad = c.take(static_cast<size_t>(in * n * rp * 4));             // [in][n 2rp] bf16
    if (expand) l.w_dq_t = c.take(static_cast<size_t>(in * N * 2));       // [in][N] bf16
    l.part = c.take(part);
    l.grad = c.take(grad_part_bytes(T, in, outs, n, r));  // token-slice sums of dA_i, dB_i
    l.split = c.take(gemm_split_bytes(T, in, N));  // split-K partials of the dX GEMM
  }
  l.total = c.off;
  return l;
}

bool linear_shapes_ok(int64_t T, int64_t in, int64_t out, int64_t r) {
  if (T < 0 || in < 64 || out < 64 || (in % 64) != 0 || (out % 64) != 0) return false;
  if (r < 1 || r > QLORA_MAX_RANK) return false;
  if (in > (int64_t(1) << 31) || out > (int64_t(1) << 31) || T > (int64_t(1) << 31)) return false;
  return true;
}

// Every bf16 operand of a linear call -- X, Y / dY, dX, and the dequantized
// weight the large-token paths build in the workspace -- stays below 2^31
// bytes: the kernels address the rows of a tile with 32-bit offsets.
constexpr int64_t kMaxOperandBytes = (int64_t(1) << 31) - 1;

bool bf16_matrix_fits(int64_t rows, int64_t cols) {
  return rows <= 0 || cols <= 0 || cols <= kMaxOperandBytes / 2 / rows;
}

bool operands_fit(int64_t T, int64_t in, int64_t N) {
  return bf16_matrix_fits(T, in) && bf16_matrix_fits(T, N) && bf16_matrix_fits(N, in);
}

bool absmax_fp32(const qlora_nf4_weight& W) { return (W.flags & QLORA_NF4_ABSMAX_FP32) != 0; }

// the descriptor's format and pointers: absmax_q is read only by the
// double-quantized format
int check_weight(const qlora_nf4_weight* W) {
  if (W == nullptr) return QLORA_ERR_NULL;
  if ((W->flags & ~QLORA_NF4_FLAGS_KNOWN) != 0) return QLORA_ERR_VALUE;
  const bool dq = !absmax_fp32(*W);
  if (W->codes == nullptr || W->absmax_scale == nullptr || (dq && W->absmax_q == nullptr))
    return QLORA_ERR_NULL;
  if (!aligned16(W->codes) || (dq && !aligned16(W->absmax_q)) || !aligned16(W->absmax_scale))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

}  // namespace

extern "C" {

int nf4_storage_bytes(int64_t numel, size_t* codes_bytes, size_t* absmax_q_bytes,
                      size_t* scale_bytes) {
  if (numel < 0 || (numel % kBlock) != 0) return QLORA_ERR_SHAPE;
  if (codes_bytes) *codes_bytes = static_cast<size_t>(numel / 2);
  if (absmax_q_bytes) *absmax_q_bytes = static_cast<size_t>(numel / kBlock);
  if (scale_bytes) *scale_bytes = static_cast<size_t>(4 * ceil_div(numel, kGroupElems));
  return QLORA_OK;
}

int nf4_quantize(const float* w, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                 float* absmax_scale, qlora_stream stream) {
  if (numel < 0 || (numel % kBlock) != 0) return QLORA_ERR_SHAPE;
  if (numel > kMaxNumel) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!w || !codes || !absmax_q || !absmax_scale) return QLORA_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax_q) || !aligned16(absmax_scale))
    return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;
  return launched(launch_nf4_quantize(w, numel, codes, absmax_q, absmax_scale,
                                      static_cast<hipStream_t>(stream)));
}

int nf4_dequantize(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_scale,
                   int64_t numel, qlora_bf16* w_out, qlora_stream stream) {
  if (numel < 0 || (numel % kBlock) != 0) return QLORA_ERR_SHAPE;
  if (numel > kMaxNumel) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!codes || !absmax_q || !absmax_scale || !w_out) return QLORA_ERR_NULL;
  if (!aligned16(codes) || !aligned16(absmax_q) || !aligned16(absmax_scale) || !aligned16(w_out))
    return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;
  return launched(launch_nf4_dequantize(codes, absmax_q, absmax_scale, numel, w_out,
                                        static_cast<hipStream_t>(stream)));
}

int nf4_quantize_nodq(const float* w, int64_t numel, uint8_t* codes, float* absmax,
                      qlora_stream stream) {
  if (numel < 0 || (numel % kBlock) != 0) return QLORA_ERR_SHAPE;
  if (numel > kMaxNumel) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!w || !codes || !absmax) return QLORA_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;
  return launched(launch_nf4_quantize_nodq(w, numel, codes, absmax, static_cast<hipStream_t>(stream)));
}

int nf4_dequantize_nodq(const uint8_t* codes, const float* absmax, int64_t numel, qlora_bf16* w_out,
                        qlora_stream stream) {
  if (numel < 0 || (numel % kBlock) != 0) return QLORA_ERR_SHAPE;
  if (numel > kMaxNumel) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!codes || !absmax || !w_out) return QLORA_ERR_NULL;
  if (!aligned16(codes) || !aligned16(absmax) || !aligned16(w_out)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;
  return launched(launch_nf4_dequantize_nodq(codes, absmax, numel, w_out, static_cast<hipStream_t>(stream)));
}

size_t qlora_workspace_bytes(int64_t T, int64_t in_features, int64_t out_features, int64_t r,
                             int backward) {
  return qlora_workspace_bytes_multi(T, in_features, &out_features, 1, r, backward);
}

size_t qlora_workspace_bytes_multi(int64_t T, int64_t in_features, const int64_t* out_features,
                                   int n, int64_t r, int backward) {
  if (n < 1 || n > kMaxProj || out_features == nullptr) return 0;
  for (int i = 0; i < n; ++i)
    if (!linear_shapes_ok(T, in_features, out_features[i], r)) return 0;
  if (!operands_fit(T, in_features, total_out(out_features, n))) return 0;
  const size_t need = backward ? bwd_layout(T, in_features, out_features, n, r, false).total
                               : fwd_layout(T, in_features, out_features, n, r, false).total;
  return need > kMinWorkspace ? need : kMinWorkspace;
}

size_t qlora_workspace_bytes_flags(int64_t T, int64_t in_features, const int64_t* out_features, int n,
                                   int64_t r, int backward, int dropout, uint32_t flags) {
  if ((flags & ~QLORA_NF4_FLAGS_KNOWN) != 0) return 0;
  if (n < 1 || n > kMaxProj || out_features == nullptr || (dropout && n != 1)) return 0;
  for (int i = 0; i < n; ++i)
    if (!linear_shapes_ok(T, in_features, out_features[i], r)) return 0;
  if (!operands_fit(T, in_features, total_out(out_features, n))) return 0;
  const bool fp32 = (flags & QLORA_NF4_ABSMAX_FP32) != 0;
  const size_t need = backward ? bwd_layout(T, in_features, out_features, n, r, dropout != 0).total
                               : fwd_layout(T, in_features, out_features, n, r, dropout != 0, fp32).total;
  return need > kMinWorkspace ? need : kMinWorkspace;
}

size_t qlora_workspace_bytes_fwd_min(int64_t T, int64_t in_features, const int64_t* out_features, int n,
                                     int64_t r, int dropout, uint32_t flags) {
  if ((flags & ~QLORA_NF4_FLAGS_KNOWN) != 0) return 0;
  if (n < 1 || n > kMaxProj || out_features == nullptr || (dropout && n != 1)) return 0;
  for (int i = 0; i < n; ++i)
    if (!linear_shapes_ok(T, in_features, out_features[i], r)) return 0;
  if (!operands_fit(T, in_features, total_out(out_features, n))) return 0;
  const bool fp32 = (flags & QLORA_NF4_ABSMAX_FP32) != 0;
  const size_t need = fwd_layout(T, in_features, out_features, n, r, dropout != 0, fp32, false).total;
  return need > kMinWorkspace ? need : kMinWorkspace;
}

size_t qlora_workspace_bytes_bwd_min(int64_t T, int64_t in_features, const int64_t* out_features, int n,
                                     int64_t r, int dropout, uint32_t flags) {
  if ((flags & ~QLORA_NF4_FLAGS_KNOWN) != 0) return 0;
  if (n < 1 || n > kMaxProj || out_features == nullptr || (dropout && n != 1)) return 0;
  for (int i = 0; i < n; ++i)
    if (!linear_shapes_ok(T, in_features, out_features[i], r)) return 0;
  if (!operands_fit(T, in_features, total_out(out_features, n))) return 0;
  const bool fuse = bwd_can_fuse(in_features, out_features, n, (flags & QLORA_NF4_ABSMAX_FP32) != 0);
  const size_t need = bwd_layout(T, in_features, out_features, n, r, dropout != 0, !fuse).total;
  return need > kMinWorkspace ? need : kMinWorkspace;
}

size_t qlora_workspace_bytes_dropout(int64_t T, int64_t in_features, int64_t out_features, int64_t r,
                                     int backward) {
  if (!linear_shapes_ok(T, in_features, out_features, r)) return 0;
  if (!operands_fit(T, in_features, out_features)) return 0;
  const size_t need = backward ? bwd_layout(T, in_features, &out_features, 1, r, true).total
                               : fwd_layout(T, in_features, &out_features, 1, r, true).total;
  return need > kMinWorkspace ? need : kMinWorkspace;
}

}  // extern "C"

namespace {

// Checks the n projections (shared in_features, rank r) and collects their
// row counts; QLORA_OK or the first error.
int check_projections(const qlora_nf4_weight* W, int n, int64_t T, int64_t r, int64_t* outs,
                      int64_t* in) {
  if (W == nullptr) return QLORA_ERR_NULL;
  if (n < 1 || n > kMaxProj) return QLORA_ERR_SHAPE;
  for (int i = 0; i < n; ++i) {
    if (int st = check_weight(&W[i])) return st;
    if (W[i].cols != W[0].cols) return QLORA_ERR_SHAPE;
    if (W[i].flags != W[0].flags) return QLORA_ERR_VALUE;
    if (!linear_shapes_ok(T, W[i].cols, W[i].rows, r)) return QLORA_ERR_SHAPE;
    outs[i] = W[i].rows;
  }
  *in = W[0].cols;
  if (!operands_fit(T, *in, total_out(outs, n))) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

// LoRA dropout arguments: no mask means no dropout; with a mask, 0 <= p < 1
int check_dropout(const uint8_t* keep, float p) {
  if (keep == nullptr) return QLORA_OK;
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return QLORA_ERR_VALUE;
  return QLORA_OK;
}

int check_factors(const qlora_bf16* const* A, const qlora_bf16* const* B, int n) {
  if (A == nullptr || B == nullptr) return QLORA_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    if (!A[i] || !B[i]) return QLORA_ERR_NULL;
    if (!aligned16(A[i]) || !aligned16(B[i])) return QLORA_ERR_ALIGN;
  }
  return QLORA_OK;
}

// keep / p: LoRA dropout (keep == nullptr: none; n == 1 only), see
// qlora_linear_fwd_dropout
int linear_fwd_impl(const qlora_nf4_weight* W, int n, const qlora_bf16* X, int64_t T,
                    const qlora_bf16* const* A, const qlora_bf16* const* B, int64_t r, float alpha,
                    qlora_bf16* Y, void* ws, size_t ws_bytes, qlora_stream stream,
                    const uint8_t* keep = nullptr, float p = 0.f) {
  int64_t outs[kMaxProj], in = 0;
  if (int st = check_projections(W, n, T, r, outs, &in)) return st;
  if (int st = check_factors(A, B, n)) return st;
  if (T > 0 && (!X || !Y)) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(Y)) return QLORA_ERR_ALIGN;
  if (!std::isfinite(alpha)) return QLORA_ERR_VALUE;
  const bool dropout = keep != nullptr;
  if (int st = check_dropout(keep, p)) return st;
  if (T == 0) return QLORA_OK;
  const bool fp32 = absmax_fp32(W[0]);
  // the expanded route when the workspace holds W_hat, else the fused GEMM
  const FwdLayout full = fwd_layout(T, in, outs, n, r, dropout, fp32, true);
  const FwdLayout least = fwd_layout(T, in, outs, n, r, dropout, fp32, false);
  const bool expand = fwd_expands(T, fp32) && ws != nullptr && ws_bytes >= full.total;
  const FwdLayout lay = expand ? full : least;
  // The small-token forward also runs without a workspace where U need not
  // be computed up front (r <= 16, at most 4096 output rows): ws = NULL
  // selects its single-launch form.
  const bool decode_no_ws = !dropout && !fp32 && ws == nullptr && fwd_uses_decode(T, in, outs, n, r) &&
                            !decode_pre_u(n, outs, r);
  if (!decode_no_ws && lay.total > 0 && (ws == nullptr || ws_bytes < lay.total)) return QLORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = alpha / static_cast<float>(r);
  const int64_t N = total_out(outs, n);
  if (!dropout && !fp32 && fwd_uses_decode(T, in, outs, n, r)) {
    DecodeProj proj[kMaxProj];
    for (int i = 0; i < n; ++i)
      proj[i] = DecodeProj{W[i].codes, W[i].absmax_q, W[i].absmax_scale, A[i], B[i], outs[i]};
    float* u_ws = ws != nullptr ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + lay.u_pad) : nullptr;
    return launched(launch_decode_fwd(n, proj, in, X, T, r, scale, Y, N, u_ws, s));
  }

  const int64_t rp = padded_rank(r);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* u_pad = reinterpret_cast<uint16_t*>(base + lay.u_pad);
  uint16_t* b_pad = reinterpret_cast<uint16_t*>(base + lay.b_pad);
  float* part = reinterpret_cast<float*>(base + lay.part);
  float* split = reinterpret_cast<float*>(base + lay.split);
  const size_t split_n = lay.total - lay.split;
  // s X A_i^T for every projection in one pass over X: [T][n 2rp]; with
  // dropout s / (1 - p) (keep o X) A^T
  const float uscale = dropout ? scale / (1.f - p) : scale;
  hipError_t e = launch_lora_down(X, in, T, in, A, n, r, uscale, u_pad, n * 2 * rp, nullptr, 0, rp, part, s,
                                  keep, in / 8);
  if (expand) {
    // W_hat of every projection into [N][in] bf16, then the bf16 GEMM.  The
    // LoRA term runs as extra K-steps: when no tile straddles two projections
    // each tile reads its own projection's sU_i against B_i (stacked [N][2rp]);
    // otherwise over [sU_0 | sU_1 | ...] against B_i placed block-diagonally
    // in [N][n 2rp]
    uint16_t* w_dq = reinterpret_cast<uint16_t*>(base + lay.w_dq);
    const bool per_proj = n > 1 && gemm_proj_aligned(T, n, outs);
    const int64_t ldb = per_proj ? 2 * rp : n * 2 * rp;
    if (e == hipSuccess && n > 1 && !per_proj)
      e = launch_fill_f32(reinterpret_cast<float*>(b_pad), N * ldb / 2, 0.f, s);
    {
      // every projection's B_i padded in one launch
      const uint16_t* bsrc[kMaxProj];
      uint16_t* bdst[kMaxProj];
      int64_t brows[kMaxProj];
      int64_t o = 0;
      for (int i = 0; i < n; ++i) {
        bsrc[i] = B[i];
        bdst[i] = b_pad + o * ldb + (per_proj ? 0 : i * 2 * rp);
        brows[i] = outs[i];
        o += outs[i];
      }
      if (e == hipSuccess) e = launch_pad_many(bsrc, brows, bdst, n, r, rp, ldb, s);
    }
    int64_t off = 0;
    for (int i = 0; i < n && e == hipSuccess; ++i) {
      e = fp32 ? launch_nf4_dequantize_nodq(W[i].codes, W[i].absmax_scale, outs[i] * in, w_dq + off * in, s)
               : launch_nf4_dequantize(W[i].codes, W[i].absmax_q, W[i].absmax_scale, outs[i] * in,
                                       w_dq + off * in, s);
      off += outs[i];
    }
    if (e == hipSuccess) {
      if (per_proj) {
        const uint16_t* act1[kMaxProj];
        for (int i = 0; i < n; ++i) act1[i] = u_pad + i * 2 * rp;
        e = launch_gemm_nt_proj(T, n, outs, act1, X, in, w_dq, in, in, n * 2 * rp, b_pad, ldb, 2 * rp, Y, N,
                                s, split, split_n);
      } else {
        e = launch_gemm_nt(T, N, X, in, w_dq, in, in, u_pad, ldb, b_pad, ldb, ldb, Y, N, s, nullptr, 0, 1.f,
                           split, split_n);
      }
    }
    return launched(e);
  }
  Nf4Proj proj[kMaxProj];
  const uint16_t* bsrc[kMaxProj];
  uint16_t* bdst[kMaxProj];
  int64_t brows[kMaxProj];
  int64_t off = 0;
  for (int i = 0; i < n; ++i) {
    bsrc[i] = B[i];
    bdst[i] = b_pad + off * 2 * rp;
    brows[i] = outs[i];
    proj[i] = Nf4Proj{W[i].codes, W[i].absmax_q, W[i].absmax_scale, outs[i], u_pad + i * 2 * rp};
    off += outs[i];
  }
  if (e == hipSuccess) e = launch_pad_many(bsrc, brows, bdst, n, r, rp, 2 * rp, s);  // every B_i padded
  if (e == hipSuccess)
    e = launch_gemm_nf4(T, n, proj, X, in, in, n * 2 * rp, b_pad, 2 * rp, 2 * rp, Y, N, s, split, split_n);
  return launched(e);
}

int linear_bwd_impl(const qlora_nf4_weight* W, int n, const qlora_bf16* X, const qlora_bf16* dY,
                    int64_t T, const qlora_bf16* const* A, const qlora_bf16* const* B, int64_t r,
                    float alpha, qlora_bf16* dX, float* const* dA, float* const* dB, void* ws,
                    size_t ws_bytes, qlora_stream stream, const uint8_t* keep = nullptr,
                    float p = 0.f) {
  int64_t outs[kMaxProj], in = 0;
  if (int st = check_projections(W, n, T, r, outs, &in)) return st;
  if (int st = check_factors(A, B, n)) return st;
  if (dA == nullptr || dB == nullptr) return QLORA_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    if (!dA[i] || !dB[i]) return QLORA_ERR_NULL;
    if (!aligned16(dA[i]) || !aligned16(dB[i])) return QLORA_ERR_ALIGN;
  }
  if (T > 0 && (!X || !dY || !dX)) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(dX)) return QLORA_ERR_ALIGN;
  if (!std::isfinite(alpha)) return QLORA_ERR_VALUE;
  if (int st = check_dropout(keep, p)) return st;
  // the expanded route when the workspace holds W_hat^T, else the fused dX
  const BwdLayout full = bwd_layout(T, in, outs, n, r, keep != nullptr, true);
  const bool can_fuse = bwd_can_fuse(in, outs, n, absmax_fp32(W[0]));
  const BwdLayout least = bwd_layout(T, in, outs, n, r, keep != nullptr, !can_fuse);
  if (T > 0 && (ws == nullptr || ws_bytes < least.total)) return QLORA_ERR_WORKSPACE;
  const bool fused = can_fuse && ws_bytes < full.total;
  const BwdLayout lay = fused ? least : full;
  if (ws != nullptr && !aligned16(ws)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = alpha / static_cast<float>(r);
  const int64_t N = total_out(outs, n);
  uint8_t* base = static_cast<uint8_t*>(ws);
  if (T > 0 && bwd_small(T, keep != nullptr)) {
    // three launches; dA and dB are written, not accumulated
    BwdSmallDev a{};
    a.set.n = a.n = n;
    int64_t row0 = 0;
    for (int i = 0; i < n; ++i) {
      a.set.proj[i] = DxProj{W[i].codes, W[i].absmax_q, W[i].absmax_scale, row0};
      a.A.p[i] = A[i];
      a.B.p[i] = B[i];
      a.out[i] = outs[i];
      a.dA[i] = dA[i];
      a.dB[i] = dB[i];
      row0 += outs[i];
    }
    a.T = static_cast<int>(T);
    a.r = static_cast<int>(r);
    a.N = N;
    a.in = in;
    a.X = X;
    a.dY = dY;
    a.dxp = reinterpret_cast<float*>(base + lay.w_dq_t);
    a.uvp = reinterpret_cast<float*>(base + lay.uvp);
    a.su = reinterpret_cast<float*>(base + lay.suv);
    a.sv = a.su + n * T * r;
    a.s = scale;
    a.dX = dX;
    return launched(launch_bwd_small(a, lay.uvp - lay.w_dq_t, absmax_fp32(W[0]), s));
  }
  hipError_t e = hipSuccess;
  if (T == 0) {
    // no tokens: dA_i and dB_i are zero (one launch)
    float* zero_dst[kMaxFill];
    int64_t zero_n[kMaxFill];
    for (int i = 0; i < n; ++i) {
      zero_dst[2 * i] = dA[i];
      zero_n[2 * i] = r * in;
      zero_dst[2 * i + 1] = dB[i];
      zero_n[2 * i + 1] = outs[i] * r;
    }
    return launched(launch_fill_many_f32(zero_dst, zero_n, 2 * n, 0.f, s));
  }

  const int64_t rp = padded_rank(r), tp = token_pitch(T);
  uint16_t* ut = reinterpret_cast<uint16_t*>(base + lay.ut);
  uint16_t* vt = reinterpret_cast<uint16_t*>(base + lay.vt);
  uint16_t* v_pad = reinterpret_cast<uint16_t*>(base + lay.v_pad);
  uint16_t* b_t = reinterpret_cast<uint16_t*>(base + lay.b_t);
  uint16_t* a_t_pad = reinterpret_cast<uint16_t*>(base + lay.a_t_pad);
  uint16_t* w_dq_t = reinterpret_cast<uint16_t*>(base + lay.w_dq_t);
  float* part = reinterpret_cast<float*>(base + lay.part);
  float* split = reinterpret_cast<float*>(base + lay.split);
  const size_t split_n = lay.total - lay.split;

  // (sU_i)^T for every projection in one pass over X (with dropout the
  // masked input: s / (1 - p) (keep o X) A^T, which dB then uses as is)
  const float inv_keep = keep != nullptr ? 1.f / (1.f - p) : 1.f;
  e = launch_lora_down(X, in, T, in, A, n, r, scale * inv_keep, nullptr, 0, ut, tp, rp, part, s, keep,
                       in / 8);
  // the dX GEMM dequantizes W_hat^T tile by tile (fused) or reads it expanded
  // (small token counts without dropout took the streamed path above)
  int64_t off = 0;
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    // B_i^T and the padded A_i^T in one launch, then s V_i = s dY_i B_i with
    // dY_i the projection's columns of dY
    e = launch_factor_prep(B[i], outs[i], r, b_t, A[i], in, a_t_pad + i * 2 * rp, rp, n * 2 * rp, s);
    const uint16_t* bt = b_t;
    if (e == hipSuccess)
      e = launch_lora_down(dY + off, N, T, outs[i], &bt, 1, r, scale, v_pad + i * 2 * rp, n * 2 * rp,
                           vt + i * 2 * rp * tp, tp, rp, part, s);
    if (e == hipSuccess && !fused)
      e = launch_nf4_dequantize_transposed(W[i].codes, W[i].absmax_q, W[i].absmax_scale, outs[i], in,
                                           w_dq_t + off, N, s, absmax_fp32(W[i]));
    off += outs[i];
  }
  if (e == hipSuccess && fused) {
    Nf4Proj proj[kMaxProj];
    for (int i = 0; i < n; ++i) proj[i] = Nf4Proj{W[i].codes, W[i].absmax_q, W[i].absmax_scale, outs[i], nullptr};
    e = launch_gemm_nf4t(T, in, n, proj, dY, N, v_pad, n * 2 * rp, a_t_pad, n * 2 * rp, n * 2 * rp, dX, in, s,
                         keep, in / 8, inv_keep, split, split_n);
  } else if (e == hipSuccess) {
    // dX = sum_i dY_i W_hat_i + (sV_i) A_i: one GEMM over the concatenated K
    // (with dropout the adapter term is masked and scaled by 1 / (1 - p)
    // before the base is added)
    e = launch_gemm_nt(T, in, dY, N, w_dq_t, N, N, v_pad, n * 2 * rp, a_t_pad, n * 2 * rp, n * 2 * rp,
                       dX, in, s, keep, in / 8, inv_keep, split, split_n);
  }
  // dA_i and dB_i: token-slice sums into the workspace, then every output
  // written once with its slices added in order (bit-reproducible).  dA of
  // every projection comes from one pass over X (the projections' ranks
  // stacked); dB_i from dY's columns of projection i, its region reused
  // projection after projection in stream order.
  float* const gp = reinterpret_cast<float*>(base + lay.grad);
  const int64_t sa = lora_grad_slices(T, in, in);
  float* const pb = gp + sa * n * r * in;
  if (e == hipSuccess)
    e = launch_lora_grad(vt, T, tp, rp, X, in, in, n * r, gp, true, s, keep, in / 8, inv_keep, r);  // dA
  off = 0;
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    const int64_t sb = lora_grad_slices(T, outs[i], N);
    e = launch_lora_grad(ut + i * 2 * rp * tp, T, tp, rp, dY + off, outs[i], N, r, pb, false, s);  // dB_i
    if (e == hipSuccess) {
      const float* part[kMaxFill];
      int slices[kMaxFill];
      int64_t cnt[kMaxFill], stride[kMaxFill];
      float* outp[kMaxFill];
      part[0] = pb;
      slices[0] = static_cast<int>(sb);
      cnt[0] = stride[0] = outs[i] * r;
      outp[0] = dB[i];
      int jobs = 1;
      if (i == n - 1) {  // with the last dB, every dA
        for (int j = 0; j < n; ++j, ++jobs) {
          part[jobs] = gp + j * r * in;
          slices[jobs] = static_cast<int>(sa);
          cnt[jobs] = r * in;
          stride[jobs] = n * r * in;
          outp[jobs] = dA[j];
        }
      }
      e = launch_sum_slices(part, slices, cnt, outp, jobs, s, stride);
    }
    off += outs[i];
  }
  return launched(e);
}

}  // namespace

extern "C" {

int qlora_linear_fwd(const qlora_nf4_weight* W, const qlora_bf16* X, int64_t T,
                     const qlora_bf16* A, const qlora_bf16* B, int64_t r, float alpha,
                     qlora_bf16* Y, void* ws, size_t ws_bytes, qlora_stream stream) {
  return linear_fwd_impl(W, 1, X, T, &A, &B, r, alpha, Y, ws, ws_bytes, stream);
}

size_t qlora_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int qlora_linear_fwd_noalloc(const qlora_nf4_weight* W, const qlora_bf16* X, int64_t T, const qlora_bf16* A,
                             const qlora_bf16* B, int64_t r, float alpha, qlora_bf16* Y, qlora_stream stream) {
  // the size check comes first, before any HIP call: a call whose workspace
  // would not fit in the library's scratch is refused without side effects
  if (W == nullptr) return QLORA_ERR_NULL;
  const size_t need = qlora_workspace_bytes_fwd_min(T, W->cols, &W->rows, 1, r, 0, W->flags);
  if (need == 0) return linear_fwd_impl(W, 1, X, T, &A, &B, r, alpha, Y, nullptr, 0, stream);  // shape error
  if (need > kNoAllocScratchBytes) return QLORA_ERR_WORKSPACE;
  if (T == 0) return linear_fwd_impl(W, 1, X, T, &A, &B, r, alpha, Y, nullptr, 0, stream);
  if (int st = check_device()) return st;
  void* ws = device_scratch();
  if (ws == nullptr) return QLORA_ERR_DEVICE;
  return linear_fwd_impl(W, 1, X, T, &A, &B, r, alpha, Y, ws, kNoAllocScratchBytes, stream);
}

int qlora_linear_fwd_multi(const qlora_nf4_weight* W, int n, const qlora_bf16* X, int64_t T,
                           const qlora_bf16* const* A, const qlora_bf16* const* B, int64_t r,
                           float alpha, qlora_bf16* Y, void* ws, size_t ws_bytes,
                           qlora_stream stream) {
  return linear_fwd_impl(W, n, X, T, A, B, r, alpha, Y, ws, ws_bytes, stream);
}

int qlora_linear_bwd(const qlora_nf4_weight* W, const qlora_bf16* X, const qlora_bf16* dY,
                     int64_t T, const qlora_bf16* A, const qlora_bf16* B, int64_t r, float alpha,
                     qlora_bf16* dX, float* dA, float* dB, void* ws, size_t ws_bytes,
                     qlora_stream stream) {
  return linear_bwd_impl(W, 1, X, dY, T, &A, &B, r, alpha, dX, &dA, &dB, ws, ws_bytes, stream);
}

int qlora_linear_bwd_multi(const qlora_nf4_weight* W, int n, const qlora_bf16* X,
                           const qlora_bf16* dY, int64_t T, const qlora_bf16* const* A,
                           const qlora_bf16* const* B, int64_t r, float alpha, qlora_bf16* dX,
                           float* const* dA, float* const* dB, void* ws, size_t ws_bytes,
                           qlora_stream stream) {
  return linear_bwd_impl(W, n, X, dY, T, A, B, r, alpha, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_linear_fwd_dropout(const qlora_nf4_weight* W, const qlora_bf16* X, int64_t T,
                             const uint8_t* keep, float p, const qlora_bf16* A, const qlora_bf16* B,
                             int64_t r, float alpha, qlora_bf16* Y, void* ws, size_t ws_bytes,
                             qlora_stream stream) {
  if (T > 0 && keep == nullptr) return QLORA_ERR_NULL;
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return QLORA_ERR_VALUE;
  if (T == 0) keep = nullptr;
  return linear_fwd_impl(W, 1, X, T, &A, &B, r, alpha, Y, ws, ws_bytes, stream, keep, p);
}

int qlora_linear_bwd_dropout(const qlora_nf4_weight* W, const qlora_bf16* X, const qlora_bf16* dY,
                             int64_t T, const uint8_t* keep, float p, const qlora_bf16* A,
                             const qlora_bf16* B, int64_t r, float alpha, qlora_bf16* dX, float* dA,
                             float* dB, void* ws, size_t ws_bytes, qlora_stream stream) {
  if (T > 0 && keep == nullptr) return QLORA_ERR_NULL;
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return QLORA_ERR_VALUE;
  if (T == 0) keep = nullptr;
  return linear_bwd_impl(W, 1, X, dY, T, &A, &B, r, alpha, dX, &dA, &dB, ws, ws_bytes, stream, keep, p);
}

size_t qlora_merge_workspace_bytes(int64_t in_features, int64_t out_features, int64_t r) {
  if (!linear_shapes_ok(0, in_features, out_features, r)) return 0;
  if (!operands_fit(0, in_features, out_features)) return 0;
  const int64_t rp = padded_rank(r);
  Carve c;
  c.take(static_cast<size_t>(out_features * rp * 4));  // B padded [out][2 rp]
  c.take(static_cast<size_t>(in_features * rp * 4));   // A^T padded [in][2 rp]
  return c.off > kMinWorkspace ? c.off : kMinWorkspace;
}

int qlora_merge(const qlora_nf4_weight* W, const qlora_bf16* A, const qlora_bf16* B, int64_t r,
                float alpha, qlora_bf16* W_out, void* ws, size_t ws_bytes, qlora_stream stream) {
  if (int st = check_weight(W)) return st;
  if (absmax_fp32(*W)) return QLORA_ERR_VALUE;  // the merge reads the double-quantized format only
  const int64_t out = W->rows, in = W->cols;
  if (!linear_shapes_ok(0, in, out, r) || !operands_fit(0, in, out)) return QLORA_ERR_SHAPE;
  if (!A || !B || !W_out) return QLORA_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(W_out)) return QLORA_ERR_ALIGN;
  if (!std::isfinite(alpha)) return QLORA_ERR_VALUE;
  const size_t need = qlora_merge_workspace_bytes(in, out, r);
  if (ws == nullptr || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (merge_direct(r))
    return launched(launch_merge_direct(W->codes, W->absmax_q, W->absmax_scale, out, in, B, A, r,
                                        alpha / static_cast<float>(r), W_out, s));
  const int64_t rp = padded_rank(r);
  uint16_t* b_pad = static_cast<uint16_t*>(ws);
  uint16_t* a_t_pad = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + round_up(out * rp * 4, 256));
  hipError_t e = launch_pad_bf16(B, out, r, false, b_pad, rp, 2 * rp, s);
  if (e == hipSuccess) e = launch_pad_bf16(A, in, r, true, a_t_pad, rp, 2 * rp, s);
  if (e == hipSuccess)
    e = launch_merge(W->codes, W->absmax_q, W->absmax_scale, out, in, b_pad, a_t_pad, 2 * rp, rp,
                     alpha / static_cast<float>(r), W_out, s);
  return launched(e);
}

void nf4_codebook(float out[16]) {
  for (int j = 0; j < 16; ++j) out[j] = level(j);
}

void nf4_code_thresholds(float out[15]) {
  for (int j = 0; j < 15; ++j) out[j] = kThresholds.t[j];
}

void nf4_code_buckets(float thr[33], uint32_t base[33]) {
  for (int i = 0; i < kBuckets; ++i) {
    thr[i] = __builtin_bit_cast(float, kBucketTable.word[2 * i]);
    base[i] = kBucketTable.word[2 * i + 1];
  }
}

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "invalid shape (negative, not a multiple of 64, or out of range)";
    case QLORA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_LAUNCH: return "kernel launch failed";
    case QLORA_ERR_DEVICE: return "no HIP device or the device is not gfx950";
    case QLORA_ERR_VALUE: return "non-finite scalar argument";
    default: return "unknown status";
  }
}

}  // extern "C"
