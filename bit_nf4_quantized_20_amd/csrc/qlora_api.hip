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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH; }

// ---------------------------------------------------------------------------
// Workspace layout.  Segments are 256-byte aligned; the workspace needs no
// initialisation.
// ---------------------------------------------------------------------------
constexpr size_t kMinWorkspace = 256;

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~static_cast<size_t>(255);
    return at;
  }
};

struct FwdLayout {
  size_t u_pad, b_pad, part, total;
};
struct BwdLayout {
  size_t ut, vt, v_pad, b_t, a_t_pad, w_dq_t, part, total;
};

int64_t padded_rank(int64_t r) { return round_up(r, 64); }

bool fwd_uses_decode(int64_t T, int64_t in, int64_t out, int64_t r) { return decode_fits(T, in, out, r); }

FwdLayout fwd_layout(int64_t T, int64_t in, int64_t out, int64_t r) {
  FwdLayout l{0, 0, 0, 0};
  Carve c;
  if (fwd_uses_decode(T, in, out, r)) return l;  // the fused small-token kernel needs none
  const int64_t rp = padded_rank(r);
  l.u_pad = c.take(static_cast<size_t>(T * rp * 4));
  l.b_pad = c.take(static_cast<size_t>(out * rp * 4));
  l.part = c.take(lora_down_part_bytes(T, in, rp));
  l.total = c.off;
  return l;
}

int64_t token_pitch(int64_t T) { return round_up(T, 8); }

BwdLayout bwd_layout(int64_t T, int64_t in, int64_t out, int64_t r) {
  const int64_t rp = padded_rank(r);
  Carve c;
  BwdLayout l;
  l.ut = c.take(static_cast<size_t>(2 * rp * token_pitch(T) * 2));
  l.vt = c.take(static_cast<size_t>(2 * rp * token_pitch(T) * 2));
  l.v_pad = c.take(static_cast<size_t>(T * rp * 4));
  l.b_t = c.take(static_cast<size_t>(r * out * 2));
  l.a_t_pad = c.take(static_cast<size_t>(in * rp * 4));
  l.w_dq_t = c.take(static_cast<size_t>(in * out * 2));
  const size_t pu = lora_down_part_bytes(T, in, rp), pv = lora_down_part_bytes(T, out, rp);
  l.part = c.take(pu > pv ? pu : pv);
  l.total = c.off;
  return l;
}

bool linear_shapes_ok(int64_t T, int64_t in, int64_t out, int64_t r) {
  if (T < 0 || in < 64 || out < 64 || (in % 64) != 0 || (out % 64) != 0) return false;
  if (r < 1 || r > QLORA_MAX_RANK) return false;
  if (in > (int64_t(1) << 31) || out > (int64_t(1) << 31) || T > (int64_t(1) << 31)) return false;
  return true;
}

int check_weight(const qlora_nf4_weight* W) {
  if (W == nullptr || W->codes == nullptr || W->absmax_q == nullptr || W->absmax_scale == nullptr)
    return QLORA_ERR_NULL;
  if (!aligned16(W->codes) || !aligned16(W->absmax_q) || !aligned16(W->absmax_scale))
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
  if (numel > (int64_t(1) << 45)) return QLORA_ERR_SHAPE;
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
  if (numel > (int64_t(1) << 45)) return QLORA_ERR_SHAPE;
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
  if (numel > (int64_t(1) << 45)) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!w || !codes || !absmax) return QLORA_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;
  return launched(launch_nf4_quantize_nodq(w, numel, codes, absmax, static_cast<hipStream_t>(stream)));
}

int nf4_dequantize_nodq(const uint8_t* codes, const float* absmax, int64_t numel, qlora_bf16* w_out,
                        qlora_stream stream) {
  if (numel < 0 || (numel % kBlock) != 0) return QLORA_ERR_SHAPE;
  if (numel > (int64_t(1) << 45)) return QLORA_ERR_SHAPE;
  if (numel == 0) return QLORA_OK;
  if (!codes || !absmax || !w_out) return QLORA_ERR_NULL;
  if (!aligned16(codes) || !aligned16(absmax) || !aligned16(w_out)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;
  return launched(launch_nf4_dequantize_nodq(codes, absmax, numel, w_out, static_cast<hipStream_t>(stream)));
}

size_t qlora_workspace_bytes(int64_t T, int64_t in_features, int64_t out_features, int64_t r,
                             int backward) {
  if (!linear_shapes_ok(T, in_features, out_features, r)) return 0;
  const size_t need = backward ? bwd_layout(T, in_features, out_features, r).total
                               : fwd_layout(T, in_features, out_features, r).total;
  return need > kMinWorkspace ? need : kMinWorkspace;
}

int qlora_linear_fwd(const qlora_nf4_weight* W, const qlora_bf16* X, int64_t T,
                     const qlora_bf16* A, const qlora_bf16* B, int64_t r, float alpha,
                     qlora_bf16* Y, void* ws, size_t ws_bytes, qlora_stream stream) {
  if (int st = check_weight(W)) return st;
  const int64_t out = W->rows, in = W->cols;
  if (!linear_shapes_ok(T, in, out, r)) return QLORA_ERR_SHAPE;
  if (!A || !B) return QLORA_ERR_NULL;
  if (T > 0 && (!X || !Y)) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y)) return QLORA_ERR_ALIGN;
  if (!std::isfinite(alpha)) return QLORA_ERR_VALUE;
  if (T == 0) return QLORA_OK;
  const FwdLayout lay = fwd_layout(T, in, out, r);
  if (lay.total > 0 && (ws == nullptr || ws_bytes < lay.total)) return QLORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = alpha / static_cast<float>(r);
  if (fwd_uses_decode(T, in, out, r))
    return launched(launch_decode_fwd(W->codes, W->absmax_q, W->absmax_scale, in, out, X, T, A, B,
                                      r, scale, Y, s));

  const int64_t rp = padded_rank(r);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* u_pad = reinterpret_cast<uint16_t*>(base + lay.u_pad);
  uint16_t* b_pad = reinterpret_cast<uint16_t*>(base + lay.b_pad);
  float* part = reinterpret_cast<float*>(base + lay.part);
  hipError_t e = launch_lora_down(X, T, in, A, r, scale, u_pad, nullptr, 0, rp, part, s);  // s X A^T
  if (e == hipSuccess) e = launch_pad_bf16(B, out, r, false, b_pad, rp, s);
  if (e == hipSuccess)
    e = launch_gemm_nf4(T, out, X, in, W->codes, W->absmax_q, W->absmax_scale, in, u_pad, 2 * rp,
                        b_pad, 2 * rp, 2 * rp, Y, out, s);
  return launched(e);
}

int qlora_linear_bwd(const qlora_nf4_weight* W, const qlora_bf16* X, const qlora_bf16* dY,
                     int64_t T, const qlora_bf16* A, const qlora_bf16* B, int64_t r, float alpha,
                     qlora_bf16* dX, float* dA, float* dB, void* ws, size_t ws_bytes,
                     qlora_stream stream) {
  if (int st = check_weight(W)) return st;
  const int64_t out = W->rows, in = W->cols;
  if (!linear_shapes_ok(T, in, out, r)) return QLORA_ERR_SHAPE;
  if (!A || !B || !dA || !dB) return QLORA_ERR_NULL;
  if (T > 0 && (!X || !dY || !dX)) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(A) || !aligned16(B) || !aligned16(dX) ||
      !aligned16(dA) || !aligned16(dB))
    return QLORA_ERR_ALIGN;
  if (!std::isfinite(alpha)) return QLORA_ERR_VALUE;
  const BwdLayout lay = bwd_layout(T, in, out, r);
  if (T > 0 && (ws == nullptr || ws_bytes < lay.total)) return QLORA_ERR_WORKSPACE;
  if (ws != nullptr && !aligned16(ws)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_fill_f32(dA, r * in, 0.f, s);
  if (e == hipSuccess) e = launch_fill_f32(dB, out * r, 0.f, s);
  if (T == 0 || e != hipSuccess) return launched(e);

  const float scale = alpha / static_cast<float>(r);
  const int64_t rp = padded_rank(r), tp = token_pitch(T);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* ut = reinterpret_cast<uint16_t*>(base + lay.ut);
  uint16_t* vt = reinterpret_cast<uint16_t*>(base + lay.vt);
  uint16_t* v_pad = reinterpret_cast<uint16_t*>(base + lay.v_pad);
  uint16_t* b_t = reinterpret_cast<uint16_t*>(base + lay.b_t);
  uint16_t* a_t_pad = reinterpret_cast<uint16_t*>(base + lay.a_t_pad);
  uint16_t* w_dq_t = reinterpret_cast<uint16_t*>(base + lay.w_dq_t);

  float* part = reinterpret_cast<float*>(base + lay.part);
  e = launch_lora_down(X, T, in, A, r, scale, nullptr, ut, tp, rp, part, s);           // (sU)^T
  if (e == hipSuccess) e = launch_transpose_bf16(B, out, r, b_t, s);                  // B^T [r][out]
  if (e == hipSuccess) e = launch_lora_down(dY, T, out, b_t, r, scale, v_pad, vt, tp, rp, part, s);  // sV
  if (e == hipSuccess) e = launch_pad_bf16(A, in, r, true, a_t_pad, rp, s);           // A^T padded
  if (e == hipSuccess)
    e = launch_nf4_dequantize_transposed(W->codes, W->absmax_q, W->absmax_scale, out, in, w_dq_t, s);
  if (e == hipSuccess)
    e = launch_gemm_nt(T, in, dY, out, w_dq_t, out, out, v_pad, 2 * rp, a_t_pad, 2 * rp, 2 * rp, dX, in, s);
  if (e == hipSuccess) e = launch_lora_grad(vt, T, tp, rp, X, in, r, dA, true, s);    // dA = (sV)^T X
  if (e == hipSuccess) e = launch_lora_grad(ut, T, tp, rp, dY, out, r, dB, false, s); // dB = dY^T (sU)
  return launched(e);
}

size_t qlora_merge_workspace_bytes(int64_t in_features, int64_t out_features, int64_t r) {
  if (!linear_shapes_ok(0, in_features, out_features, r)) return 0;
  const int64_t rp = padded_rank(r);
  Carve c;
  c.take(static_cast<size_t>(out_features * rp * 4));  // B padded [out][2 rp]
  c.take(static_cast<size_t>(in_features * rp * 4));   // A^T padded [in][2 rp]
  return c.off > kMinWorkspace ? c.off : kMinWorkspace;
}

int qlora_merge(const qlora_nf4_weight* W, const qlora_bf16* A, const qlora_bf16* B, int64_t r,
                float alpha, qlora_bf16* W_out, void* ws, size_t ws_bytes, qlora_stream stream) {
  if (int st = check_weight(W)) return st;
  const int64_t out = W->rows, in = W->cols;
  if (!linear_shapes_ok(0, in, out, r)) return QLORA_ERR_SHAPE;
  if (!A || !B || !W_out) return QLORA_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(W_out)) return QLORA_ERR_ALIGN;
  if (!std::isfinite(alpha)) return QLORA_ERR_VALUE;
  const size_t need = qlora_merge_workspace_bytes(in, out, r);
  if (ws == nullptr || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (int st = check_device()) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rp = padded_rank(r);
  uint16_t* b_pad = static_cast<uint16_t*>(ws);
  uint16_t* a_t_pad = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + round_up(out * rp * 4, 256));
  hipError_t e = launch_pad_bf16(B, out, r, false, b_pad, rp, s);
  if (e == hipSuccess) e = launch_pad_bf16(A, in, r, true, a_t_pad, rp, s);
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
