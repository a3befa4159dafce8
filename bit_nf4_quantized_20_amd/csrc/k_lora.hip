// k_lora.hip -- the rank-r parts of the QLoRA linear (paperclase lesson
// "QLoRA", Parte 4: h = W_hat x + (alpha/r) B A x and its gradients), on MFMA:
//   F1  sU = s X A^T             B1  sV = s dY B
//   B3  dA = (sV)^T X            dB = dY^T (sU)
// sU and sV are kept as bf16 pairs hi + lo (hi = bf16(v), lo = bf16(v - hi)),
// so products with them carry ~16 bits of the fp32 value; all accumulation is
// fp32.  Also the zero-padding / transposition of the small LoRA matrices
// into the layouts the GEMM's extra K-steps read.
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

typedef float f32x4v __attribute__((ext_vector_type(4)));

namespace {
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
}  // namespace

// ---------------------------------------------------------------------------
// lora_down: D[j][t] = sum_k P[j][k] in[t][k] for 16 tokens per workgroup and
// all ranks.  4 waves split K in 32-wide slices (wave w takes slices w, w+4,
// ...); per slice a lane (n = l%16, g = l/16) loads 8 activations of token
// t0+n and 8 weights of rank row 16*rt+n, and each rank tile issues one
// v_mfma_f32_16x16x32_bf16.  Partial tiles meet in LDS.
// ---------------------------------------------------------------------------
template <int RT>
__global__ __launch_bounds__(256) void k_lora_down(const uint16_t* __restrict__ in, int64_t T,
                                                   int64_t K, const uint16_t* __restrict__ P,
                                                   int r, float scale, uint16_t* __restrict__ pad,
                                                   uint16_t* __restrict__ hilo_t, int64_t ldt,
                                                   int rp) {
  __shared__ f32x4v red[4][RT][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
  const bool tok_ok = t0 + n < T;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  f32x4v acc[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) acc[i] = f32x4v{0.f, 0.f, 0.f, 0.f};

  const int64_t slices = K / 32;
  const uint16_t* xrow = in + (t0 + n) * K + 8 * g;
  int64_t sl = wv;
  // two slices per iteration so the loads of both are in flight together
  for (; sl + 4 < slices; sl += 8) {
    const int64_t k0 = sl * 32, k1 = (sl + 4) * 32;
    const u32x4 x0 = tok_ok ? *reinterpret_cast<const u32x4*>(xrow + k0) : zero4;
    const u32x4 x1 = tok_ok ? *reinterpret_cast<const u32x4*>(xrow + k1) : zero4;
    u32x4 p0[RT], p1[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int j = rt * 16 + n;
      const uint16_t* prow = P + static_cast<int64_t>(j) * K + 8 * g;
      p0[rt] = j < r ? *reinterpret_cast<const u32x4*>(prow + k0) : zero4;
      p1[rt] = j < r ? *reinterpret_cast<const u32x4*>(prow + k1) : zero4;
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p0[rt]), as_bf16x8(x0), acc[rt], 0, 0, 0);
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p1[rt]), as_bf16x8(x1), acc[rt], 0, 0, 0);
    }
  }
  for (; sl < slices; sl += 4) {
    const int64_t k0 = sl * 32;
    const u32x4 x0 = tok_ok ? *reinterpret_cast<const u32x4*>(xrow + k0) : zero4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int j = rt * 16 + n;
      const u32x4 p0 = j < r ? *reinterpret_cast<const u32x4*>(P + static_cast<int64_t>(j) * K + 8 * g + k0) : zero4;
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p0), as_bf16x8(x0), acc[rt], 0, 0, 0);
    }
  }

  // lane holds D[16*rt + 4*g + i][n], i = 0..3
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) red[wv][rt][lane] = acc[rt];
  __syncthreads();
  // thread -> (token tt = tid % 16, rank j = tid / 16 + 16 * m)
  const int tt = tid & 15;
  const int64_t t = t0 + tt;
  if (t >= T) return;
  for (int j = tid >> 4; j < rp; j += 16) {
    float v = 0.f;
    if (j < 16 * RT) {
      const int rt = j >> 4, gi = (j & 15) >> 2, i = j & 3;
      const int l = tt + 16 * gi;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += red[w][rt][l][i];
    }
    v *= scale;  // zero for j >= r (rows of P beyond r are zero)
    const float hi = __builtin_bit_cast(float, static_cast<uint32_t>(pack_bf16x2(v, 0.f)) << 16);
    const uint16_t hb = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
    const uint16_t lb = static_cast<uint16_t>(pack_bf16x2(v - hi, 0.f) & 0xffffu);
    if (pad != nullptr) {
      pad[t * 2 * rp + j] = hb;
      pad[t * 2 * rp + rp + j] = lb;
    }
    if (hilo_t != nullptr) {
      hilo_t[static_cast<int64_t>(j) * ldt + t] = hb;
      hilo_t[static_cast<int64_t>(rp + j) * ldt + t] = lb;
    }
  }
}

hipError_t launch_lora_down(const uint16_t* in, int64_t T, int64_t K, const uint16_t* P, int64_t r,
                            float scale, uint16_t* pad, uint16_t* hilo_t, int64_t ldt, int64_t rp,
                            hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(ceil_div(T, 16))), block(256);
  const int rt = static_cast<int>(ceil_div(r, 16));
  const int ir = static_cast<int>(r), irp = static_cast<int>(rp);
#define QLORA_DOWN(RTV) hipLaunchKernelGGL((k_lora_down<RTV>), grid, block, 0, s, in, T, K, P, ir, scale, pad, hilo_t, ldt, irp)
  if (rt <= 1) QLORA_DOWN(1);
  else if (rt <= 2) QLORA_DOWN(2);
  else if (rt <= 4) QLORA_DOWN(4);
  else if (rt <= 8) QLORA_DOWN(8);
  else QLORA_DOWN(16);
#undef QLORA_DOWN
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// lora_grad: G[j][c] = sum_t Pt[j][t] Q[t][c] + sum_t Pt[rp+j][t] Q[t][c]
// (the hi and lo halves of the transposed rank factor), for 64 columns per
// workgroup and a slice of tokens; partial sums over token slices go to the
// zeroed fp32 output with atomics.  The Q tile [64 t][64 c] is transposed on
// its way into LDS (pairs of token rows interleaved with v_perm, written as
// dwords) so the MFMA B operand reads 8 consecutive tokens of one column.
// Wave w owns the 32x32 output tiles (jt, ct) with jt*2 + ct = w (mod 4).
// ---------------------------------------------------------------------------
constexpr int kGradSlice = 512;
constexpr int kQPitch = 72;  // bf16 per LDS row (144 B, 16-byte aligned rows)

template <int JT>  // rank tiles of 32
__global__ __launch_bounds__(256) void k_lora_grad(const uint16_t* __restrict__ Pt, int64_t T,
                                                   int64_t ldt, int rp,
                                                   const uint16_t* __restrict__ Q, int64_t C, int r,
                                                   float* __restrict__ out, int out_jc) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q[64 * kQPitch];
  constexpr int kTiles = JT * 2;                 // (jt, ct) tiles
  constexpr int kPerWave = (kTiles + 3) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t ts = static_cast<int64_t>(blockIdx.y) * kGradSlice;
  const int64_t te = ts + kGradSlice < T ? ts + kGradSlice : T;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  f32x16 acc[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  // staging role: token pair tp, column group cg (8 columns)
  const int tp = tid >> 3, cg = tid & 7;
  for (int64_t tb = ts; tb < te; tb += 64) {
    {
      const int64_t ta = tb + 2 * tp, tb1 = ta + 1;
      const u32x4 a = ta < te ? *reinterpret_cast<const u32x4*>(Q + ta * C + c0 + 8 * cg) : zero4;
      const u32x4 b = tb1 < te ? *reinterpret_cast<const u32x4*>(Q + tb1 * C + c0 + 8 * cg) : zero4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // columns 2e and 2e+1 of the group: (Q[ta][c], Q[tb1][c]) pairs
        const uint32_t lo = perm(b[e], a[e], 0x05040100u);
        const uint32_t hi = perm(b[e], a[e], 0x07060302u);
        *reinterpret_cast<uint32_t*>(s_q + (8 * cg + 2 * e) * kQPitch + 2 * tp) = lo;
        *reinterpret_cast<uint32_t*>(s_q + (8 * cg + 2 * e + 1) * kQPitch + 2 * tp) = hi;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // 16 tokens per MFMA step
      const int64_t tk = tb + 16 * s + 8 * h;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int tile = wv + 4 * i;
        if (tile >= kTiles) continue;
        const int jt = tile >> 1, ct = tile & 1;
        const u32x4 qf = *reinterpret_cast<const u32x4*>(s_q + (32 * ct + r32) * kQPitch + 16 * s + 8 * h);
        const int j = 32 * jt + r32;
        u32x4 ph = zero4, pl = zero4;
        if (tk < te && j < rp) {  // te - tk is a multiple of 8 except at the very end
          const uint16_t* rh = Pt + static_cast<int64_t>(j) * ldt;
          const uint16_t* rl = Pt + static_cast<int64_t>(rp + j) * ldt;
          if (tk + 8 <= te) {
            ph = *reinterpret_cast<const u32x4*>(rh + tk);
            pl = *reinterpret_cast<const u32x4*>(rl + tk);
          } else {
            uint16_t hv[8], lv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool ok = tk + e < te;
              hv[e] = ok ? rh[tk + e] : 0;
              lv[e] = ok ? rl[tk + e] : 0;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ph[e] = hv[2 * e] | (static_cast<uint32_t>(hv[2 * e + 1]) << 16);
              pl[e] = lv[2 * e] | (static_cast<uint32_t>(lv[2 * e + 1]) << 16);
            }
          }
        }
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ph), as_bf16x8(qf), acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pl), as_bf16x8(qf), acc[i], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // D[j][c]: lane holds column c = r32, rows j = 8*(e/4) + 4*h + e%4
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int tile = wv + 4 * i;
    if (tile >= kTiles) continue;
    const int jt = tile >> 1, ct = tile & 1;
    const int64_t c = c0 + 32 * ct + r32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = 32 * jt + 8 * (e >> 2) + 4 * h + (e & 3);
      if (j < r) {
        float* dst = out_jc ? out + static_cast<int64_t>(j) * C + c : out + c * r + j;
        atomicAdd(dst, acc[i][e]);
      }
    }
  }
}

hipError_t launch_lora_grad(const uint16_t* Pt, int64_t T, int64_t ldt, int64_t rp, const uint16_t* Q,
                            int64_t C, int64_t r, float* out, bool out_jc, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(C / 64), static_cast<uint32_t>(ceil_div(T, kGradSlice)));
  const int jt = static_cast<int>(ceil_div(r, 32));
  const int irp = static_cast<int>(rp), ir = static_cast<int>(r), jc = out_jc ? 1 : 0;
#define QLORA_GRAD(JTV) hipLaunchKernelGGL((k_lora_grad<JTV>), grid, dim3(256), 0, s, Pt, T, ldt, irp, Q, C, ir, out, jc)
  if (jt <= 1) QLORA_GRAD(1);
  else if (jt <= 2) QLORA_GRAD(2);
  else if (jt <= 4) QLORA_GRAD(4);
  else QLORA_GRAD(8);
#undef QLORA_GRAD
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pad_bf16(const uint16_t* __restrict__ src, int64_t R,
                                                  int64_t C, int transpose,
                                                  uint16_t* __restrict__ dst, int64_t Cp) {
  // dst row i = [src row i zero-padded to Cp | the same again]
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= R * Cp) return;
  const int64_t i = idx / Cp, j = idx % Cp;
  uint16_t v = 0;
  if (j < C) v = transpose ? src[j * R + i] : src[i * C + j];
  dst[i * 2 * Cp + j] = v;
  dst[i * 2 * Cp + Cp + j] = v;
}

hipError_t launch_pad_bf16(const uint16_t* src, int64_t R, int64_t C, bool transpose, uint16_t* dst,
                           int64_t Cp, hipStream_t s) {
  hipLaunchKernelGGL(k_pad_bf16, dim3(static_cast<uint32_t>(ceil_div(R * Cp, 256))), dim3(256), 0,
                     s, src, R, C, transpose ? 1 : 0, dst, Cp);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src, int64_t R,
                                                        int64_t C, uint16_t* __restrict__ dst) {
  // dst[c][r] = src[r][c]
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= R * C) return;
  const int64_t c = idx / R, rr = idx % R;
  dst[idx] = src[rr * C + c];
}

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst,
                                 hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_bf16, dim3(static_cast<uint32_t>(ceil_div(R * C, 256))), dim3(256),
                     0, s, src, R, C, dst);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ dst, int64_t n, float v) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx < n) dst[idx] = v;
}

hipError_t launch_fill_f32(float* dst, int64_t n, float v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_f32, dim3(static_cast<uint32_t>(ceil_div(n, 256))), dim3(256), 0, s,
                     dst, n, v);
  return hipGetLastError();
}

}  // namespace qlora
