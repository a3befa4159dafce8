// k_lora.hip -- the rank-r parts of the QLoRA linear (paperclase lesson
// "QLoRA", Parte 4: h = W_hat x + (alpha/r) B A x and its gradients):
//   F1  U = X A^T            B1  V = dY B
//   B3  dA = s V^T X         dB = s dY^T U
// plus zero-padding / transposition of the small LoRA matrices into the
// layouts the GEMM's extra K-steps read.  All fp32 accumulation.
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// lora_down: U[t][j] = sum_k in[t][k] * P(j, k) over a [32 tokens x 64 ranks]
// tile per workgroup, K staged through LDS in chunks of 64 (converted to
// fp32).  Thread (tt = tid/8, jg = tid%8) owns 8 consecutive ranks of token tt.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lora_down(const uint16_t* __restrict__ in, int64_t T,
                                                   int64_t K, const uint16_t* __restrict__ p,
                                                   int p_rows_are_r, int64_t r, float scale,
                                                   float* __restrict__ u_out,
                                                   uint16_t* __restrict__ u_pad, int64_t rp) {
  __shared__ float s_in[32][65];
  __shared__ __attribute__((aligned(16))) float s_p[64][64];  // [k][j]
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int64_t j0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int tt = tid >> 3, jg = tid & 7;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < K; k0 += 64) {
    {  // activations: 32 rows x 64 k, 16 B per thread
      const int row = tid >> 3, q = tid & 7;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (t0 + row < T) v = *reinterpret_cast<const u32x4*>(in + (t0 + row) * K + k0 + q * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_in[row][q * 8 + 2 * e] = bf16_lo(v[e]);
        s_in[row][q * 8 + 2 * e + 1] = bf16_hi(v[e]);
      }
    }
    {  // P tile, 64 j x 64 k, 16 elements per thread, stored [k][j]
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int idx = e * 256 + tid;
        const int jj = p_rows_are_r ? (idx >> 6) : (idx & 63);
        const int kk = p_rows_are_r ? (idx & 63) : (idx >> 6);
        const int64_t j = j0 + jj, k = k0 + kk;
        float val = 0.f;
        if (j < r) {
          const uint16_t b = p_rows_are_r ? p[j * K + k] : p[k * r + j];
          val = __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
        }
        s_p[kk][jj] = val;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 64; ++kk) {
      const float a = s_in[tt][kk];
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(&s_p[kk][jg * 8]);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(&s_p[kk][jg * 8 + 4]);
      acc[0] += a * p0.x; acc[1] += a * p0.y; acc[2] += a * p0.z; acc[3] += a * p0.w;
      acc[4] += a * p1.x; acc[5] += a * p1.y; acc[6] += a * p1.z; acc[7] += a * p1.w;
    }
    __syncthreads();
  }
  const int64_t t = t0 + tt;
  if (t >= T) return;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t j = j0 + jg * 8 + e;
    if (u_out != nullptr && j < r) u_out[t * r + j] = acc[e];
  }
  if (u_pad != nullptr) {
    // s*U as a bf16 pair hi + lo (hi = bf16(s*U), lo = bf16(s*U - hi)): row t
    // holds hi in columns [0, rp) and lo in [rp, 2*rp)
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v0 = scale * acc[2 * e], v1 = scale * acc[2 * e + 1];
      hi[e] = pack_bf16x2(v0, v1);
      lo[e] = pack_bf16x2(v0 - bf16_lo(hi[e]), v1 - bf16_hi(hi[e]));
    }
    const int64_t j = j0 + jg * 8;
    if (j < rp) {
      uint16_t* row = u_pad + t * (2 * rp);
      *reinterpret_cast<u32x4*>(row + j) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<u32x4*>(row + rp + j) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
}

hipError_t launch_lora_down(const uint16_t* in, int64_t T, int64_t K, const uint16_t* p,
                            bool p_rows_are_r, int64_t r, float scale, float* u_out,
                            uint16_t* u_pad, int64_t rp, hipStream_t s) {
  const int64_t jt = u_pad != nullptr ? rp / 64 : ceil_div(r, 64);
  hipLaunchKernelGGL(k_lora_down, dim3(static_cast<uint32_t>(ceil_div(T, 32)),
                                       static_cast<uint32_t>(jt)),
                     dim3(256), 0, s, in, T, K, p, p_rows_are_r ? 1 : 0, r, scale, u_out, u_pad, rp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// lora_grad: G(j, c) = scale * sum_t P[t][j] Q[t][c].  Workgroup = 64 columns x
// 64 ranks x a slice of 256 tokens; wave w owns ranks j0 + 16w .. +16; lane =
// column.  Partial sums over token slices are combined with fp32 atomics into
// a zeroed output.
// ---------------------------------------------------------------------------
constexpr int kGradSlice = 256;

__global__ __launch_bounds__(256) void k_lora_grad(const float* __restrict__ P,
                                                   const uint16_t* __restrict__ Q, int64_t T,
                                                   int64_t r, int64_t C, float scale,
                                                   float* __restrict__ out, int out_jc) {
  __shared__ __attribute__((aligned(16))) float s_p[64][64];  // [t][j]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const int64_t j0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int64_t ts = static_cast<int64_t>(blockIdx.z) * kGradSlice;
  const int64_t te = ts + kGradSlice < T ? ts + kGradSlice : T;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  for (int64_t tb = ts; tb < te; tb += 64) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = e * 256 + tid;
      const int tt = idx >> 6, jj = idx & 63;
      const int64_t t = tb + tt, j = j0 + jj;
      s_p[tt][jj] = (t < te && j < r) ? P[t * r + j] : 0.f;
    }
    __syncthreads();
    const int n = static_cast<int>(te - tb < 64 ? te - tb : 64);
    for (int tt = 0; tt < n; ++tt) {
      const float q = __builtin_bit_cast(float, static_cast<uint32_t>(Q[(tb + tt) * C + c]) << 16);
      const f32x4* pr = reinterpret_cast<const f32x4*>(&s_p[tt][wv * 16]);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 pv = pr[e4];
        acc[4 * e4 + 0] += pv.x * q;
        acc[4 * e4 + 1] += pv.y * q;
        acc[4 * e4 + 2] += pv.z * q;
        acc[4 * e4 + 3] += pv.w * q;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t j = j0 + wv * 16 + e;
    if (j < r) {
      float* dst = out_jc ? out + j * C + c : out + c * r + j;
      atomicAdd(dst, scale * acc[e]);
    }
  }
}

hipError_t launch_lora_grad(const float* P, const uint16_t* Q, int64_t T, int64_t r, int64_t C,
                            float scale, float* out, bool out_jc, hipStream_t s) {
  hipLaunchKernelGGL(k_lora_grad,
                     dim3(static_cast<uint32_t>(C / 64), static_cast<uint32_t>(ceil_div(r, 64)),
                          static_cast<uint32_t>(ceil_div(T, kGradSlice))),
                     dim3(256), 0, s, P, Q, T, r, C, scale, out, out_jc ? 1 : 0);
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
