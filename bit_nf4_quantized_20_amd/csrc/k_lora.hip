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
  if (t >= T) {  // padding tokens of the transposed copy read as zero
    if (hilo_t != nullptr && t < ldt)
      for (int j = tid >> 4; j < rp; j += 16) {
        hilo_t[static_cast<int64_t>(j) * ldt + t] = 0;
        hilo_t[static_cast<int64_t>(rp + j) * ldt + t] = 0;
      }
    return;
  }
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
// (the hi and lo halves of the transposed rank factor) for ranks
// [j0, j0 + 32*JT), 128 columns per workgroup and a slice of tokens; slices
// add into the zeroed fp32 output with atomics.  Bound by streaming Q (dY or
// X) from HBM once.
//
// Per 64-token step the Q tile [64 t][128 c] and the Pt tile [64*JT rows][64 t]
// are loaded contiguously into registers one step ahead and written into a
// double-buffered LDS stage.  Q is transposed on the way: a thread holds two
// token rows of 8 columns, pairs them with v_perm and writes one dword
// (Q[2w][c], Q[2w+1][c]) per column; dword w of column c sits at
// 36c + (w ^ 4((c >> 4) & 7)), which makes both these writes and the MFMA
// fragment reads (8 tokens of one column) free of bank conflicts.  Wave w
// owns columns [32w, 32w + 32) and all JT rank tiles:
// v_mfma_f32_32x32x16_bf16 with Pt rows as A operand and Q columns as B.
// ---------------------------------------------------------------------------
constexpr int kGradCT = 128;    // columns per workgroup
constexpr int kGradPitch = 36;  // dwords per LDS row: 64 tokens + 8 padding
constexpr int kGradMaxJT = 4;   // rank tiles per launch (128 ranks)
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kPastEnd = 0x80000000u;

namespace {
__device__ __forceinline__ int grad_qslot(int c, int w) { return kGradPitch * c + (w ^ (4 * ((c >> 4) & 7))); }
}  // namespace

// kJC: output out[j*C + c] (else out[c*r + j]).  The MFMA orientation
// follows it, so a wave's 32 lanes always add to 32 consecutive floats.
template <int JT, bool kJC>
__global__ __launch_bounds__(256) void k_lora_grad(const uint16_t* __restrict__ Pt, int64_t T,
                                                   int64_t ldt, int rp, const uint16_t* __restrict__ Q,
                                                   int64_t C, int r, int j0, float* __restrict__ out,
                                                   int64_t TS) {
  constexpr int kPRows = 64 * JT;  // hi rows [0, 32JT), lo rows [32JT, 64JT)
  __shared__ uint32_t s_q[2][kGradCT * kGradPitch];
  __shared__ uint32_t s_p[2][kPRows * kGradPitch];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kGradCT;
  const int64_t ts = static_cast<int64_t>(blockIdx.y) * TS;
  const int64_t te = ts + TS < T ? ts + TS : T;
  const int nsteps = static_cast<int>((te - ts + 63) / 64);

  // Q resource starts at this slice and ends at row T (or 2^31 - 1 bytes;
  // the host keeps a slice under 2^30 bytes)
  const uint64_t q_bytes = static_cast<uint64_t>(T - ts) * C * 2;
  const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Q + ts * C), 0, static_cast<int>(q_bytes < 0x7fffffffu ? q_bytes : 0x7fffffffu),
      kBufferWord3);
  const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Pt), 0, static_cast<int>(static_cast<uint64_t>(2 * rp) * ldt * 2), kBufferWord3);

  // Q staging items: column group cg (8 columns), token pairs tp and tp + 16
  const int cg = tid & 15, tp0 = tid >> 4;
  const bool col_ok = c0 + 8 * cg < C;
  u32x4 qv[4];
  u32x4 pv[2 * JT];
  auto load = [&](int step) {
    const int64_t t0 = ts + 64 * static_cast<int64_t>(step);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 - ts + 2 * (tp0 + 16 * (i >> 1)) + (i & 1);  // rows past T read as zero
      const uint32_t off = col_ok ? static_cast<uint32_t>((t * C + c0 + 8 * cg) * 2) : kPastEnd;
      qv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_q, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 2 * JT; ++i) {
      const int id = tid + 256 * i, prow = id >> 3, q = id & 7;
      const int64_t grow = prow < 32 * JT ? j0 + prow : rp + j0 + (prow - 32 * JT);
      const int64_t tk = t0 + 8 * q;  // tokens in [T, ldt) are zero in Pt
      const uint32_t off = tk < ldt ? static_cast<uint32_t>((grow * ldt + tk) * 2) : kPastEnd;
      pv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_p, off, 0, 0));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 a = qv[2 * i], b = qv[2 * i + 1];
      const int w = tp0 + 16 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_q[buf][grad_qslot(8 * cg + 2 * e, w)] = perm(b[e], a[e], 0x05040100u);
        s_q[buf][grad_qslot(8 * cg + 2 * e + 1, w)] = perm(b[e], a[e], 0x07060302u);
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * JT; ++i) {
      const int id = tid + 256 * i, prow = id >> 3, q = id & 7;
      *reinterpret_cast<u32x4*>(&s_p[buf][kGradPitch * prow + 4 * q]) = pv[i];
    }
  };

  f32x16 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[jt][e] = 0.f;

  if (nsteps > 0) {
    load(0);
    store(0);
    if (nsteps > 1) load(1);
  }
  const int c = 32 * wv + r32;
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    __syncthreads();  // stage buf complete, stage buf ^ 1 free
    if (step + 1 < nsteps) {
      store(buf ^ 1);
      if (step + 2 < nsteps) load(step + 2);
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int w0 = 8 * s4 + 4 * h;
      const u32x4 qf = *reinterpret_cast<const u32x4*>(&s_q[buf][grad_qslot(c, w0)]);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 ph = *reinterpret_cast<const u32x4*>(&s_p[buf][kGradPitch * (32 * jt + r32) + w0]);
        const u32x4 pl = *reinterpret_cast<const u32x4*>(&s_p[buf][kGradPitch * (32 * JT + 32 * jt + r32) + w0]);
        if constexpr (kJC) {  // D[j][c]
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ph), as_bf16x8(qf), acc[jt], 0, 0, 0);
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pl), as_bf16x8(qf), acc[jt], 0, 0, 0);
        } else {  // D[c][j]
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qf), as_bf16x8(ph), acc[jt], 0, 0, 0);
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qf), as_bf16x8(pl), acc[jt], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (kJC) {
    // D[j][c]: lane holds column c, rows j = 8*(e/4) + 4*h + e%4
    const int64_t cc = c0 + c;
    if (cc >= C) return;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + 32 * jt + 8 * (e >> 2) + 4 * h + (e & 3);
        if (j < r) atomicAdd(out + static_cast<int64_t>(j) * C + cc, acc[jt][e]);
      }
  } else {
    // D[c][j]: lane holds rank j, rows c = 8*(e/4) + 4*h + e%4 of the wave's tile
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const int j = j0 + 32 * jt + r32;
      if (j >= r) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t cc = c0 + 32 * wv + 8 * (e >> 2) + 4 * h + (e & 3);
        if (cc < C) atomicAdd(out + cc * r + j, acc[jt][e]);
      }
    }
  }
}

hipError_t launch_lora_grad(const uint16_t* Pt, int64_t T, int64_t ldt, int64_t rp, const uint16_t* Q,
                            int64_t C, int64_t r, float* out, bool out_jc, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // token slices (multiples of 64) for about 512 workgroups
  const int64_t ctiles = ceil_div(C, kGradCT);
  int64_t slices = ceil_div(512, ctiles);
  const int64_t max_slices = ceil_div(T, 64);
  if (slices > max_slices) slices = max_slices;
  if (slices < 1) slices = 1;
  // 32-bit buffer offsets: a slice of Q stays under 2^30 bytes, Pt under 2^31
  const int64_t min_slices = ceil_div(T * C * 2, int64_t(1) << 30);
  if (slices < min_slices) slices = min_slices;
  if (2 * rp * ldt * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const int64_t TS = round_up(ceil_div(T, slices), 64);
  slices = ceil_div(T, TS);
  const dim3 grid(static_cast<uint32_t>(ctiles), static_cast<uint32_t>(slices));
  const int irp = static_cast<int>(rp), ir = static_cast<int>(r);
  for (int64_t j0 = 0; j0 < r; j0 += 32 * kGradMaxJT) {
    const int64_t left = r - j0;
    const int jt = static_cast<int>(ceil_div(left < 32 * kGradMaxJT ? left : 32 * kGradMaxJT, 32));
    const int ij0 = static_cast<int>(j0);
#define QLORA_GRAD(JTV, JC)                                                                          \
  hipLaunchKernelGGL((k_lora_grad<JTV, JC>), grid, dim3(256), 0, s, Pt, T, ldt, irp, Q, C, ir, ij0, out, TS)
    if (out_jc) {
      if (jt <= 1) QLORA_GRAD(1, true);
      else if (jt <= 2) QLORA_GRAD(2, true);
      else QLORA_GRAD(4, true);
    } else {
      if (jt <= 1) QLORA_GRAD(1, false);
      else if (jt <= 2) QLORA_GRAD(2, false);
      else QLORA_GRAD(4, false);
    }
#undef QLORA_GRAD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
