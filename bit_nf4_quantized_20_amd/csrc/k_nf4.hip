// k_nf4.hip -- NF4 quantize (Q1..Q4) and dequantize (D1) kernels for gfx950.
//
// Quantize follows ultralytics glossary "QLoRA", "Como funciona a QLoRA"
// (absmax per 64 weights, nearest normal-quantile level, absmax values to 8
// bits in blocks of 256) and paperclase lesson "QLoRA", Parte 4 (argmin of the
// distance to the levels, two codes per byte).  Dequantize follows paperclase
// Parte 2 (w_hat = NF4[c] * absmax) with the bf16 result of ultralytics
// "QLoRA" (dequantized to bfloat16 right before the matmul).
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

// ---------------------------------------------------------------------------
// Quantize: one workgroup per double-quant group (256 blocks = 16384 fp32 =
// 64 KiB), 256 threads, single HBM pass.  Thread t loads float4 chunks
// f = i*256 + t (i = 0..15): each load instruction covers 1 KiB contiguous per
// wave, and the 16 chunks of one 64-weight block sit in 16 adjacent lanes,
// so the block absmax is a 16-lane DPP max.
// ---------------------------------------------------------------------------
// kDQ = false: no double quantization; absmax_q and scale are unused and
// the exact fp32 block absmax goes to absmax[numel/64] (4.5 bits per weight).
template <bool kDQ>
__global__ __launch_bounds__(256) void k_nf4_quantize(const float* __restrict__ w, int64_t numel,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ absmax_q,
                                                      float* __restrict__ scale,
                                                      float* __restrict__ absmax) {
  __shared__ float wave_max[4];
  const int t = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t base = g * kGroupElems;

  f32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t e = base + static_cast<int64_t>(i * 256 + t) * 4;
    if (e < numel)
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w + e));
    else
      v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Q1: block absmax (exact max of |w|), replicated over the block's 16 lanes
  float am[16];
  float tmax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
    m = max16(m);
    am[i] = m;
    tmax = fmaxf(tmax, m);
  }
  if constexpr (!kDQ) {
    if ((t & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t e = base + static_cast<int64_t>(i * 256 + t) * 4;
        if (e < numel) absmax[e >> 6] = am[i];
      }
    }
  }
  // group scale s_g = max over the 256 blocks
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  if ((t & 63) == 0) wave_max[t >> 6] = tmax;
  __syncthreads();
  const float sg = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));

  // Q2: 8-bit absmax codes, q = rne(fl32(fl32(a / s) * 255)); zero group -> 0
  if (kDQ && (t & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t e = base + static_cast<int64_t>(i * 256 + t) * 4;
      if (e < numel) {
        uint32_t q = 0;
        if (sg > 0.f) {
          const float ratio = am[i] / sg;
          const float scaled = ratio * 255.0f;
          q = static_cast<uint32_t>(__builtin_rintf(scaled));
        }
        absmax_q[e >> 6] = static_cast<uint8_t>(q);
      }
    }
  }
  if (kDQ && t == 0) scale[g] = sg;

  // Q3 + Q4: codes from x = fl32(w / a) and the 15 thresholds; a zero block
  // has x = 0 everywhere (code 7).  4 codes -> 16 bits per chunk.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t e = base + static_cast<int64_t>(i * 256 + t) * 4;
    if (e < numel) {
      const float a = am[i];
      uint32_t c0, c1, c2, c3;
      if (a > 0.f) {
        c0 = nf4_code(v[i].x / a);
        c1 = nf4_code(v[i].y / a);
        c2 = nf4_code(v[i].z / a);
        c3 = nf4_code(v[i].w / a);
      } else {
        c0 = c1 = c2 = c3 = 7u;
      }
      const uint16_t packed = static_cast<uint16_t>(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
      *reinterpret_cast<uint16_t*>(codes + (e >> 1)) = packed;
    }
  }
}

hipError_t launch_nf4_quantize(const float* w, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                               float* scale, hipStream_t s) {
  const int64_t groups = ceil_div(numel, kGroupElems);
  hipLaunchKernelGGL(k_nf4_quantize<true>, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, s, w,
                     numel, codes, absmax_q, scale, nullptr);
  return hipGetLastError();
}

hipError_t launch_nf4_quantize_nodq(const float* w, int64_t numel, uint8_t* codes, float* absmax,
                                    hipStream_t s) {
  const int64_t groups = ceil_div(numel, kGroupElems);
  hipLaunchKernelGGL(k_nf4_quantize<false>, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, s, w,
                     numel, codes, nullptr, nullptr, absmax);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize: each thread expands 32 weights (16 code bytes, half a block)
// into 64 bytes of bf16 with the per-block v_perm table.  The results go
// through a per-wave LDS buffer so that each store instruction writes 1 KB
// of consecutive output (a lane's own 64 bytes written directly would put
// 64 separate 16-byte pieces into every store instruction).
// ---------------------------------------------------------------------------
// kDQ = false: a_hat is the fp32 block absmax (absmax[blk]) itself.
template <bool kDQ>
__global__ __launch_bounds__(256) void k_nf4_dequantize(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ absmax_q,
                                                        const float* __restrict__ scale,
                                                        const float* __restrict__ absmax,
                                                        int64_t numel, uint16_t* __restrict__ out) {
  __shared__ u32x4 s_o[4][64 * 5];  // lane l's four pieces at 5 l .. 5 l + 3 (conflict-free)
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nch = numel / 32;  // 32-weight chunks
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  u32x4* so = s_o[wv];
  if (c < nch) {
    const int64_t blk = c >> 1;
    const float ahat = kDQ ? dq_absmax(absmax_q[blk], scale[blk >> 8]) : absmax[blk];
    const Nf4Table tab = make_table(ahat);
    const u32x4 cw = *reinterpret_cast<const u32x4*>(codes + c * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t o[4];
      lookup8(tab, cw[k], o);
      so[lane * 5 + k] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
  // the buffer is private to this wave: a wave-level barrier orders the
  // writes of all lanes before the reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the wave's 64 chunks are 4 KB of consecutive output: piece P (16 B) is
  // piece P % 4 of chunk P / 4
  const int64_t cw0 = static_cast<int64_t>(blockIdx.x) * 256 + wv * 64;
  u32x4* dst = reinterpret_cast<u32x4*>(out + cw0 * 32);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int P = 64 * k + lane, sl = P >> 2;
    if (cw0 + sl < nch) dst[P] = so[sl * 5 + (P & 3)];
  }
}

hipError_t launch_nf4_dequantize(const uint8_t* codes, const uint8_t* absmax_q, const float* scale,
                                 int64_t numel, uint16_t* out, hipStream_t s) {
  const int64_t chunks = numel / 32;
  hipLaunchKernelGGL(k_nf4_dequantize<true>, dim3(static_cast<uint32_t>(ceil_div(chunks, 256))),
                     dim3(256), 0, s, codes, absmax_q, scale, nullptr, numel, out);
  return hipGetLastError();
}

hipError_t launch_nf4_dequantize_nodq(const uint8_t* codes, const float* absmax, int64_t numel,
                                      uint16_t* out, hipStream_t s) {
  const int64_t chunks = numel / 32;
  hipLaunchKernelGGL(k_nf4_dequantize<false>, dim3(static_cast<uint32_t>(ceil_div(chunks, 256))),
                     dim3(256), 0, s, codes, nullptr, nullptr, absmax, numel, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Transposed dequantize (the backward's W_hat^T): one wave per 64 x 64 tile.
// Lane l dequantizes the tile's part of weight row r0 + l (one block) into an
// LDS tile, piece p (8 columns, 16 B) of row r at slot 8 r + (p ^ key(r)),
// key(r) = (r ^ (r >> 3)) & 7, which keeps both the row writes and the
// transposed 16-bit reads free of bank conflicts.  Then eight lanes write one
// output row: lane l takes output row (l >> 3) + 8 i and its elements
// 8 (l & 7) .. + 7, so each store instruction writes eight full 128-byte
// row segments.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_nf4_dequantize_t(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ absmax_q,
                                                          const float* __restrict__ scale,
                                                          int64_t rows, int64_t cols,
                                                          uint16_t* __restrict__ out, int64_t ldo) {
  __shared__ u32x4 tile[4][64 * 8];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t col_blocks = cols / 64;
  const int64_t tile_id = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  const int64_t n_tiles = (rows / 64) * col_blocks;
  if (tile_id >= n_tiles) return;  // whole wave leaves; no workgroup barrier below
  const int64_t r0 = (tile_id / col_blocks) * 64, c0 = (tile_id % col_blocks) * 64;
  u32x4* tl = tile[wv];
  const int64_t row = r0 + lane;
  const int64_t blk = (row * cols + c0) >> 6;
  const Nf4Table tab = make_table(dq_absmax(absmax_q[blk], scale[blk >> 8]));
  const u32x4* src = reinterpret_cast<const u32x4*>(codes + ((row * cols + c0) >> 1));
  const int key = (lane ^ (lane >> 3)) & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 cw = src[h];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t o[4];
      lookup8(tab, cw[k], o);
      tl[lane * 8 + ((4 * h + k) ^ key)] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
  // the tile is private to this wave: a wave-level barrier orders the LDS
  // writes of all lanes before the transposed reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint16_t* t16 = reinterpret_cast<const uint16_t*>(tl);
  const int pr = lane & 7, cl = lane >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cc = cl + 8 * i;  // output row c0 + cc = weight column; its piece i of the tile row
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ra = 8 * pr + 2 * e, rb = ra + 1;
      const int ka = (ra ^ (ra >> 3)) & 7, kb = (rb ^ (rb >> 3)) & 7;
      const uint32_t va = t16[(ra * 8 + (i ^ ka)) * 8 + cl];
      const uint32_t vb = t16[(rb * 8 + (i ^ kb)) * 8 + cl];
      d[e] = va | (vb << 16);
    }
    *reinterpret_cast<u32x4*>(out + (c0 + cc) * ldo + r0 + 8 * pr) = u32x4{d[0], d[1], d[2], d[3]};
  }
}

hipError_t launch_nf4_dequantize_transposed(const uint8_t* codes, const uint8_t* absmax_q,
                                            const float* scale, int64_t rows, int64_t cols,
                                            uint16_t* out, int64_t ldo, hipStream_t s) {
  const int64_t tiles = (rows / 64) * (cols / 64);
  hipLaunchKernelGGL(k_nf4_dequantize_t, dim3(static_cast<uint32_t>(ceil_div(tiles, 4))), dim3(256),
                     0, s, codes, absmax_q, scale, rows, cols, out, ldo);
  return hipGetLastError();
}

}  // namespace qlora
