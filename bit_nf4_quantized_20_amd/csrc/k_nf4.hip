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
// Quantize: persistent workgroups of 1024 threads, one per CU, each walking
// double-quant groups g, g + G, g + 2G, ... (G workgroups; a group is 256
// blocks = 16384 fp32 = 64 KiB).  The next group's loads are issued before
// the current group's arithmetic, so every CU keeps a group of loads in
// flight while it computes: one HBM pass, read 4 B and write 0.516 B per
// weight.
//
// Within a group, thread t holds float4 chunks f = i*1024 + t (i = 0..3):
// each load instruction covers 1 KiB contiguous per wave, and the 16 chunks
// of one 64-weight block sit in 16 adjacent lanes, so the block absmax is a
// 16-lane DPP max (on the fp32 bit patterns of |w|, whose unsigned order is
// the order of the values).
//
// Per-block work is spread over the lanes instead of repeated in each of a
// block's 16: a wave holds 16 blocks (4 chunks x 4 lane groups), and lane
// l < 16 takes block (i = l % 4, lane group l / 4) for the block reciprocal,
// the 8-bit absmax code and the absmax store; the reciprocals go back to the
// lanes through LDS.  The group scale is needed only for the absmax codes,
// so the codes are stored before the workgroup barrier that forms it.
// ---------------------------------------------------------------------------
constexpr int kQThreads = 1024;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQChunks = kGroupElems / 4 / kQThreads;  // float4 chunks per thread
constexpr int kQBlocksPerWave = kQChunks * 4;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource, 32-bit data format
constexpr int kStreamOnce = 2;            // cache policy nt: each weight is read once
static_assert(kQChunks == 4, "one float4 of block values per lane group");

// the bucket table of the code lookup, copied into LDS by each workgroup
__constant__ BucketTable kBucketTableDev = kBucketTable;

__device__ __forceinline__ uint32_t abs_bits(float v) { return __builtin_bit_cast(uint32_t, v) & 0x7fffffffu; }

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  return max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xf, 0xf,
                                                                  false)));
}

// orders this wave's LDS writes before its later LDS reads
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// floor(X) as an integer (v_cvt_flr_i32_f32; NaN gives 0)
__device__ __forceinline__ int floor_to_int(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// 4 codes of one chunk from X = 16 w / a, packed into 16 bits
__device__ __forceinline__ uint32_t bucket_codes(const uint2* s_bucket, const float (&X)[4]) {
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint2 bk = s_bucket[floor_to_int(X[k]) + 16];
    const uint32_t c = bk.y + (X[k] > __builtin_bit_cast(float, bk.x) ? 1u : 0u);
    packed |= c << (4 * k);
  }
  return packed;
}

// Group g's chunks of this thread through a buffer resource over the group:
// chunks past numel (a ragged last group, or g past the last group) read as
// zero, without a branch, so the waits for these loads are counted exactly.
__device__ __forceinline__ void load_group(const float* w, int64_t numel, int64_t g, int t,
                                           f32x4 (&v)[kQChunks]) {
  const int64_t rem = numel - g * kGroupElems;
  const int bytes = rem <= 0 ? 0 : (rem >= kGroupElems ? kGroupElems * 4 : static_cast<int>(rem) * 4);
  const float* gp = rem > 0 ? w + g * kGroupElems : w;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(gp), 0, bytes,
                                                                      kBufferWord3);
#pragma unroll
  for (int i = 0; i < kQChunks; ++i)
    v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (i * kQThreads + t) * 16, 0,
                                                                           kStreamOnce));
}

// kDQ = false: no double quantization; absmax_q and scale are unused and
// the exact fp32 block absmax goes to absmax[numel/64] (4.5 bits per weight).
template <bool kDQ>
__global__ __launch_bounds__(kQThreads) void k_nf4_quantize(const float* __restrict__ w, int64_t numel,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ absmax_q,
                                                            float* __restrict__ scale,
                                                            float* __restrict__ absmax) {
  __shared__ uint32_t wave_max[2][kQWaves];  // by group parity: a fast wave may start the next group
  __shared__ uint2 s_bucket[kBuckets];
  // per wave: its blocks' absmax values, then their reciprocals; block
  // (chunk i, lane group q) at slot q * kQChunks + i
  __shared__ __attribute__((aligned(16))) float s_blk[kQWaves][kQBlocksPerWave];
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int64_t groups = (numel + kGroupElems - 1) / kGroupElems;
  const int64_t full_groups = numel / kGroupElems;
  const int64_t stride = gridDim.x;

  f32x4 v[kQChunks], vn[kQChunks];
  int64_t g = blockIdx.x;
  load_group(w, numel, g, t, v);
  if (t < 2 * kBuckets) reinterpret_cast<uint32_t*>(s_bucket)[t] = kBucketTableDev.word[t];
  __syncthreads();

  for (int par = 0; g < groups; g += stride, par ^= 1) {
    load_group(w, numel, g + stride, t, vn);  // the next group, in flight during this one
    const int64_t base = g * kGroupElems;
    const bool full = g < full_groups;  // every chunk in range (all groups but a ragged last)

    // Q1: block absmax (exact max of |w|), replicated over the block's 16 lanes
    float am[kQChunks];
    uint32_t tmax = 0;
#pragma unroll
    for (int i = 0; i < kQChunks; ++i) {
      uint32_t m = max(max(abs_bits(v[i].x), abs_bits(v[i].y)), max(abs_bits(v[i].z), abs_bits(v[i].w)));
      m = dpp_max_u32<kDppQuadXor1>(m);
      m = dpp_max_u32<kDppQuadXor2>(m);
      m = dpp_max_u32<kDppRowHalfMirror>(m);
      m = dpp_max_u32<kDppRowMirror>(m);
      am[i] = __builtin_bit_cast(float, m);
      tmax = max(tmax, m);
    }
    if ((lane & 15) == 0)
      *reinterpret_cast<f32x4*>(&s_blk[wv][(lane >> 4) * kQChunks]) = f32x4{am[0], am[1], am[2], am[3]};
    wave_lds_sync();
    // lane l < 16 owns slot l: chunk i = l % 4 of lane group l / 4, block
    // i * (kQThreads / 16) + 4 wv + l / 4 of the group (lanes >= 16 repeat it)
    const int slot = lane % kQBlocksPerWave;
    const float a_own = s_blk[wv][slot];
    const int own_blk = (slot % kQChunks) * (kQThreads / 16) + 4 * wv + slot / kQChunks;
    const bool own_valid = lane < kQBlocksPerWave && base + static_cast<int64_t>(own_blk) * kBlock < numel;
    const bool own_fast = a_own >= kFastAbsmaxMin && a_own <= kFastAbsmaxMax;
    const float y_own = 1.0f / (a_own * 0.0625f);
    wave_lds_sync();  // every lane has read its a_own before the reciprocals overwrite them
    if (lane < kQBlocksPerWave) s_blk[wv][slot] = y_own;
    if constexpr (!kDQ) {
      if (own_valid) absmax[(base >> 6) + own_blk] = a_own;
    }
    // the reciprocal path for the whole wave when it covers all its blocks
    const bool wave_fast = full && __builtin_amdgcn_ballot_w64(!own_fast) == 0;
    wave_lds_sync();
    const f32x4 y4 = *reinterpret_cast<const f32x4*>(&s_blk[wv][(lane >> 4) * kQChunks]);
    wave_lds_sync();  // read before the next group's absmax values overwrite them

    // Q3 + Q4: the code of x = fl32(w / a) = #{j : x > t_j}, taken as the
    // bucket lookup on X = 16 x, X from the block reciprocal with the exact
    // correction (both in nf4_format.hpp).  A zero block has X = 0 (code 7).
    // X stays within [-16, 16] (or is NaN, which converts to bucket 16), so
    // the bucket index is in 0..32.  4 codes -> 16 bits per chunk.
    uint16_t* const code_t = reinterpret_cast<uint16_t*>(codes + (base >> 1)) + t;  // chunk i at [i * kQThreads]
    if (wave_fast) {
#pragma unroll
      for (int i = 0; i < kQChunks; ++i) {
        const float b = am[i] * 0.0625f, y = y4[i];
        const float X[4] = {div_by_reciprocal(v[i].x, b, y), div_by_reciprocal(v[i].y, b, y),
                            div_by_reciprocal(v[i].z, b, y), div_by_reciprocal(v[i].w, b, y)};
        code_t[i * kQThreads] = static_cast<uint16_t>(bucket_codes(s_bucket, X));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kQChunks; ++i) {
        if (base + static_cast<int64_t>(i * kQThreads + t) * 4 < numel) {
          const float a = am[i];
          float X[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          if (a >= kFastAbsmaxMin && a <= kFastAbsmaxMax) {
            const float b = a * 0.0625f, y = y4[i];
#pragma unroll
            for (int k = 0; k < 4; ++k) X[k] = div_by_reciprocal(X[k], b, y);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) X[k] = a > 0.f ? (X[k] / a) * 16.0f : 0.f;
          }
          code_t[i * kQThreads] = static_cast<uint16_t>(bucket_codes(s_bucket, X));
        }
      }
    }

    if constexpr (kDQ) {
      // group scale s_g = max over the 256 blocks
      tmax = max(tmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(tmax), 16)));
      tmax = max(tmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(tmax), 32)));
      if (lane == 0) wave_max[par][wv] = tmax;
      __syncthreads();
      uint32_t gm = 0;
#pragma unroll
      for (int k = 0; k < kQWaves; ++k) gm = max(gm, wave_max[par][k]);
      const float sg = __builtin_bit_cast(float, gm);
      // Q2: 8-bit absmax codes, q = rne(fl32(fl32(a / s) * 255)); zero group -> 0
      if (own_valid) {
        uint32_t q = 0;
        if (sg > 0.f) {
          const float ratio = a_own / sg;
          const float scaled = ratio * 255.0f;
          q = static_cast<uint32_t>(__builtin_rintf(scaled));
        }
        absmax_q[(base >> 6) + own_blk] = static_cast<uint8_t>(q);
      }
      if (t == 0) scale[g] = sg;
    }
#pragma unroll
    for (int i = 0; i < kQChunks; ++i) v[i] = vn[i];
  }
}

// one workgroup per CU (fewer for small tensors)
static uint32_t quantize_grid(int64_t numel) {
  const int64_t groups = ceil_div(numel, kGroupElems);
  const int cus = device_cus();
  const int64_t g = cus > 0 && groups > cus ? cus : groups;
  return static_cast<uint32_t>(g);
}

hipError_t launch_nf4_quantize(const float* w, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                               float* scale, hipStream_t s) {
  hipLaunchKernelGGL(k_nf4_quantize<true>, dim3(quantize_grid(numel)), dim3(kQThreads), 0, s, w, numel, codes,
                     absmax_q, scale, nullptr);
  return hipGetLastError();
}

hipError_t launch_nf4_quantize_nodq(const float* w, int64_t numel, uint8_t* codes, float* absmax,
                                    hipStream_t s) {
  hipLaunchKernelGGL(k_nf4_quantize<false>, dim3(quantize_grid(numel)), dim3(kQThreads), 0, s, w, numel, codes,
                     nullptr, nullptr, absmax);
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
// kDQ = false: the 4.5-bit format, a_hat = scale[blk] (the fp32 block absmax)
template <bool kDQ>
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
  const Nf4Table tab = make_table(kDQ ? dq_absmax(absmax_q[blk], scale[blk >> 8]) : scale[blk]);
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
                                            uint16_t* out, int64_t ldo, hipStream_t s, bool absmax_fp32) {
  const int64_t tiles = (rows / 64) * (cols / 64);
  const dim3 grid(static_cast<uint32_t>(ceil_div(tiles, 4)));
  if (absmax_fp32)
    hipLaunchKernelGGL(k_nf4_dequantize_t<false>, grid, dim3(256), 0, s, codes, nullptr, scale, rows, cols, out,
                       ldo);
  else
    hipLaunchKernelGGL(k_nf4_dequantize_t<true>, grid, dim3(256), 0, s, codes, absmax_q, scale, rows, cols, out,
                       ldo);
  return hipGetLastError();
}

}  // namespace qlora
