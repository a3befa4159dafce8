// k_merge.hip -- folds the adapter into the frozen weight for serving:
//   W_merged = bf16(W_hat + (alpha/r) B A)        [out, in]
// (coddykit "LoRA y QLoRA", merging the adapter into the base with
// merge_and_unload; ultralytics glossary "QLoRA", "Compromissos": the 4-bit
// base has to be dequantized to 16 bits before the merge).  Each element is
// rounded once: bf16_rne(fl32(w_hat + fl32(s * sum_j B[m][j] A[j][n]))), the
// rank-r sum accumulated in fp32 by MFMA.
//
// One workgroup per 64 rows (out) x 256 columns (in).  Four waves compute
// the rank-r product of the tile with v_mfma_f32_32x32x16_bf16 (B rows and
// A^T rows are K-contiguous after zero-padding r to rp, both small and
// L2-resident) and park it, scaled, in LDS; then each thread owns one
// 64-weight block of the tile: it loads the block's 32 code bytes and
// absmax, expands them with the block's v_perm table (bit-identical to
// nf4_dequantize) and adds the rank-r term; the tile then leaves through LDS
// in whole row segments.
// Bound by the HBM stream (0.5 B read + 2 B written per weight).
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {
constexpr int kMRows = 64, kMCols = 256, kMPitch = kMCols + 4;
constexpr int kMBufWord3 = 0x00020000;
__device__ __forceinline__ bf16x8 m_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
}  // namespace

__global__ __launch_bounds__(256) void k_merge(const uint8_t* __restrict__ codes,
                                               const uint8_t* __restrict__ absmax_q,
                                               const float* __restrict__ scale, int64_t in,
                                               const uint16_t* __restrict__ Bp,
                                               const uint16_t* __restrict__ Atp, int64_t ldp, int rp,
                                               float s, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float s_c[kMRows * kMPitch];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kMCols;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kMRows;

  // rank-r product of the tile: wave wv takes columns n0 + 64 wv .. + 64
  // (rows of A^T past `in` read as zero)
  const uint64_t at_bytes = static_cast<uint64_t>(in > n0 ? in - n0 : 0) * ldp * 2;
  const __amdgpu_buffer_rsrc_t rs_at = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Atp + n0 * ldp), 0,
      static_cast<int>(at_bytes < 0x7fffffffu ? at_bytes : 0x7fffffffu), kMBufWord3);
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.f;
#pragma unroll 4
  for (int k0 = 0; k0 < rp; k0 += 16) {
    bf16x8 fa[2], fb[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint32_t off = static_cast<uint32_t>(((64 * wv + 32 * a + r32) * ldp + k0 + 8 * half) * 2);
      fa[a] = m_as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_at, off, 0, 0)));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
      fb[c] = m_as_bf16x8(*reinterpret_cast<const u32x4*>(Bp + (m0 + 32 * c + r32) * ldp + k0 + 8 * half));
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[c], acc[a][c], 0, 0, 0);
  }
  // D[n][m]: lane holds m = 32 c + r32, n = 64 wv + 32 a + 8 (e/4) + 4 half + e%4
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = 64 * wv + 32 * a + 8 * (e >> 2) + 4 * half + (e & 3);
        s_c[(32 * c + r32) * kMPitch + n] = __fmul_rn(s, acc[a][c][e]);
      }
  __syncthreads();

  // thread -> row m0 + tid / 4, block (n0 + 64 (tid % 4)) of 64 weights
  const int ml = tid >> 2, nl = 64 * (tid & 3);
  const int64_t col = n0 + nl;
  const bool live = col < in;
  u32x4 ov[8];
  if (live) {
    const int64_t e0 = (m0 + ml) * in + col;  // first element of the block
    const int64_t blk = e0 >> 6;
    const Nf4Table tab = make_table(dq_absmax(absmax_q[blk], scale[blk >> 8]));
    const u32x4* src = reinterpret_cast<const u32x4*>(codes + (e0 >> 1));
    const float* lr = s_c + ml * kMPitch + nl;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 cw = src[h];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t w[4];
        lookup8(tab, cw[k], w);
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int j = 32 * h + 8 * k + 2 * p;
          o[p] = pack_bf16x2(bf16_lo(w[p]) + lr[j], bf16_hi(w[p]) + lr[j + 1]);
        }
        ov[4 * h + k] = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
  }
  // The results go out through LDS (reusing s_c, 33 pieces of 16 B per row)
  // so that each store instruction writes whole 512-byte row segments; a
  // thread's own 128 bytes written directly would put 64 separate 16-byte
  // pieces into every store instruction.
  __syncthreads();  // every thread is done reading s_c
  u32x4* s_o = reinterpret_cast<u32x4*>(s_c);
  if (live) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_o[ml * 33 + (nl >> 3) + j] = ov[j];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int P = 256 * i + tid, rl = P >> 5, pc = P & 31;
    const int64_t cp = n0 + 8 * pc;
    if (cp < in) *reinterpret_cast<u32x4*>(out + (m0 + rl) * in + cp) = s_o[rl * 33 + pc];
  }
}

hipError_t launch_merge(const uint8_t* codes, const uint8_t* absmax_q, const float* scale,
                        int64_t out, int64_t in, const uint16_t* Bp, const uint16_t* Atp,
                        int64_t ldp, int64_t rp, float s, uint16_t* w_out, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>(ceil_div(in, kMCols)), static_cast<uint32_t>(out / kMRows));
  hipLaunchKernelGGL(k_merge, grid, dim3(256), 0, st, codes, absmax_q, scale, in, Bp, Atp, ldp,
                     static_cast<int>(rp), s, w_out);
  return hipGetLastError();
}

}  // namespace qlora
