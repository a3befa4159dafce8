// k_gemm.hip -- bf16 MFMA GEMM for gfx950 with fp32 accumulation and one
// rounding to bf16 at the end:
//   C[M][N] = sum_k act0[m][k] wt0[n][k]  +  sum_k act1[m][k] wt1[n][k]
// The second segment carries the LoRA term as extra K-steps (act1 = s*U or
// s*V zero-padded to a multiple of 64 ranks, wt1 = B or A^T padded the same
// way), so the base product and the adapter product share one accumulator
// and Y / dX are rounded once (paperclase lesson "QLoRA", Parte 4: the layer
// adds the scaled adapter output to the linear output).
//
// Tile: BM x BN per workgroup of 4 waves (2 x 2), K-step 64, operands staged
// through LDS with a 16-byte-chunk XOR swizzle, v_mfma_f32_32x32x16_bf16.
// The MFMA's A operand is the weight tile (rows n), its B operand the
// activation tile (rows m), so each lane ends up holding 4 consecutive n of
// one output row m and stores them as one 8-byte write.
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {

constexpr int kBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row & 7)); }

template <int ROWS>
struct TileLoader {
  // ROWS x 64 bf16 = ROWS*8 chunks of 16 B, spread over 256 threads
  static constexpr int kPer = ROWS * 8 / 256;
  u32x4 v[kPer];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int64_t row0,
                                       int64_t nrows, int64_t k0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3, q = id & 7;
      if (row0 + row < nrows)
        v[i] = *reinterpret_cast<const u32x4*>(src + (row0 + row) * ld + k0 + q * 8);
      else
        v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3, q = id & 7;
      *reinterpret_cast<u32x4*>(lds + row * kBK + swz(row, q) * 8) = v[i];
    }
  }
};

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* lds, int row, int chunk) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * kBK + swz(row, chunk) * 8);
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace

template <int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_nt(int64_t M, int64_t N, const uint16_t* __restrict__ act0,
                                                 int64_t lda0, const uint16_t* __restrict__ wt0,
                                                 int64_t ldw0, int64_t K0,
                                                 const uint16_t* __restrict__ act1, int64_t lda1,
                                                 const uint16_t* __restrict__ wt1, int64_t ldw1,
                                                 int64_t K1, uint16_t* __restrict__ C, int64_t ldc) {
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  __shared__ __attribute__((aligned(16))) uint16_t s_act[BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_wt[BN * kBK];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int r32 = lane & 31, half = lane >> 5;

  f32x16 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int64_t s0 = K0 / kBK, steps = s0 + K1 / kBK;
  TileLoader<BM> la;
  TileLoader<BN> lw;
  auto fetch = [&](int64_t st) {
    if (st < s0) {
      la.load(act0, lda0, m0, M, st * kBK, tid);
      lw.load(wt0, ldw0, n0, N, st * kBK, tid);
    } else {
      la.load(act1, lda1, m0, M, (st - s0) * kBK, tid);
      lw.load(wt1, ldw1, n0, N, (st - s0) * kBK, tid);
    }
  };

  if (steps > 0) fetch(0);
  for (int64_t st = 0; st < steps; ++st) {
    __syncthreads();
    la.store(s_act, tid);
    lw.store(s_wt, tid);
    __syncthreads();
    if (st + 1 < steps) fetch(st + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int chunk = 2 * j + half;
      bf16x8 fw[FN], fa[FM];
#pragma unroll
      for (int a = 0; a < FN; ++a) fw[a] = lds_frag(s_wt, wn * WN + a * 32 + r32, chunk);
#pragma unroll
      for (int b = 0; b < FM; ++b) fa[b] = lds_frag(s_act, wm * WM + b * 32 + r32, chunk);
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[a], fa[b], acc[a][b], 0, 0, 0);
    }
  }

  // epilogue: D[n][m] -> C[m][n]; lane holds m = r32, n = 8*(e/4) + 4*half + e%4
#pragma unroll
  for (int b = 0; b < FM; ++b) {
    const int64_t m = m0 + wm * WM + b * 32 + r32;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * WN + a * 32 + 8 * g + 4 * half;
        if (n < N) {
          const uint32_t p0 = pack_bf16x2(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1]);
          const uint32_t p1 = pack_bf16x2(acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]);
          *reinterpret_cast<u32x2*>(C + m * ldc + n) = u32x2{p0, p1};
        }
      }
    }
  }
}

hipError_t launch_gemm_nt(int64_t M, int64_t N, const uint16_t* act0, int64_t lda0,
                          const uint16_t* wt0, int64_t ldw0, int64_t K0, const uint16_t* act1,
                          int64_t lda1, const uint16_t* wt1, int64_t ldw1, int64_t K1, uint16_t* C,
                          int64_t ldc, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  dim3 grid(static_cast<uint32_t>(ceil_div(M, BM)), static_cast<uint32_t>(ceil_div(N, BN)));
  hipLaunchKernelGGL((k_gemm_nt<BM, BN>), grid, dim3(256), 0, s, M, N, act0, lda0, wt0, ldw0, K0,
                     act1, lda1, wt1, ldw1, K1, C, ldc);
  return hipGetLastError();
}

}  // namespace qlora
