// k_gemm.hip -- bf16 MFMA GEMM for gfx950 with fp32 accumulation and one
// rounding to bf16 at the end:
//   C[M][N] = sum_k act0[m][k] wt0[n][k]  +  sum_k act1[m][k] wt1[n][k]
// The main segment's weight operand is either a bf16 matrix or an NF4 weight
// (codes + double-quantized absmax) that is dequantized while it is staged
// into LDS: each thread turns 32 or 64 packed codes of one block into bf16
// with the block's v_perm table and writes them straight into the swizzled
// LDS tile, so W_hat never exists in HBM (ultralytics glossary "QLoRA": the
// frozen weight is dequantized to bfloat16 right before the matmul;
// paperclase lesson "QLoRA", Parte 4: W_hat is built, used and discarded).
// The second segment carries the LoRA term as extra K-steps (act1 = s*U or
// s*V as a bf16 hi/lo pair, wt1 = B or A^T padded to match), so base and
// adapter products share one fp32 accumulator and Y / dX are rounded once.
//
// Tile: BM x BN per workgroup of 4 waves (2 x 2), K-step 64, operands staged
// through LDS with a 16-byte-chunk XOR swizzle, v_mfma_f32_32x32x16_bf16.
// The MFMA A operand is the weight tile (rows n), its B operand the
// activation tile (rows m), so each lane ends up holding 4 consecutive n of
// one output row m and stores them as one 8-byte write.
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {

constexpr int kBK = 64;

// 16-byte chunk swizzle of a 128-byte LDS row.  A fragment read has 32
// lanes on 32 consecutive rows at one chunk; the key (row & 7) ^ (row >> 3 & 1)
// gives every 8 consecutive rows distinct chunks (32-bank view) and every 16
// consecutive rows distinct (row parity, chunk) pairs (64-bank view), so the
// reads are conflict-free either way.  Writes cover whole rows, so any
// per-row permutation is conflict-free for them.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

// bf16 rows [ROWS][64] from a K-contiguous matrix, staged through registers
// by NT threads
template <int ROWS, int NT>
struct Bf16Loader {
  static constexpr int kPer = ROWS * 8 / NT;  // 16-byte chunks per thread
  u32x4 v[kPer];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int64_t row0,
                                       int64_t nrows, int64_t k0, int tid) {
    if (row0 + ROWS <= nrows) {  // whole tile in range (uniform): no per-row branches
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int id = tid + NT * i;
        const int row = id >> 3, q = id & 7;
        v[i] = *reinterpret_cast<const u32x4*>(src + (row0 + row) * ld + k0 + q * 8);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + NT * i;
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
      const int id = tid + NT * i;
      const int row = id >> 3, q = id & 7;
      *reinterpret_cast<u32x4*>(lds + row * kBK + swz(row, q) * 8) = v[i];
    }
  }
};

// NF4 rows [ROWS][64]: one 64-weight block per row per K-step.  NT/ROWS
// threads share a row; each loads its share of the 32 code bytes plus the
// block's 8-bit absmax and group scale, and expands them at store time.
template <int ROWS, int NT>
struct Nf4Loader {
  static constexpr int kTPR = NT / ROWS;   // threads per row
  static constexpr int kDw = 8 / kTPR;     // code dwords (8 weights each) per thread
  static_assert(kTPR == 1 || kTPR == 2 || kTPR == 4, "unsupported tile");
  uint32_t cw[kDw];
  uint32_t q;
  float sg;

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ absmax_q,
                                       const float* __restrict__ scale, int64_t in, int64_t row0,
                                       int64_t nrows, int64_t k0, int tid) {
    const int row = tid / kTPR, part = tid % kTPR;
    const int64_t grow = row0 + row;
    if (grow < nrows) {
      const int64_t e = grow * in + k0;  // first weight of the block
      const uint8_t* src = codes + (e >> 1) + part * kDw * 4;
      if constexpr (kDw >= 4) {
#pragma unroll
        for (int i = 0; i < kDw / 4; ++i) {
          const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i);
          cw[4 * i + 0] = v[0]; cw[4 * i + 1] = v[1]; cw[4 * i + 2] = v[2]; cw[4 * i + 3] = v[3];
        }
      } else {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
        cw[0] = v[0]; cw[1] = v[1];
      }
      const int64_t bi = e >> 6;
      q = absmax_q[bi];
      sg = scale[bi >> 8];
    } else {
#pragma unroll
      for (int i = 0; i < kDw; ++i) cw[i] = 0u;
      q = 0u;
      sg = 0.f;
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const int row = tid / kTPR, part = tid % kTPR;
    const Nf4Table tab = make_table(dq_absmax(q, sg));
#pragma unroll
    for (int d = 0; d < kDw; ++d) {
      uint32_t o[4];
      lookup8(tab, cw[d], o);
      const int chunk = part * kDw + d;
      *reinterpret_cast<u32x4*>(lds + row * kBK + swz(row, chunk) * 8) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
};

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* lds, int row, int chunk) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * kBK + swz(row, chunk) * 8);
  return __builtin_bit_cast(bf16x8, v);
}

// XCD-aware tile order.  Workgroups are dispatched round-robin over the 8
// XCDs (linear id % 8), and each XCD has its own L2.  The tiles are renumbered
// so that XCD x runs a contiguous stretch of the tile sequence, and the
// sequence walks groups of 8 M-tiles column by column, so the ~32 workgroups an
// XCD runs at once cover a compact block of C and share A and B panels in
// that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;
__device__ __forceinline__ void xcd_tile(int64_t gm, int64_t gn, int64_t& mt, int64_t& nt) {
  const int64_t total = gm * gn;
  const int64_t lin = static_cast<int64_t>(blockIdx.y) * gm + blockIdx.x;
  int64_t t = lin;
  if (total % kXcds == 0) t = (lin % kXcds) * (total / kXcds) + lin / kXcds;
  const int64_t per_group = kGroupM * gn;
  const int64_t g = t / per_group;
  const int64_t gm_g = (gm - g * kGroupM) < kGroupM ? (gm - g * kGroupM) : kGroupM;
  const int64_t in_g = t - g * per_group;
  mt = g * kGroupM + in_g % gm_g;
  nt = in_g / gm_g;
}

struct GemmArgs {
  int64_t M, N;
  // main segment activation and weight (bf16 weight, or NF4 when codes != nullptr)
  const uint16_t* act0; int64_t lda0;
  const uint16_t* wt0; int64_t ldw0;
  const uint8_t* codes; const uint8_t* absmax_q; const float* scale;
  int64_t K0;
  // LoRA extension segment
  const uint16_t* act1; int64_t lda1;
  const uint16_t* wt1; int64_t ldw1;
  int64_t K1;
  uint16_t* C; int64_t ldc;
};

}  // namespace

// WAVES_M x WAVES_N waves; each wave computes a (BM/WAVES_M) x (BN/WAVES_N)
// sub-tile.  With 8 waves two share each SIMD, so one wave's loads and LDS
// traffic overlap the other's MFMAs.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kNf4>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm(GemmArgs p) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, FM = WM / 32, FN = WN / 32;
  // two LDS stages: while the waves compute on one, the next tile is written
  // into the other, so each K-step needs a single barrier
  __shared__ __attribute__((aligned(16))) uint16_t s_act[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_wt[2][BN * kBK];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv % WAVES_M, wn = wv / WAVES_M;
  int64_t mt, nt;
  xcd_tile(gridDim.x, gridDim.y, mt, nt);
  const int64_t m0 = mt * BM;
  const int64_t n0 = nt * BN;
  const int r32 = lane & 31, half = lane >> 5;

  f32x16 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int64_t s0 = p.K0 / kBK, steps = s0 + p.K1 / kBK;
  Bf16Loader<BM, NT> la;
  Bf16Loader<BN, NT> lw;
  Nf4Loader<BN, NT> lq;
  auto fetch = [&](int64_t st) {
    if (st < s0) {
      la.load(p.act0, p.lda0, m0, p.M, st * kBK, tid);
      if constexpr (kNf4)
        lq.load(p.codes, p.absmax_q, p.scale, p.K0, n0, p.N, st * kBK, tid);
      else
        lw.load(p.wt0, p.ldw0, n0, p.N, st * kBK, tid);
    } else {
      la.load(p.act1, p.lda1, m0, p.M, (st - s0) * kBK, tid);
      lw.load(p.wt1, p.ldw1, n0, p.N, (st - s0) * kBK, tid);
    }
  };
  auto stash = [&](int64_t st, int buf) {
    la.store(s_act[buf], tid);
    if constexpr (kNf4) {
      if (st < s0) { lq.store(s_wt[buf], tid); return; }
    }
    lw.store(s_wt[buf], tid);
  };

  if (steps > 0) {
    fetch(0);
    stash(0, 0);
    if (steps > 1) fetch(1);
  }
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = static_cast<int>(st & 1);
    __syncthreads();  // stage buf complete; stage buf^1 free
    if (st + 1 < steps) {
      stash(st + 1, buf ^ 1);
      if (st + 2 < steps) fetch(st + 2);
    }
    const uint16_t* sa = s_act[buf];
    const uint16_t* sw = s_wt[buf];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int chunk = 2 * j + half;
      bf16x8 fw[FN], fa[FM];
#pragma unroll
      for (int a = 0; a < FN; ++a) fw[a] = lds_frag(sw, wn * WN + a * 32 + r32, chunk);
#pragma unroll
      for (int b = 0; b < FM; ++b) fa[b] = lds_frag(sa, wm * WM + b * 32 + r32, chunk);
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
    if (m >= p.M) continue;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * WN + a * 32 + 8 * g + 4 * half;
        if (n < p.N) {
          const uint32_t p0 = pack_bf16x2(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1]);
          const uint32_t p1 = pack_bf16x2(acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]);
          *reinterpret_cast<u32x2*>(p.C + m * p.ldc + n) = u32x2{p0, p1};
        }
      }
    }
  }
}

namespace {
template <bool kNf4>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t s) {
  // 256 x 256 tiles (8 waves) when they give at least one full wave of
  // workgroups, else 128 x 128 (4 waves)
  const int64_t big = ceil_div(a.M, 256) * ceil_div(a.N, 256);
  if (big >= 256) {
    dim3 grid(static_cast<uint32_t>(ceil_div(a.M, 256)), static_cast<uint32_t>(ceil_div(a.N, 256)));
    hipLaunchKernelGGL((k_gemm<256, 256, 2, 4, kNf4>), grid, dim3(512), 0, s, a);
  } else {
    dim3 grid(static_cast<uint32_t>(ceil_div(a.M, 128)), static_cast<uint32_t>(ceil_div(a.N, 128)));
    hipLaunchKernelGGL((k_gemm<128, 128, 2, 2, kNf4>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_nt(int64_t M, int64_t N, const uint16_t* act0, int64_t lda0,
                          const uint16_t* wt0, int64_t ldw0, int64_t K0, const uint16_t* act1,
                          int64_t lda1, const uint16_t* wt1, int64_t ldw1, int64_t K1, uint16_t* C,
                          int64_t ldc, hipStream_t s) {
  GemmArgs a{M, N, act0, lda0, wt0, ldw0, nullptr, nullptr, nullptr, K0,
             act1, lda1, wt1, ldw1, K1, C, ldc};
  return launch_tiles<false>(a, s);
}

hipError_t launch_gemm_nf4(int64_t M, int64_t N, const uint16_t* act0, int64_t lda0,
                           const uint8_t* codes, const uint8_t* absmax_q, const float* scale,
                           int64_t K0, const uint16_t* act1, int64_t lda1, const uint16_t* wt1,
                           int64_t ldw1, int64_t K1, uint16_t* C, int64_t ldc, hipStream_t s) {
  GemmArgs a{M, N, act0, lda0, nullptr, 0, codes, absmax_q, scale, K0,
             act1, lda1, wt1, ldw1, K1, C, ldc};
  return launch_tiles<true>(a, s);
}

}  // namespace qlora
