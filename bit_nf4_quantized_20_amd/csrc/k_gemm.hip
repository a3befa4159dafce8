// k_gemm.hip -- bf16 MFMA GEMM for gfx950 with fp32 accumulation and one
// rounding to bf16 at the end:
//   C[M][N] = sum_k act0[m][k] wt0[n][k]  +  sum_k act1[m][k] wt1[n][k]
// The main segment's weight operand is either a bf16 matrix or an NF4 weight
// (codes + double-quantized absmax) that is dequantized while it is staged
// into LDS: each thread turns 32 packed codes of one block into bf16 with the
// block's v_perm table and writes them straight into the swizzled LDS tile,
// so W_hat never exists in HBM (ultralytics glossary "QLoRA": the frozen
// weight is dequantized to bfloat16 right before the matmul; paperclase
// lesson "QLoRA", Parte 4: W_hat is built, used and discarded).
// The second segment carries the LoRA term as extra K-steps (act1 = s*U or
// s*V as a bf16 hi/lo pair, wt1 = B or A^T padded to match), so base and
// adapter products share one fp32 accumulator and Y / dX are rounded once.
//
// Tile BM x BN, K-step 64 (whole 128-byte lines per tile row: half-line
// steps measured markedly slower), two LDS stages and two register stages:
// the tiles of step st + 3 are loaded into registers while step st is
// computed and written into LDS two steps later, so ~128 KB of loads are in
// flight per CU (the loads are latency bound; ordinary loads into registers
// measured faster here than copies straight into LDS).  One barrier per
// K-step.  v_mfma_f32_32x32x16_bf16; the MFMA A operand is the weight tile
// (rows n), its B operand the activation tile (rows m), so each lane ends up
// holding 4 consecutive n of one output row m and stores them as one 8-byte
// write.
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

constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource, 32-bit data format
constexpr int kStream = 2;                // cache policy nt: streamed once

// A buffer resource for rows [row0, nrows) of a row-major matrix (ld
// elements per row, elem_bytes each): loads past the last row return zeros
// without a branch.  The size is capped at 2^31 - 1 bytes; a tile's own rows
// start at offset 0, so only rows far past the tile could fall beyond it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t ld, int64_t row0,
                                                            int64_t nrows, int elem_bytes) {
  const uint64_t bytes = static_cast<uint64_t>(nrows > row0 ? nrows - row0 : 0) * ld * elem_bytes;
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(base) + row0 * ld * elem_bytes), 0,
      static_cast<int>(bytes < 0x7fffffffu ? bytes : 0x7fffffffu), kBufferWord3);
}

// bf16 tile rows [ROWS][64] of a K-contiguous matrix, through registers by NT
// threads: per-lane row offsets are fixed, the K offset is scalar.
template <int ROWS, int NT>
struct Bf16Tile {
  static constexpr int kPer = ROWS * 8 / NT;  // 16-byte chunks per thread
  typedef u32x4 Regs[kPer];
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[kPer];

  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int64_t row0, int64_t nrows, int tid) {
    rs = rows_rsrc(base, ld, row0, nrows, 2);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int id = tid + NT * i;
      voff[i] = static_cast<uint32_t>(((id >> 3) * ld + (id & 7) * 8) * 2);
    }
  }
  __device__ __forceinline__ void load(Regs& v, int64_t k0) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], static_cast<int>(k0 * 2), 0));
  }
  __device__ __forceinline__ static void store(const Regs& v, uint16_t* lds, int tid) {
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
struct Nf4Tile {
  static constexpr int kTPR = NT / ROWS;  // threads per row
  static constexpr int kDw = 8 / kTPR;    // code dwords (8 weights each) per thread
  static_assert(kTPR == 2 || kTPR == 4, "unsupported tile");
  struct Regs {
    uint32_t cw[kDw];
    uint32_t q;
    float sg;
  };
  __amdgpu_buffer_rsrc_t rc, rq;
  const float* scale;
  int64_t blk0;        // first block of this thread's row
  uint32_t coff, qoff;

  __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* absmax_q, const float* sc,
                                       int64_t in, int64_t row0, int64_t nrows, int tid) {
    const int row = tid / kTPR, part = tid % kTPR;
    rc = rows_rsrc(codes, in / 2, row0, nrows, 1);
    rq = rows_rsrc(absmax_q, in / 64, row0, nrows, 1);
    scale = sc;
    coff = static_cast<uint32_t>(row * (in / 2) + part * kDw * 4);
    qoff = static_cast<uint32_t>(row * (in / 64));
    int64_t g = row0 + row;
    if (g >= nrows) g = nrows - 1;  // its scale read stays in range (codes read as zero)
    blk0 = g * (in / 64);
  }
  __device__ __forceinline__ void load(Regs& r, int64_t k0) const {
    if constexpr (kDw == 4) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff, static_cast<int>(k0 / 2), kStream));
      r.cw[0] = v[0]; r.cw[1] = v[1]; r.cw[2] = v[2]; r.cw[3] = v[3];
    } else {
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, coff, static_cast<int>(k0 / 2), kStream));
      r.cw[0] = v[0]; r.cw[1] = v[1];
    }
    r.q = __builtin_amdgcn_raw_buffer_load_b8(rq, qoff, static_cast<int>(k0 / 64), 0);
    r.sg = scale[(blk0 + k0 / 64) >> 8];
  }
  __device__ __forceinline__ static void store(const Regs& r, uint16_t* lds, int tid) {
    const int row = tid / kTPR, part = tid % kTPR;
    const Nf4Table tab = make_table(dq_absmax(r.q, r.sg));
#pragma unroll
    for (int d = 0; d < kDw; ++d) {
      uint32_t o[4];
      lookup8(tab, r.cw[d], o);
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

// WAVES_M x WAVES_N waves; each computes a (BM/WAVES_M) x (BN/WAVES_N) sub-tile.
//
// Step st: barrier (LDS stage st % 2 complete; stage (st + 1) % 2 free), write
// step st + 1's tiles from register set (st + 1) % 2 into LDS (NF4 weights
// are dequantized here), load step st + 3's tiles into that register set,
// compute step st.  The main and LoRA segments run this pipeline one after
// the other, each with register sets of its own operand types.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kNf4>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm(GemmArgs p) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, FM = WM / 32, FN = WN / 32;
  __shared__ __attribute__((aligned(16))) uint16_t s_act[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_wt[2][BN * kBK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % WAVES_M, wn = wv / WAVES_M;
  // NF4: waves 4-7 (sharing SIMDs with waves 0-3) dequantize after computing
  const bool late = kNf4 && wv >= 4;
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

  auto compute = [&](int b) {
    const uint16_t* sa = s_act[b];
    const uint16_t* sw = s_wt[b];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int chunk = 2 * j + half;
      bf16x8 fw[FN], fa[FM];
#pragma unroll
      for (int a = 0; a < FN; ++a) fw[a] = lds_frag(sw, wn * WN + a * 32 + r32, chunk);
#pragma unroll
      for (int c = 0; c < FM; ++c) fa[c] = lds_frag(sa, wm * WM + c * 32 + r32, chunk);
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int c = 0; c < FM; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[a], fa[c], acc[a][c], 0, 0, 0);
    }
  };

  // One K segment [first, last) of global steps; the LDS stage of step st is
  // st % 2 throughout.  Two register sets by step parity; Regs::fetch(r, e)
  // loads segment-relative step e, Regs::stash(r, b) writes stage b.
  auto segment = [&](auto& r0, auto& r1, int64_t first, int64_t last, auto fetch, auto stash) {
    const int64_t n = last - first;
    if (n <= 0) return;
    fetch(r0, 0);
    if (n > 1) fetch(r1, 1);
    stash(r0, static_cast<int>(first & 1));
    if (n > 2) fetch(r0, 2);
    // with an NF4 weight, waves 0-3 write and load before computing and waves
    // 4-7 after: the two waves sharing a SIMD then alternate MFMAs with the
    // dequantization's vector-ALU work instead of doing both at once (for a
    // bf16 weight the fixed order measured slightly faster)
    auto step = [&](int64_t e, auto& nxt) {  // nxt holds step e + 1
      __syncthreads();
      if (!late) {
        if (e + 1 < n) stash(nxt, static_cast<int>((first + e + 1) & 1));
        if (e + 3 < n) fetch(nxt, e + 3);
      }
      compute(static_cast<int>((first + e) & 1));
      if (late) {
        if (e + 1 < n) stash(nxt, static_cast<int>((first + e + 1) & 1));
        if (e + 3 < n) fetch(nxt, e + 3);
      }
    };
    for (int64_t e = 0; e < n; e += 2) {
      step(e, r1);
      if (e + 1 < n) step(e + 1, r0);
    }
  };

  const int64_t s0 = p.K0 / kBK, s1 = p.K1 / kBK;
  using TA = Bf16Tile<BM, NT>;
  using TW = Bf16Tile<BN, NT>;
  if constexpr (kNf4) {
    using TQ = Nf4Tile<BN, NT>;
    TA ta;
    TQ tq;
    ta.init(p.act0, p.lda0, m0, p.M, tid);
    tq.init(p.codes, p.absmax_q, p.scale, p.K0, n0, p.N, tid);
    struct R { typename TA::Regs a; typename TQ::Regs w; };
    R r0, r1;
    segment(r0, r1, 0, s0,
            [&](R& r, int64_t e) {
              ta.load(r.a, e * kBK);
              tq.load(r.w, e * kBK);
            },
            [&](const R& r, int b) {
              TA::store(r.a, s_act[b], tid);
              TQ::store(r.w, s_wt[b], tid);
            });
  } else {
    TA ta;
    TW tw;
    ta.init(p.act0, p.lda0, m0, p.M, tid);
    tw.init(p.wt0, p.ldw0, n0, p.N, tid);
    struct R { typename TA::Regs a; typename TW::Regs w; };
    R r0, r1;
    segment(r0, r1, 0, s0,
            [&](R& r, int64_t e) {
              ta.load(r.a, e * kBK);
              tw.load(r.w, e * kBK);
            },
            [&](const R& r, int b) {
              TA::store(r.a, s_act[b], tid);
              TW::store(r.w, s_wt[b], tid);
            });
  }
  if (s1 > 0) {  // LoRA extension segment
    TA ta;
    TW tw;
    ta.init(p.act1, p.lda1, m0, p.M, tid);
    tw.init(p.wt1, p.ldw1, n0, p.N, tid);
    struct R { typename TA::Regs a; typename TW::Regs w; };
    R r0, r1;
    segment(r0, r1, s0, s0 + s1,
            [&](R& r, int64_t e) {
              ta.load(r.a, e * kBK);
              tw.load(r.w, e * kBK);
            },
            [&](const R& r, int b) {
              TA::store(r.a, s_act[b], tid);
              TW::store(r.w, s_wt[b], tid);
            });
  }

  // epilogue: D[n][m] -> C[m][n]; lane holds m = r32, n = 8*(e/4) + 4*half + e%4
#pragma unroll
  for (int c = 0; c < FM; ++c) {
    const int64_t m = m0 + wm * WM + c * 32 + r32;
    if (m >= p.M) continue;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * WN + a * 32 + 8 * g + 4 * half;
        if (n < p.N) {
          const uint32_t p0 = pack_bf16x2(acc[a][c][4 * g + 0], acc[a][c][4 * g + 1]);
          const uint32_t p1 = pack_bf16x2(acc[a][c][4 * g + 2], acc[a][c][4 * g + 3]);
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
