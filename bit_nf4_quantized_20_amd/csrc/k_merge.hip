// k_merge.hip -- folds the adapter into the frozen weight for serving:
//   W_merged = bf16(W_hat + (alpha/r) B A)        [out, in]
// (coddykit "LoRA y QLoRA", merging the adapter into the base with
// merge_and_unload; ultralytics glossary "QLoRA", "Compromissos": the 4-bit
// base has to be dequantized to 16 bits before the merge).  Each element is
// bf16_rne(fma(s, sum_j B[m][j] A[j][n], w_hat)): the rank-r sum accumulated
// in fp32 by MFMA, scaled and added to the dequantized weight with one fp32
// rounding, then rounded once to bf16.
//
// Tiles of 64 rows (out) x 256 columns (in); wave wv owns tile columns
// 64 wv .. + 64, i.e. one 64-weight block of each of the 64 rows.  The wave
// forms the rank-r product of its 64 x 64 piece with v_mfma_f32_32x32x16_bf16
// (B rows and A^T rows are K-contiguous after zero-padding r to rp) and keeps
// it in the MFMA registers: lane l holds rows 32 c + l % 32 (c = 0, 1) and,
// of each group of 8 columns, the four at 4 (l / 32) .. + 3.  It dequantizes
// exactly those weights from the row's codes (4 codes per v_perm lookup with
// the block's table, bit-identical to nf4_dequantize), adds the scaled
// product and rounds; the bf16 tile leaves through LDS in whole row segments.
//
// The workgroups are persistent: workgroup j takes column strip
// j % strips and walks the strip's row tiles j / strips, + G / strips, ...
// (G workgroups, a multiple of the strip count).  Its A^T fragments stay in
// registers for the whole walk (rp = 64, i.e. r <= 64).  The tile's B rows
// (64 x 128 bytes) and codes (64 x 128 bytes) are fetched once per workgroup
// with whole-line loads into LDS -- the next tile's while this one is
// computed -- and the waves read their fragments and blocks from there.
// Bound by the HBM stream (0.5 B read + 2 B written per weight).
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {
constexpr int kMRows = 64, kMCols = 256;
constexpr int kMPitch = kMCols / 2 + 2;  // dwords per output row in LDS: 2 padding dwords keep the 8-byte writes conflict-free
constexpr int kMBufWord3 = 0x00020000;
constexpr uint32_t kMPastEnd = 0x80000000u;  // past every buffer (all < 2^31 bytes): reads zero
constexpr int kMWgPerCu = 2;
constexpr int kMRowBytes = 128;  // a staged row: 64 bf16 of B (rp = 64), or 256 codes
__device__ __forceinline__ bf16x8 m_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 4 codes -> their 4 dequantized weights as fp32, from the block's table.
// z holds the code bytes b0 (codes 0, 1) in bytes 0 and 1 and b1 (codes 2,
// 3) in bytes 2 and 3; code k ends up in the low nibble of byte k of idx
// (the high nibbles are ignored by both selectors).  The bf16 table entries
// widen to fp32 by placing their two bytes over two zero bytes (v_perm
// selector 0x0C gives 0x00).
__device__ __forceinline__ void lookup4_f32(const Nf4Table& t, uint32_t z, float (&w)[4]) {
  const uint32_t idx = (z & 0x00FF00FFu) | ((z >> 4) & 0xFF00FF00u);
  const uint32_t sel = idx & 0x07070707u;
  const uint32_t pick = __builtin_amdgcn_bitop3_b32(idx >> 1, 0x04040404u, 0x03020100u, 0xEA);
  const uint32_t lo = lookup_plane(t.lo, sel, pick);
  const uint32_t hi = lookup_plane(t.hi, sel, pick);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = __builtin_bit_cast(float, perm(hi, lo, (static_cast<uint32_t>(4 + k) << 24) | (k << 16) | 0x0C0Cu));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t m_rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kMBufWord3);
}

// 16-byte chunk j of staged row r sits at chunk position j ^ (r & 7): the
// 32 rows a fragment or block read touches spread over 8 bank groups
__device__ __forceinline__ int m_swz(int r, int j) { return r * (kMRowBytes / 16) + (j ^ (r & 7)); }

// what a thread fetches for the next tile: two 16-byte chunks of the B
// rows, two of the codes (staged through LDS), and its lanes' absmax codes
// and group scales (kept in registers)
struct MergeFetch {
  u32x4 b[2], c[2];
  uint32_t aq[2];
  float sc[2];
};
}  // namespace

// kDirect (r <= 64, r % 8 == 0): Bp is B itself ([out][r], ldp = r) and Atp
// is A ([r][in]); the A^T fragments are gathered from A's rows once per
// workgroup.  Otherwise Bp / Atp are the zero-padded B [out][ldp] and A^T
// [in][ldp] (kHoldA: rp = 64).
template <bool kHoldA, bool kDirect>
__global__ __launch_bounds__(256, 2) void k_merge(const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ absmax_q,
                                                  const float* __restrict__ scale, int64_t n_out, int64_t in,
                                                  const uint16_t* __restrict__ Bp,
                                                  const uint16_t* __restrict__ Atp, int64_t ldp, int rp,
                                                  float s, uint16_t* __restrict__ out, int strips) {
  static_assert(kHoldA || !kDirect, "the direct form holds A");
  __shared__ __attribute__((aligned(16))) uint32_t s_o[kMRows * kMPitch];
  __shared__ __attribute__((aligned(16))) u32x4 s_b[2][kMRows * kMRowBytes / 16];
  __shared__ __attribute__((aligned(16))) u32x4 s_c[2][kMRows * kMRowBytes / 16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int strip = static_cast<int>(blockIdx.x) % strips;
  const int step = static_cast<int>(gridDim.x) / strips;
  const int rowtiles = static_cast<int>(n_out / kMRows);
  const int64_t n0 = static_cast<int64_t>(strip) * kMCols;
  const int64_t nw = n0 + 64 * wv;  // this wave's 64 columns
  const bool live = nw < in;        // whole waves: in is a multiple of 64
  // byte selector spreading the lane's two code bytes of a dword (bytes
  // 2 half, 2 half + 1) to [b0, b0, b1, b1]
  const uint32_t zsel = half ? 0x03030202u : 0x01010000u;

  // every operand through a buffer resource: offsets past the end (columns
  // past `in`, or the tile after the last) read zero, so all loads are
  // issued unconditionally and their waits are counted exactly
  // A^T [in][ldp], or A [r = ldp][in]: in * ldp elements either way
  const __amdgpu_buffer_rsrc_t rs_at = m_rsrc(Atp, static_cast<uint64_t>(in) * ldp * 2);
  const __amdgpu_buffer_rsrc_t rs_b = m_rsrc(Bp, static_cast<uint64_t>(n_out) * ldp * 2);
  const __amdgpu_buffer_rsrc_t rs_c = m_rsrc(codes, static_cast<uint64_t>(n_out) * in / 2);
  const __amdgpu_buffer_rsrc_t rs_q = m_rsrc(absmax_q, static_cast<uint64_t>(n_out) * in / 64);
  const __amdgpu_buffer_rsrc_t rs_s = m_rsrc(scale, static_cast<uint64_t>(ceil_div(n_out * in, kGroupElems)) * 4);

  // A^T rows of this wave: lane's rows nw + 32 a + r32, K from 8 half
  uint32_t a_off[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
    a_off[a] = live ? static_cast<uint32_t>(((nw + 32 * a + r32) * ldp + 8 * half) * 2) : kMPastEnd;
  auto load_a = [&](int kc, bf16x8 (&fa)[4][2]) {
    if constexpr (kDirect) {
      // A[k][n] for k = 16 st + 8 half + e (e = 0..7), n = nw + 32 a + r32;
      // r % 8 == 0, so a lane's 8 K values are all below r or all past it
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const uint32_t vo = live && 16 * st + 8 * half < ldp
                                  ? static_cast<uint32_t>(((8 * half) * in + nw + 32 * a + r32) * 2)
                                  : kMPastEnd;
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            h[e] = __builtin_amdgcn_raw_buffer_load_b16(rs_at, vo, static_cast<int>((16 * st + e) * in * 2), 0);
          fa[st][a] = m_as_bf16x8(u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                        h[6] | (h[7] << 16)});
        }
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int a = 0; a < 2; ++a)
          fa[st][a] = m_as_bf16x8(__builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_at, a_off[a], (kc + 16 * st) * 2, 0)));
    }
  };

  // staging: thread piece P = 256 i + tid (i = 0, 1) is chunk P % 8 of
  // staged row P / 8
  auto fetch = [&](int mt, int kc, MergeFetch& F) {
    const bool ok = mt < rowtiles;
    const int64_t m0 = static_cast<int64_t>(mt) * kMRows;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int P = 256 * i + tid, r = P >> 3, j = P & 7;
      // chunk j holds K = kc + 8 j .. + 7 (all past the stored rank: zero)
      const uint32_t bo = ok && kc + 8 * j < ldp ? static_cast<uint32_t>(((m0 + r) * ldp + kc) * 2 + 16 * j)
                                                 : kMPastEnd;
      F.b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_b, bo, 0, 0));
      const int64_t cb = ((m0 + r) * in + n0) / 2 + 16 * j;  // codes of columns n0 + 32 j ..
      const uint32_t co = ok && n0 + 32 * j < in ? static_cast<uint32_t>(cb) : kMPastEnd;
      F.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_c, co, 0, 0));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool lok = live && ok;
      const int64_t e0 = (m0 + 32 * c + r32) * in + nw;
      F.aq[c] = __builtin_amdgcn_raw_buffer_load_b8(rs_q, lok ? static_cast<uint32_t>(e0 >> 6) : kMPastEnd, 0, 0);
      F.sc[c] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(
                     rs_s, lok ? static_cast<uint32_t>(e0 >> 14) * 4 : kMPastEnd, 0, 0));
    }
  };
  auto stage = [&](const MergeFetch& F, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int P = 256 * i + tid, r = P >> 3, j = P & 7;
      s_b[buf][m_swz(r, j)] = F.b[i];
      s_c[buf][m_swz(r, j)] = F.c[i];
    }
  };

  // rank-r product of the wave's piece, epilogue into s_o
  auto compute = [&](const bf16x8 (&fa0)[4][2], const MergeFetch& F, int buf, int mt) {
    // D[n][m] = sum_k A^T[n][k] B[m][k]: lane holds m = 32 c + r32,
    // n = 32 a + 8 (e / 4) + 4 half + e % 4 within the wave's 64 columns
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.f;
    auto mfma_chunk = [&](const bf16x8 (&fa)[4][2], int bbuf) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 fb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) fb[c] = m_as_bf16x8(s_b[bbuf][m_swz(32 * c + r32, 2 * st + half)]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st][a], fb[c], acc[a][c], 0, 0, 0);
      }
    };
    if constexpr (kHoldA) {
      mfma_chunk(fa0, buf);
    } else {
      // rp > 64: further 64-wide chunks of B restaged through the same
      // buffer, A^T chunks loaded directly
      for (int kc = 0; kc < rp; kc += 64) {
        if (kc > 0) {
          MergeFetch G;
          fetch(mt, kc, G);
          __syncthreads();  // every wave is done with the previous chunk
          stage(G, buf);
          __syncthreads();
        }
        bf16x8 fa[4][2];
        load_a(kc, fa);
        if (live) mfma_chunk(fa, buf);
      }
    }
    if (!live) return;
    // each element: bf16_rne(fma(s, sum, w_hat)), the scaled sum added with one fp32 rounding
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const Nf4Table tab = make_table(dq_absmax(F.aq[c], F.sc[c]));
      const int r = 32 * c + r32;
      const u32x4 cw[2] = {s_c[buf][m_swz(r, 2 * wv)], s_c[buf][m_swz(r, 2 * wv + 1)]};
      uint32_t* row = s_o + r * kMPitch + 32 * wv + 2 * half;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // columns 32 a + 8 q + 4 half .. + 3: code bytes 2 half, 2 half + 1 of dword q
          float w[4];
          lookup4_f32(tab, perm(cw[a][q], cw[a][q], zsel), w);
          const f32x16& d = acc[a][c];
          const uint32_t o01 = pack_bf16x2(__builtin_fmaf(s, d[4 * q], w[0]), __builtin_fmaf(s, d[4 * q + 1], w[1]));
          const uint32_t o23 = pack_bf16x2(__builtin_fmaf(s, d[4 * q + 2], w[2]), __builtin_fmaf(s, d[4 * q + 3], w[3]));
          *reinterpret_cast<u32x2*>(row + 16 * a + 4 * q) = u32x2{o01, o23};
        }
    }
  };

  // 64 rows x 512 bytes: thread piece P = 256 i + tid is 16 bytes of row P / 32
  auto store = [&](int mt) {
    const int64_t m0 = static_cast<int64_t>(mt) * kMRows;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int P = 256 * i + tid, rl = P >> 5, pc = P & 31;
      const int64_t cp = n0 + 8 * pc;
      if (cp < in) {
        const u32x2* src = reinterpret_cast<const u32x2*>(s_o + rl * kMPitch + 4 * pc);
        const u32x2 lo = src[0], hi = src[1];
        *reinterpret_cast<u32x4*>(out + (m0 + rl) * in + cp) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
  };

  bf16x8 fa0[4][2];
  if constexpr (kHoldA) load_a(0, fa0);
  // Fetches run two tiles ahead: while tile t is computed, tile t + 1's
  // fetch (issued a tile earlier) lands and tile t + 2's is issued.  Three
  // register sets rotate statically (the loop body appears three times);
  // the LDS buffers alternate by tile parity.
  int mt = static_cast<int>(blockIdx.x) / strips;
  int buf = 0;
  MergeFetch F0, F1, F2;
  fetch(mt, 0, F0);
  stage(F0, 0);
  fetch(mt + step, 0, F1);
  // per tile: issue the fetch two ahead; barrier (this tile staged, the
  // previous tile's output stored); compute; barrier (output complete);
  // store; stage the next tile into the other buffers
  auto tile = [&](const MergeFetch& cur, const MergeFetch& nxt, MergeFetch& ahead) {
    fetch(mt + 2 * step, 0, ahead);
    __syncthreads();
    compute(fa0, cur, buf, mt);
    __syncthreads();
    store(mt);
    stage(nxt, buf ^ 1);
    mt += step;
    buf ^= 1;
  };
  while (mt < rowtiles) {
    tile(F0, F1, F2);
    if (mt >= rowtiles) break;
    tile(F1, F2, F0);
    if (mt >= rowtiles) break;
    tile(F2, F0, F1);
  }
}

static uint32_t merge_grid(int64_t out, int64_t in, int* strips_out) {
  const int strips = static_cast<int>(ceil_div(in, kMCols));
  const int64_t rowtiles = out / kMRows;
  const int cus = device_cus();
  const int64_t target = static_cast<int64_t>(kMWgPerCu) * (cus > 0 ? cus : 256);
  int64_t per_strip = target / strips;
  if (per_strip < 1) per_strip = 1;
  if (per_strip > rowtiles) per_strip = rowtiles;
  *strips_out = strips;
  return static_cast<uint32_t>(strips * per_strip);
}

bool merge_direct(int64_t r) { return r <= 64 && r % 8 == 0; }

hipError_t launch_merge(const uint8_t* codes, const uint8_t* absmax_q, const float* scale,
                        int64_t out, int64_t in, const uint16_t* Bp, const uint16_t* Atp,
                        int64_t ldp, int64_t rp, float s, uint16_t* w_out, hipStream_t st) {
  int strips = 0;
  const dim3 grid(merge_grid(out, in, &strips));
  if (rp == 64)
    hipLaunchKernelGGL((k_merge<true, false>), grid, dim3(256), 0, st, codes, absmax_q, scale, out, in, Bp, Atp,
                       ldp, static_cast<int>(rp), s, w_out, strips);
  else
    hipLaunchKernelGGL((k_merge<false, false>), grid, dim3(256), 0, st, codes, absmax_q, scale, out, in, Bp, Atp,
                       ldp, static_cast<int>(rp), s, w_out, strips);
  return hipGetLastError();
}

hipError_t launch_merge_direct(const uint8_t* codes, const uint8_t* absmax_q, const float* scale, int64_t out,
                               int64_t in, const uint16_t* B, const uint16_t* A, int64_t r, float s,
                               uint16_t* w_out, hipStream_t st) {
  int strips = 0;
  const dim3 grid(merge_grid(out, in, &strips));
  hipLaunchKernelGGL((k_merge<true, true>), grid, dim3(256), 0, st, codes, absmax_q, scale, out, in, B, A, r, 64,
                     s, w_out, strips);
  return hipGetLastError();
}

}  // namespace qlora
