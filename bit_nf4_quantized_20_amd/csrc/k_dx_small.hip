// k_dx_small.hip -- the backward's input gradient for small token counts
// (T <= 16), bound by the packed-nibble weight stream:
//
//   dX = dY W_hat + (s V) A          (paperclase lesson "QLoRA", Parte 4:
//                                     the gradient passes through the frozen
//                                     4-bit base, dX = (W_hat + s B A)^T dY)
//
// over n projections stacked along the rows of W (q|k|v: dY's columns
// [row0_i, row0_i + out_i) belong to projection i).  The weight is read once
// as codes; W_hat exists only in LDS, one 64 x 64 tile per wave at a time.
//
// k_dx_small_part: workgroup (strip, split) takes the 64 columns
// n0 = 64 strip .. + 64 of W (one block of every row) and a contiguous range
// of its 64-row chunks; its four waves take the chunks in turn.  For a chunk,
// lane l dequantizes row m0 + l's block (the same v_perm lookup as
// nf4_dequantize, bit-identical) into the wave's LDS tile [64 rows][64 cols];
// the tile is then read back transposed as the A operand of
// v_mfma_f32_16x16x32_bf16 (16 columns x 32 rows: eight 16-bit reads per
// lane), against dY's matching 32 columns for 16 tokens (tokens >= T read
// zero).  The four waves' fp32 sums meet in LDS and the workgroup writes its
// partial dX^T[strip cols][T] to part[split][t][n].
//
// k_dx_small_fin: dX[t][n] = bf16(sum over splits of part + sum_i sum_j
// sV_i[t][j] A_i[j][n]), the splits added in order (bit-reproducible), sV as
// the backward's hi + lo bf16 pairs; one rounding.
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {
constexpr int kDxPitch = 68;  // bf16 per LDS tile row: 136 bytes keep the transposed reads conflict-free
constexpr int kDxBufWord3 = 0x00020000;
constexpr uint32_t kDxPastEnd = 0x80000000u;
__device__ __forceinline__ bf16x8 dx_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
}  // namespace

// Workgroup -> (strip, split).  A 128-byte line of codes holds one row's
// blocks of four consecutive strips, so when those four workgroups run on
// different XCDs (workgroups go to the 8 XCDs round-robin by linear id) each
// line is fetched from HBM by four L2s.  The mapping puts them on one XCD,
// dispatched back to back: XCD x runs linear ids x, x + 8, x + 16, ...; its
// k-th workgroup is member k % 4 of line group k / 4 there.  Needs
// strips % 4 == 0 and a multiple of 32 workgroups; otherwise the plain
// order.
__device__ __forceinline__ void dx_strip_split(int strips, int total, int& strip, int& split) {
  const int L = static_cast<int>(blockIdx.x);
  if (strips % 4 == 0 && total % 32 == 0) {
    const int xcd = L % 8, k = L / 8;
    const int G = (k / 4) * 8 + xcd;  // line group x split, numbered over all XCDs
    strip = 4 * (G % (strips / 4)) + k % 4;
    split = G / (strips / 4);
  } else {
    strip = L % strips;
    split = L / strips;
  }
}

template <bool kFp32>
__global__ __launch_bounds__(256) void k_dx_small_part(DxSet P, int64_t in, const uint16_t* __restrict__ dY,
                                                       int T, int64_t N, int chunks_per_split, int nsplits,
                                                       float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[4][64 * kDxPitch];
  __shared__ f32x4 s_acc[4][4][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  int strip, split;
  dx_strip_split(static_cast<int>(in / 64), static_cast<int>(in / 64) * nsplits, strip, split);
  const int64_t n0 = static_cast<int64_t>(strip) * 64;
  const int nchunks = static_cast<int>(N / 64);
  const int c0 = split * chunks_per_split;
  const int c1 = min(c0 + chunks_per_split, nchunks);

  // dY [T][N]: tokens >= T read zero
  const __amdgpu_buffer_rsrc_t rs_dy = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(dY), 0, static_cast<int>(static_cast<uint64_t>(T) * N * 2), kDxBufWord3);
  // lane (token i16, K group g) reads dY[i16][chunk row + 32 ks + 8 g .. + 7]:
  // the token and group in the per-lane offset, the chunk and step in the
  // scalar one
  const uint32_t dy_row = i16 < T ? static_cast<uint32_t>(i16 * N * 2 + 16 * g) : kDxPastEnd;

  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* tile = s_w[wv];

  for (int c = c0 + wv; c < c1; c += 4) {
    const int64_t R0 = static_cast<int64_t>(c) * 64;  // the chunk's first row of the stack
    int pj = 0;
#pragma unroll
    for (int i = 1; i < kMaxProj; ++i)
      if (i < P.n && R0 >= P.proj[i].row0) pj = i;
    // lane's row within its projection, and the row's block at columns n0
    const int64_t m = R0 - P.proj[pj].row0 + lane;
    const int64_t e0 = m * in + n0;
    const u32x4* src = reinterpret_cast<const u32x4*>(P.proj[pj].codes + (e0 >> 1));
    const u32x4 cw0 = src[0], cw1 = src[1];
    const float ahat = kFp32 ? P.proj[pj].scale[e0 >> 6]
                             : dq_absmax(P.proj[pj].absmax_q[e0 >> 6], P.proj[pj].scale[e0 >> 14]);
    const Nf4Table tab = make_table(ahat);
    uint16_t* trow = tile + lane * kDxPitch;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 cw = h == 0 ? cw0 : cw1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t w[4];
        lookup8(tab, cw[k], w);  // columns 32 h + 8 k .. + 7 of the row
        u32x2* dst = reinterpret_cast<u32x2*>(trow + 32 * h + 8 * k);
        dst[0] = u32x2{w[0], w[1]};
        dst[1] = u32x2{w[2], w[3]};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // D[n][t] += sum_m W_hat[m][n] dY[t][m] over the chunk's 64 rows
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int mk = 32 * ks + 8 * g;  // this lane's 8 rows of the K step
      const bf16x8 fb = dx_bf16x8(__builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_dy, dy_row, static_cast<int>((R0 + 32 * ks) * 2), 0)));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint16_t* col = tile + mk * kDxPitch + 16 * nt + i16;
        uint32_t a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[e] = static_cast<uint32_t>(col[(2 * e) * kDxPitch]) |
                 (static_cast<uint32_t>(col[(2 * e + 1) * kDxPitch]) << 16);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dx_bf16x8(u32x4{a[0], a[1], a[2], a[3]}), fb, acc[nt],
                                                          0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the tile is read before the next chunk overwrites it
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // lane holds D[16 nt + 4 g + e][t = i16]; the waves' sums meet in LDS
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) s_acc[wv][nt][lane] = acc[nt];
  __syncthreads();
  // 64 columns x T tokens; thread -> (token t, column j) pairs
  for (int o = tid; o < T * 64; o += 256) {
    const int t = o >> 6, j = o & 63;
    const int nt = j >> 4, gg = (j >> 2) & 3, e = j & 3, l = 16 * gg + t;
    const float v = ((s_acc[0][nt][l][e] + s_acc[1][nt][l][e]) + s_acc[2][nt][l][e]) + s_acc[3][nt][l][e];
    part[(static_cast<int64_t>(split) * T + t) * in + n0 + j] = v;
  }
}

// dX[t][n] = bf16(sum_s part[s][t][n] + sum_i sum_j (hi + lo)_i[t][j] A_i[j][n]).
// One workgroup per 64 columns and 4 tokens: each projection's A rows for
// those columns (64 ranks at a time) and the tokens' sV are staged in LDS
// with coalesced loads, then thread (t, n) sums its output from there; the
// splits' partials are added in order.
__global__ __launch_bounds__(256) void k_dx_small_fin(const float* __restrict__ part, int splits, int T, int64_t in,
                                                      DownFactors A, int nproj, int r,
                                                      const uint16_t* __restrict__ v_pad, int64_t ldv, int64_t rp,
                                                      uint16_t* __restrict__ dX) {
  __shared__ float s_a[64][65];  // [rank][column]
  __shared__ float s_v[4][65];  // [token][rank]
  const int tid = threadIdx.x;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tb = 4 * static_cast<int>(blockIdx.y);  // the workgroup's first token
  const int nt = min(4, T - tb);
  // thread -> column tid % 64, token tb + tid / 64
  const int col = tid & 63, tl = tid >> 6, t = tb + tl;
  float lora = 0.f;
  for (int i = 0; i < nproj; ++i) {
    for (int j0 = 0; j0 < r; j0 += 64) {
      const int nj = min(64, r - j0);
      __syncthreads();  // the previous ranks are consumed
      for (int idx = tid; idx < 64 * nj; idx += 256) {
        const int j = idx >> 6, c = idx & 63;
        s_a[j][c] = __builtin_bit_cast(float, static_cast<uint32_t>(A.p[i][(j0 + j) * in + n0 + c]) << 16);
      }
      for (int idx = tid; idx < nt * nj; idx += 256) {
        const int tt = idx / nj, j = idx % nj;
        const uint16_t* vt = v_pad + (tb + tt) * ldv + i * 2 * rp + j0 + j;
        s_v[tt][j] = __builtin_bit_cast(float, static_cast<uint32_t>(vt[0]) << 16) +
                     __builtin_bit_cast(float, static_cast<uint32_t>(vt[rp]) << 16);
      }
      __syncthreads();
      if (tl < nt)
        for (int j = 0; j < nj; ++j) lora = __builtin_fmaf(s_v[tl][j], s_a[j][col], lora);
    }
  }
  if (tl < nt) {
    const int64_t o = static_cast<int64_t>(t) * in + n0 + col;
    float base = 0.f;
    for (int sp = 0; sp < splits; ++sp) base += part[static_cast<int64_t>(sp) * T * in + o];
    dX[o] = static_cast<uint16_t>(pack_bf16x2(base + lora, 0.f));
  }
}

namespace {
// row splits for about `target` workgroups over the in / 64 column strips,
// at most one 64-row chunk each
int splits_for(int64_t N, int64_t in, int target) {
  const int strips = static_cast<int>(in / 64);
  const int nchunks = static_cast<int>(N / 64);
  int splits = (target + strips - 1) / strips;
  if (splits > nchunks) splits = nchunks;
  return splits < 1 ? 1 : splits;
}
}  // namespace

int dx_small_max_splits(int64_t N, int64_t in) { return splits_for(N, in, kDxSmallTargetWgs); }

int dx_small_splits(int64_t N, int64_t in, int T, size_t part_bytes) {
  const int cus = device_cus();
  int splits = splits_for(N, in, 2 * (cus > 0 ? cus : 256));
  const int64_t per = static_cast<int64_t>(T) * in * 4;  // bytes of one split's partial
  if (per > 0 && static_cast<int64_t>(splits) * per > static_cast<int64_t>(part_bytes))
    splits = static_cast<int>(static_cast<int64_t>(part_bytes) / per);
  return splits < 1 ? 1 : splits;
}

hipError_t launch_dx_small(const DxSet& set, int64_t N, int64_t in, const uint16_t* dY, int T, const DownFactors& A,
                           int r, const uint16_t* v_pad, int64_t ldv, int64_t rp, uint16_t* dX, float* part,
                           size_t part_bytes, bool absmax_fp32, hipStream_t s) {
  const int splits = dx_small_splits(N, in, T, part_bytes);
  const int nchunks = static_cast<int>(N / 64);
  const int per = (nchunks + splits - 1) / splits;
  const int used = (nchunks + per - 1) / per;  // splits that get chunks
  const dim3 grid(static_cast<uint32_t>(in / 64 * used));  // (strip, split) pairs, see dx_strip_split
  if (absmax_fp32)
    hipLaunchKernelGGL(k_dx_small_part<true>, grid, dim3(256), 0, s, set, in, dY, T, N, per, used, part);
  else
    hipLaunchKernelGGL(k_dx_small_part<false>, grid, dim3(256), 0, s, set, in, dY, T, N, per, used, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dx_small_fin, dim3(static_cast<uint32_t>(in / 64), static_cast<uint32_t>((T + 3) / 4)),
                     dim3(256), 0, s, part, used, T, in, A, set.n, r, v_pad, ldv, rp, dX);
  return hipGetLastError();
}

}  // namespace qlora
