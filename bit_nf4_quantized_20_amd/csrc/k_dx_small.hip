// k_dx_small.hip -- the whole backward for small token counts (T <= 16, no
// dropout), in three launches, bound by the packed-nibble weight stream:
//
//   dX = dY W_hat + (s V) A,  dA = (s V)^T X,  dB = dY^T (s U),
//   U = X A^T,  V = dY B      (paperclase lesson "QLoRA", Parte 4: the
//                              gradient passes through the frozen 4-bit
//                              base, dX = (W_hat + s B A)^T dY; dA, dB by the
//                              chain rule, no gradient for W_hat)
//
// over n projections stacked along the rows of W (q|k|v: dY's columns
// [row0_i, row0_i + out_i) belong to projection i).  The weight is read once
// as codes; W_hat exists only in LDS, one 64 x 64 tile per wave at a time.
//
// k_bwd_small_part (launch 1), two kinds of workgroup:
//  * (strip, split): the 64 columns n0 = 64 strip .. + 64 of W (one block of
//    every row) over a contiguous range of its 64-row chunks; its four waves
//    take the chunks in turn.  For a chunk, lane l dequantizes row m0 + l's
//    block (the same v_perm lookup as nf4_dequantize, bit-identical) into the
//    wave's LDS tile [64 rows][64 cols]; the tile is read back transposed as
//    the A operand of v_mfma_f32_16x16x32_bf16 (16 columns x 32 rows: eight
//    16-bit reads per lane), against dY's matching 32 columns for 16 tokens
//    (tokens >= T read zero).  The waves' fp32 sums meet in LDS and the
//    workgroup writes its partial dX^T[strip cols][T] to dxp[split][t][n].
//  * a 128-wide chunk of a rank-r reduction: U's (128 columns of X and of
//    every A_i) or V's (128 rows of one projection's dY columns and B_i),
//    staged in LDS, each thread summing T x r products for 4 ranks of one
//    token; fp32 partials per chunk.
// k_bwd_small_uv (launch 2): s U and s V in fp32, the chunks added in a
// fixed order.
// k_bwd_small_fin (launch 3), three kinds of workgroup:
//  * dX[t][n] = bf16(sum over splits of dxp + sum_i sum_j sV_i[t][j]
//    A_i[j][n]), the splits added in order (bit-reproducible), one rounding;
//  * dA_i[j][k] = sum_t sV_i[t][j] X[t][k] and dB_i[m][j] = sum_t dY[t][m]
//    sU_i[t][j], each element once (no atomics: written, reproducible).
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
__device__ __forceinline__ void dx_strip_split(int L, int strips, int total, int& strip, int& split) {
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

namespace {
constexpr int kUvChunk = 128;  // columns of X / rows of dY per rank-reduction chunk

// One chunk of U = X A_i^T (q < nu: columns [128 q, + 128) of X and of every
// A_i) or of V = dY_i B_i (the chunk's 128 rows of one projection): the
// chunk's activations [T][128] and the factor's [128][64] ranks at a time
// staged in LDS (bf16), then thread (token tid / 16, ranks 4 (tid % 16) .. + 3)
// sums its 4 x 128 products in fp32.  Partials: up[q][i][t][j], then
// vp[c][t][j] after them.
__device__ __forceinline__ void uv_part(const BwdSmallDev& a, int q, uint16_t* lds) {
  uint16_t* xs = lds;                    // [16][kUvChunk]
  uint16_t* ps = lds + 16 * kUvChunk;    // [kUvChunk][64]
  const int tid = threadIdx.x, t = tid >> 4, jq = tid & 15;
  const int T = a.T, r = a.r, n = a.n;
  float* const up = a.uvp;
  float* const vp = a.uvp + static_cast<int64_t>(a.nu) * n * T * r;
  auto f = [](uint16_t h) { return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16); };
  // sum over the chunk's kn positions of xs[t][k] ps[k][4 jq + e]
  auto dot4 = [&](int kn, float (&acc)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = 0.f;
    for (int k = 0; k < kn; ++k) {
      const float x = f(xs[t * kUvChunk + k]);
      const u32x2 pv = *reinterpret_cast<const u32x2*>(ps + k * 64 + 4 * jq);
      acc[0] = __builtin_fmaf(x, __builtin_bit_cast(float, pv[0] << 16), acc[0]);
      acc[1] = __builtin_fmaf(x, __builtin_bit_cast(float, pv[0] & 0xffff0000u), acc[1]);
      acc[2] = __builtin_fmaf(x, __builtin_bit_cast(float, pv[1] << 16), acc[2]);
      acc[3] = __builtin_fmaf(x, __builtin_bit_cast(float, pv[1] & 0xffff0000u), acc[3]);
    }
  };
  if (q < a.nu) {
    const int64_t k0 = static_cast<int64_t>(q) * kUvChunk;
    const int kn = static_cast<int>(a.in - k0 < kUvChunk ? a.in - k0 : kUvChunk);
    for (int idx = tid; idx < 16 * kUvChunk; idx += 256) {
      const int tt = idx / kUvChunk, k = idx % kUvChunk;
      xs[idx] = (tt < T && k < kn) ? a.X[tt * a.in + k0 + k] : uint16_t(0);
    }
    for (int i = 0; i < n; ++i)
      for (int j0 = 0; j0 < r; j0 += 64) {
        const int nj = min(64, r - j0);
        __syncthreads();  // xs written / the previous ranks consumed
        for (int idx = tid; idx < 64 * kUvChunk; idx += 256) {
          const int j = idx / kUvChunk, k = idx % kUvChunk;  // coalesced along a row of A_i
          ps[k * 64 + j] = (j < nj && k < kn) ? a.A.p[i][static_cast<int64_t>(j0 + j) * a.in + k0 + k] : uint16_t(0);
        }
        __syncthreads();
        if (t < T) {
          float acc[4];
          dot4(kn, acc);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * jq + e < nj) up[((static_cast<int64_t>(q) * n + i) * T + t) * r + j0 + 4 * jq + e] = acc[e];
        }
      }
  } else {
    const int c = q - a.nu;
    int i = 0;
    for (int k = 1; k < n; ++k)
      if (c >= a.vc0[k]) i = k;
    const int64_t m0 = static_cast<int64_t>(c - a.vc0[i]) * kUvChunk;
    const int mn = static_cast<int>(a.out[i] - m0 < kUvChunk ? a.out[i] - m0 : kUvChunk);
    const int64_t col0 = a.set.proj[i].row0 + m0;  // the chunk's first column of dY
    for (int idx = tid; idx < 16 * kUvChunk; idx += 256) {
      const int tt = idx / kUvChunk, m = idx % kUvChunk;
      xs[idx] = (tt < T && m < mn) ? a.dY[tt * a.N + col0 + m] : uint16_t(0);
    }
    for (int j0 = 0; j0 < r; j0 += 64) {
      const int nj = min(64, r - j0);
      __syncthreads();
      for (int idx = tid; idx < 64 * kUvChunk; idx += 256) {
        const int m = idx / 64, j = idx % 64;  // B_i is [out][r]: coalesced along a row
        ps[idx] = (j < nj && m < mn) ? a.B.p[i][(m0 + m) * r + j0 + j] : uint16_t(0);
      }
      __syncthreads();
      if (t < T) {
        float acc[4];
        dot4(mn, acc);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * jq + e < nj) vp[(static_cast<int64_t>(c) * T + t) * r + j0 + 4 * jq + e] = acc[e];
      }
    }
  }
}
}  // namespace

// Launch 1: workgroups [0, a.uvw) the U and V chunks (first, so that they
// run beside the dX row splits instead of after them; the count is padded to
// a multiple of 8, the padding exits at once, so the splits keep their XCD
// order), then [a.uvw, a.uvw + gp) the dX row splits.
template <bool kFp32>
__global__ __launch_bounds__(256) void k_bwd_small_part(BwdSmallDev a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[4][64 * kDxPitch];
  __shared__ f32x4 s_acc[4][4][64];
  const int L0 = static_cast<int>(blockIdx.x);
  if (L0 < a.uvw) {  // (uniform)
    if (L0 < a.nu + a.vc0[a.n]) uv_part(a, L0, &s_w[0][0]);
    return;
  }
  const int L = L0 - a.uvw;
  const DxSet& P = a.set;
  const int64_t in = a.in, N = a.N;
  const uint16_t* __restrict__ dY = a.dY;
  const int T = a.T, chunks_per_split = a.per, nsplits = a.splits;
  float* __restrict__ part = a.dxp;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  int strip, split;
  dx_strip_split(L, static_cast<int>(in / 64), static_cast<int>(in / 64) * nsplits, strip, split);
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



// Launch 2: s U_i and s V_i [n][T][r] in fp32.  Workgroup (projection i,
// 64 of its T r outputs): thread (output o, quarter qq) adds the chunks
// qq, qq + 4, ... of U and of V (independent loads, eight in flight), then
// the four quarter sums meet in LDS in a fixed order.
__global__ __launch_bounds__(256) void k_bwd_small_uv(BwdSmallDev a) {
  __shared__ float s_u[4][64], s_v[4][64];
  const int T = a.T, r = a.r, n = a.n, TR = T * r;
  const int blocks = (TR + 63) / 64;
  const int i = static_cast<int>(blockIdx.x) / blocks;
  const int o = (static_cast<int>(blockIdx.x) % blocks) * 64 + (threadIdx.x & 63);
  const int qq = threadIdx.x >> 6;
  const float* up = a.uvp;
  const float* vp = a.uvp + static_cast<int64_t>(a.nu) * n * TR;
  float u = 0.f, v = 0.f;
  if (o < TR) {
#pragma unroll 8
    for (int q = qq; q < a.nu; q += 4) u += up[(static_cast<int64_t>(q) * n + i) * TR + o];
#pragma unroll 8
    for (int c = a.vc0[i] + qq; c < a.vc0[i + 1]; c += 4) v += vp[static_cast<int64_t>(c) * TR + o];
  }
  s_u[qq][threadIdx.x & 63] = u;
  s_v[qq][threadIdx.x & 63] = v;
  __syncthreads();
  if (qq == 0 && o < TR) {
    const int l = threadIdx.x;
    a.su[static_cast<int64_t>(i) * TR + o] = a.s * (((s_u[0][l] + s_u[1][l]) + s_u[2][l]) + s_u[3][l]);
    a.sv[static_cast<int64_t>(i) * TR + o] = a.s * (((s_v[0][l] + s_v[1][l]) + s_v[2][l]) + s_v[3][l]);
  }
}

// Launch 3: workgroups [0, gx) dX (64 columns x 4 tokens each), then
// [gx, gx + n in / 64) dA (one projection's 64 columns each), then N / 64
// for dB (64 stacked rows each).
__global__ __launch_bounds__(256) void k_bwd_small_fin(BwdSmallDev a) {
  __shared__ float s_a[64][65];   // dX: [rank][column]
  __shared__ float s_t[16][65];   // dX: sV [token][rank]; dA: X [token][column]; dB: dY [token][row]
  __shared__ float s_r[16][257];  // dA: sV, dB: sU [token][rank]
  const int tid = threadIdx.x, T = a.T, r = a.r;
  const int64_t in = a.in;
  const int strips = static_cast<int>(in / 64);
  const int gx = strips * ((T + 3) / 4), ga = a.n * strips;
  const int L = static_cast<int>(blockIdx.x);
  if (L < gx) {
    // dX[t][n] = bf16(sum_s dxp[s][t][n] + sum_i sum_j sV_i[t][j] A_i[j][n])
    const int64_t n0 = static_cast<int64_t>(L % strips) * 64;
    const int tb = 4 * (L / strips);  // the workgroup's first token
    const int nt = min(4, T - tb);
    const int col = tid & 63, tl = tid >> 6, t = tb + tl;
    float lora = 0.f;
    for (int i = 0; i < a.n; ++i) {
      for (int j0 = 0; j0 < r; j0 += 64) {
        const int nj = min(64, r - j0);
        __syncthreads();  // the previous ranks are consumed
        for (int idx = tid; idx < 64 * nj; idx += 256) {
          const int j = idx >> 6, c = idx & 63;
          s_a[j][c] = __builtin_bit_cast(float, static_cast<uint32_t>(a.A.p[i][(j0 + j) * in + n0 + c]) << 16);
        }
        for (int idx = tid; idx < nt * nj; idx += 256) {
          const int tt = idx / nj, j = idx % nj;
          s_t[tt][j] = a.sv[(static_cast<int64_t>(i) * T + tb + tt) * r + j0 + j];
        }
        __syncthreads();
        if (tl < nt)
          for (int j = 0; j < nj; ++j) lora = __builtin_fmaf(s_t[tl][j], s_a[j][col], lora);
      }
    }
    if (tl < nt) {
      const int64_t o = static_cast<int64_t>(t) * in + n0 + col;
      float base = 0.f;
#pragma unroll 8
      for (int sp = 0; sp < a.splits; ++sp) base += a.dxp[static_cast<int64_t>(sp) * T * in + o];
      a.dX[o] = static_cast<uint16_t>(pack_bf16x2(base + lora, 0.f));
    }
    return;
  }
  if (L < gx + ga) {
    // dA_i[j][k0 + c] = sum_t sV_i[t][j] X[t][k0 + c]
    const int q = L - gx, i = q / strips;
    const int64_t k0 = static_cast<int64_t>(q % strips) * 64;
    for (int idx = tid; idx < T * 64; idx += 256)
      s_t[idx >> 6][idx & 63] = __builtin_bit_cast(float, static_cast<uint32_t>(a.X[(idx >> 6) * in + k0 + (idx & 63)]) << 16);
    for (int idx = tid; idx < T * r; idx += 256) s_r[idx / r][idx % r] = a.sv[static_cast<int64_t>(i) * T * r + idx];
    __syncthreads();
    const int c = tid & 63;
    float* __restrict__ dA = a.dA[i];
    for (int j = tid >> 6; j < r; j += 4) {
      float d = 0.f;
      for (int tt = 0; tt < T; ++tt) d = __builtin_fmaf(s_r[tt][j], s_t[tt][c], d);
      dA[static_cast<int64_t>(j) * in + k0 + c] = d;
    }
    return;
  }
  // dB_i[m0 + m][j] = sum_t dY[t][row] sU_i[t][j] for the 64 stacked rows
  // row = 64 (L - gx - ga) + m
  const int64_t R0 = static_cast<int64_t>(L - gx - ga) * 64;
  int i = 0;
  for (int k = 1; k < a.n; ++k)
    if (R0 >= a.set.proj[k].row0) i = k;
  const int64_t m0 = R0 - a.set.proj[i].row0;
  for (int idx = tid; idx < T * 64; idx += 256)
    s_t[idx >> 6][idx & 63] = __builtin_bit_cast(float, static_cast<uint32_t>(a.dY[(idx >> 6) * a.N + R0 + (idx & 63)]) << 16);
  for (int idx = tid; idx < T * r; idx += 256) s_r[idx / r][idx % r] = a.su[static_cast<int64_t>(i) * T * r + idx];
  __syncthreads();
  float* __restrict__ dB = a.dB[i];
  for (int j0 = 0; j0 < r; j0 += 64) {
    const int j = j0 + (tid & 63);
    if (j < r)
      for (int m = tid >> 6; m < 64; m += 4) {
        float d = 0.f;
        for (int tt = 0; tt < T; ++tt) d = __builtin_fmaf(s_t[tt][m], s_r[tt][j], d);
        dB[(m0 + m) * r + j] = d;
      }
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

hipError_t launch_bwd_small(BwdSmallDev a, size_t dxp_bytes, bool absmax_fp32, hipStream_t s) {
  const int strips = static_cast<int>(a.in / 64);
  const int nchunks = static_cast<int>(a.N / 64);
  const int splits = dx_small_splits(a.N, a.in, a.T, dxp_bytes);
  a.per = (nchunks + splits - 1) / splits;
  a.splits = (nchunks + a.per - 1) / a.per;  // splits that get chunks
  a.gp = strips * a.splits;
  a.nu = static_cast<int>(ceil_div(a.in, kUvChunk));
  a.vc0[0] = 0;
  for (int i = 0; i < a.n; ++i) a.vc0[i + 1] = a.vc0[i] + static_cast<int>(ceil_div(a.out[i], kUvChunk));
  a.uvw = static_cast<int>(round_up(a.nu + a.vc0[a.n], 8));
  const uint32_t g1 = static_cast<uint32_t>(a.uvw + a.gp);
  if (absmax_fp32) hipLaunchKernelGGL(k_bwd_small_part<true>, dim3(g1), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_bwd_small_part<false>, dim3(g1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bwd_small_uv, dim3(static_cast<uint32_t>(a.n * ((a.T * a.r + 63) / 64))), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t g3 = static_cast<uint32_t>(strips * ((a.T + 3) / 4) + a.n * strips + nchunks);
  hipLaunchKernelGGL(k_bwd_small_fin, dim3(g3), dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t bwd_small_uv_bytes(int64_t T, int64_t in, const int64_t* outs, int n, int64_t r) {
  int64_t chunks = ceil_div(in, kUvChunk) * n;
  for (int i = 0; i < n; ++i) chunks += ceil_div(outs[i], kUvChunk);
  return static_cast<size_t>(chunks * T * r * 4);
}

}  // namespace qlora
