// common.hpp -- vector types, DPP helpers and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlora {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// DPP lane moves within a row of 16 lanes (bound_ctrl off, all rows/banks).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                               0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

// max over each aligned group of 16 lanes, result in every lane of the group
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
  return v;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// ---------------------------------------------------------------------------
// Launchers (host side).  Each returns hipSuccess or the launch error.
// Shapes are validated by the caller (the C ABI layer).
// ---------------------------------------------------------------------------
hipError_t launch_nf4_quantize(const float* w, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                               float* scale, hipStream_t s);
hipError_t launch_nf4_dequantize(const uint8_t* codes, const uint8_t* absmax_q, const float* scale,
                                 int64_t numel, uint16_t* out, hipStream_t s);
// Without double quantization: the exact fp32 block absmax [numel/64].
hipError_t launch_nf4_quantize_nodq(const float* w, int64_t numel, uint8_t* codes, float* absmax,
                                    hipStream_t s);
hipError_t launch_nf4_dequantize_nodq(const uint8_t* codes, const float* absmax, int64_t numel,
                                      uint16_t* out, hipStream_t s);
// out[c][r] = W_hat[r][c] for W_hat [rows][cols]; rows % 64 == 0, cols % 64 == 0
// (out rows have stride ldo elements, ldo >= rows)
// absmax_fp32: the 4.5-bit format (scale = the fp32 block absmax, one per
// block; absmax_q unused)
hipError_t launch_nf4_dequantize_transposed(const uint8_t* codes, const uint8_t* absmax_q,
                                            const float* scale, int64_t rows, int64_t cols,
                                            uint16_t* out, int64_t ldo, hipStream_t s,
                                            bool absmax_fp32 = false);

// Projections that share one input (q|k|v, gate|up) go through one call.
constexpr int kMaxProj = 8;
struct DownFactors { const uint16_t* p[kMaxProj]; };

// sU[t][p rp + j] = scale * sum_k in[t][k] P_p[j][k] for the nP rank factors
// P_p [r][K] (K-contiguous; in [T][K] with row stride ldin), j < r; 0 for
// r <= j < rp; as bf16 pairs hi + lo.  Written to (either may be null)
//   pad    [T][ldpad]        projection p: hi in columns [2p rp, 2p rp + rp),
//                            lo in [2p rp + rp, 2(p+1) rp)
//   hilo_t [nP][2 rp][ldt]   transposed: hi rows [0, rp), lo rows [rp, 2 rp)
// `part` is fp32 scratch of lora_down_part_bytes(T, K, nP * rp) bytes.
// K % 64 == 0, rp % 64 == 0.
size_t lora_down_part_bytes(int64_t T, int64_t K, int64_t nprp);
// keep (optional, LoRA dropout): in[t][k] counts only where bit k % 8 of
// keep[t * ldk + k / 8] is set.
hipError_t launch_lora_down(const uint16_t* in, int64_t ldin, int64_t T, int64_t K,
                            const uint16_t* const* P, int nP, int64_t r, float scale, uint16_t* pad,
                            int64_t ldpad, uint16_t* hilo_t, int64_t ldt, int64_t rp, float* part,
                            hipStream_t s, const uint8_t* keep = nullptr, int64_t ldk = 0);
// out(j, c) = sum_t (Pt[j'][t] + Pt[rp + j'][t]) Q[t][c] for j < r, c < C (C % 64
// == 0), laid out as out[j * C + c] (out_jc) or out[c * r + j], where rank j is
// rank j' = j % rproj of the projection j / rproj of Pt (projections stacked,
// 2 rp rows each; rproj = r: one projection, j' = j), as
// lora_grad_slices(T, C, ldq) token-slice sums: slice z written to
// part[z * r * C ...] (every element once), to be added in order by
// launch_sum_slices.  (Q rows have stride ldq elements, ldq >= C.)  keep
// (optional, LoRA dropout, out_jc only): Q[t][c] counts only where bit c % 8 of
// keep[t * ldk + c / 8] is set; every sum is multiplied by oscale.
int64_t lora_grad_slices(int64_t T, int64_t C, int64_t ldq);
hipError_t launch_lora_grad(const uint16_t* Pt, int64_t T, int64_t ldt, int64_t rp, const uint16_t* Q,
                            int64_t C, int64_t ldq, int64_t r, float* part, bool out_jc, hipStream_t s,
                            const uint8_t* keep = nullptr, int64_t ldk = 0, float oscale = 1.f,
                            int64_t rproj = 0);
// dst[c][r] = src[r][c] for src [R][C]
hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst,
                                 hipStream_t s);
// dst[i][j] = dst[i][Cp + j] (R x 2Cp, bf16) = src(i, j) for j < C, else 0, where
// src(i, j) = src[i * C + j] (!transpose) or src[j * R + i] (transpose).
// (dst rows have stride ldd elements, ldd >= 2 Cp)
hipError_t launch_pad_bf16(const uint16_t* src, int64_t R, int64_t C, bool transpose, uint16_t* dst,
                           int64_t Cp, int64_t ldd, hipStream_t s);
// launch_pad_bf16(src[i], R[i], C, false, dst[i], Cp, ldd) for i < n (<= kMaxProj)
// in one launch
hipError_t launch_pad_many(const uint16_t* const* src, const int64_t* R, uint16_t* const* dst, int n, int64_t C,
                           int64_t Cp, int64_t ldd, hipStream_t s);
// one launch doing launch_transpose_bf16(B, out, r, bt) and
// launch_pad_bf16(A, in, r, true, a_t_pad, rp, ldd)
hipError_t launch_factor_prep(const uint16_t* B, int64_t out, int64_t r, uint16_t* bt, const uint16_t* A,
                              int64_t in, uint16_t* a_t_pad, int64_t rp, int64_t ldd, hipStream_t s);
hipError_t launch_fill_f32(float* dst, int64_t n, float v, hipStream_t s);
// count (<= kMaxFill) buffers dst[i] of n[i] floats set to v in one launch
constexpr int kMaxFill = 2 * kMaxProj;
hipError_t launch_fill_many_f32(float* const* dst, const int64_t* n, int count, float v, hipStream_t s);
// out[b][i] = sum over z < slices[b] of part[b][z * stride[b] + i] (stride
// NULL: n), in order, for count (<= kMaxFill) jobs in one launch; n[b] and
// stride[b] multiples of 4, 16-byte aligned.
hipError_t launch_sum_slices(const float* const* part, const int* slices, const int64_t* n, float* const* out,
                             int count, hipStream_t s, const int64_t* stride = nullptr);

// Split-K of the GEMM launches below: grids of 128 x 128 tiles below one
// workgroup per CU split K into gemm_splits(M, N, K0) ranges (1: none), each
// written as fp32 partials into `part` (gemm_split_bytes(M, N, K0) bytes, part
// of the caller's workspace), then added in order and rounded once; with no
// or too small a `part` the launch does not split.  The split count depends
// on the shape only.
int gemm_splits(int64_t M, int64_t N, int64_t K);
size_t gemm_split_bytes(int64_t M, int64_t N, int64_t K);

// C[M][N] (bf16, ldc) = sum over the two K segments of act_i[m][k] * wt_i[n][k]
// (bf16, K-contiguous, leading dims lda_i / ldw_i).  K0, K1 multiples of 64
// (K1 may be 0).  N % 64 == 0.
// keep (optional): LoRA dropout mask of C's elements, bit n % 8 of byte
// keep[m * ldk + n / 8]; the extension segment's product is multiplied by
// keep_scale where the bit is set and by 0 elsewhere before the main segment
// is added, so C is still rounded once.
hipError_t launch_gemm_nt(int64_t M, int64_t N, const uint16_t* act0, int64_t lda0,
                          const uint16_t* wt0, int64_t ldw0, int64_t K0, const uint16_t* act1,
                          int64_t lda1, const uint16_t* wt1, int64_t ldw1, int64_t K1, uint16_t* C,
                          int64_t ldc, hipStream_t s, const uint8_t* keep = nullptr, int64_t ldk = 0,
                          float keep_scale = 1.f, float* part = nullptr, size_t part_bytes = 0);

// Same, with the main segment's weight given as NF4 projections stacked
// along N (nproj <= kMaxProj; projection i owns output columns
// [sum_{j<i} rows_j, ... + rows_i) and is dequantized while staged into
// LDS); the LoRA segment's activation is each projection's act1 (row stride
// lda1), its weight wt1 [N][ldw1] shared.
struct Nf4Proj {
  const uint8_t* codes; const uint8_t* absmax_q; const float* scale;
  int64_t rows;
  const uint16_t* act1;
};
// bf16 weight of nproj stacked projections (rows[i] rows each, N = sum) whose
// LoRA extension reads projection i's own activation block act1[i] for the
// output columns of projection i (K1 = 2 rp, wt1 the stacked [N][2 rp] factor).
// Needs every tile inside one projection: gemm_proj_aligned(M, nproj, rows).
bool gemm_proj_aligned(int64_t M, int nproj, const int64_t* rows);
hipError_t launch_gemm_nt_proj(int64_t M, int nproj, const int64_t* rows, const uint16_t* const* act1,
                               const uint16_t* act0, int64_t lda0, const uint16_t* wt0, int64_t ldw0,
                               int64_t K0, int64_t lda1, const uint16_t* wt1, int64_t ldw1, int64_t K1,
                               uint16_t* C, int64_t ldc, hipStream_t s, float* part = nullptr,
                               size_t part_bytes = 0);
hipError_t launch_gemm_nf4(int64_t M, int nproj, const Nf4Proj* proj, const uint16_t* act0,
                           int64_t lda0, int64_t K0, int64_t lda1, const uint16_t* wt1,
                           int64_t ldw1, int64_t K1, uint16_t* C, int64_t ldc, hipStream_t s,
                           float* part = nullptr, size_t part_bytes = 0);
// dX-shaped product with NF4 weights read transposed: C[M][N] = sum_i
// act0[m][k_i + k] W_hat_i[k][n] + (LoRA segment, as in launch_gemm_nt), where
// projection i (proj[i].rows rows of N = in columns, rows % 64 == 0) owns the
// K range [k_i, k_i + rows) of act0 (row stride lda0), k_i the rows before it.
// Each weight tile is dequantized and transposed while it is staged into LDS,
// so W_hat^T never exists in HBM.  proj[i].act1 is not read.  Needs
// nf4t_fits(rows, in) for every projection (its codes addressed with 32-bit
// offsets).
bool nf4t_fits(int64_t rows, int64_t in);
hipError_t launch_gemm_nf4t(int64_t M, int64_t N, int nproj, const Nf4Proj* proj, const uint16_t* act0,
                            int64_t lda0, const uint16_t* act1, int64_t lda1, const uint16_t* wt1,
                            int64_t ldw1, int64_t K1, uint16_t* C, int64_t ldc, hipStream_t s,
                            const uint8_t* keep = nullptr, int64_t ldk = 0, float keep_scale = 1.f,
                            float* part = nullptr, size_t part_bytes = 0);

// W_merged[m][n] = bf16(W_hat[m][n] + s * sum_j Bp[m][j] Atp[n][j]) for the
// NF4 weight [out][in] (out % 64 == 0, in % 64 == 0); Bp [out][ldp] and Atp
// [in][ldp] hold B and A^T zero-padded to rp (a multiple of 16) columns.
hipError_t launch_merge(const uint8_t* codes, const uint8_t* absmax_q, const float* scale,
                        int64_t out, int64_t in, const uint16_t* Bp, const uint16_t* Atp,
                        int64_t ldp, int64_t rp, float s, uint16_t* w_out, hipStream_t st);
// r <= 64 with r % 8 == 0: B [out][r] and A [r][in] read as they are (no
// padded copies)
bool merge_direct(int64_t r);
hipError_t launch_merge_direct(const uint8_t* codes, const uint8_t* absmax_q, const float* scale, int64_t out,
                               int64_t in, const uint16_t* B, const uint16_t* A, int64_t r, float s,
                               uint16_t* w_out, hipStream_t st);

// Small-token forward (T <= 16, r <= 64): Y = X W_hat^T + s (X A^T) B^T.
// decode_fits() lists the shapes it takes.  For r <= 16 and at most
// kDecodeFusedMaxWgs workgroups (16 output rows each) it is one launch with
// no workspace, every workgroup computing U = X A^T itself; otherwise
// (decode_pre_u) U is computed once into a workspace of decode_u_bytes()
// first, which saves each workgroup reading all of A.
constexpr int64_t kDecodeMaxT = 16;
constexpr int64_t kDecodeFusedMaxWgs = 256;
constexpr int64_t kDecodeMaxRank = 64;
bool decode_fits(int64_t T, int64_t in, int64_t out, int64_t r);
// Small-token backward (T <= kDxSmallMaxT, no dropout): dX, dA and dB of n
// projections stacked along W's rows (projection i's rows start at row0, its
// dY columns), in three launches (k_dx_small.hip).
constexpr int kDxSmallMaxT = 16;
// The row splits' partials are sized for this many workgroups (two per CU
// on a 256-CU device); with more CUs the split count is capped by the space.
constexpr int kDxSmallTargetWgs = 512;
// Most row splits the partials of dX can need ([splits][T][in] fp32).
int dx_small_max_splits(int64_t N, int64_t in);
struct DxProj {
  const uint8_t* codes; const uint8_t* absmax_q; const float* scale;
  int64_t row0;
};
struct DxSet {
  DxProj proj[kMaxProj];
  int n;
};
// Everything the small-token backward's kernels read, by value.  The host
// fills the inputs; launch_bwd_small fills the split and chunk counts.
struct BwdSmallDev {
  DxSet set;
  DownFactors A, B;           // A_i [r][in], B_i [out_i][r]
  int64_t out[kMaxProj];
  int vc0[kMaxProj + 1];      // first V chunk of each projection
  int n, T, r, splits, per, nu, gp, uvw;
  int64_t N, in;
  const uint16_t* X;          // [T][in]
  const uint16_t* dY;         // [T][N]
  float* dxp;                 // dX row-split partials [splits][T][in]
  float* uvp;                 // U and V chunk partials (bwd_small_uv_bytes)
  float* su;                  // s U_i [n][T][r]
  float* sv;                  // s V_i [n][T][r]
  float s;
  uint16_t* dX;
  float* dA[kMaxProj];
  float* dB[kMaxProj];
};
// dxp_bytes: the space at dxp (caps the row splits)
hipError_t launch_bwd_small(BwdSmallDev a, size_t dxp_bytes, bool absmax_fp32, hipStream_t s);
size_t bwd_small_uv_bytes(int64_t T, int64_t in, const int64_t* outs, int n, int64_t r);

struct DecodeProj {
  const uint8_t* codes; const uint8_t* absmax_q; const float* scale;
  const uint16_t* A; const uint16_t* B;
  int64_t out;
};
// The projections of one launch (kernel argument): workgroup ranges and the
// output columns of each, Y = the first projection's column 0.
struct DecodeSet {
  DecodeProj proj[kMaxProj];
  int wg0[kMaxProj];
  int64_t col0[kMaxProj];
  uint16_t* Y;
  int n;
};
bool decode_pre_u(int n, const int64_t* outs, int64_t r);
inline size_t decode_u_bytes(int n, int64_t T, int64_t r) { return static_cast<size_t>(n * T * r * 4); }
// n (1..kMaxProj) projections sharing X, outputs side by side in Y [T][ldy]
// (projection i from column sum_{j<i} out_j), all in one launch (two with
// decode_pre_u, which needs u_ws of decode_u_bytes(n, T, r)).
hipError_t launch_decode_fwd(int n, const DecodeProj* proj, int64_t in, const uint16_t* X, int64_t T,
                             int64_t r, float s, uint16_t* Y, int64_t ldy, float* u_ws, hipStream_t st);

// The persistent weight-stream form of the small-token forward
// (k_decode_stream.hip): one workgroup per CU over contiguous ranges of
// 16-row blocks, U = X A^T taken from u_ws.  Shapes it takes: in % 4096 == 0,
// T * in <= kStreamMaxTokElems (the tokens' X fits in LDS), r <= 64, 2 to 8
// row blocks per CU and at most two projections per workgroup.
constexpr int64_t kStreamMaxTokElems = 65536;
bool stream_fits(int n, const int64_t* outs, int64_t in, int64_t T, int64_t r, int num_cus);
hipError_t launch_decode_stream(const DecodeSet& set, int64_t in, const uint16_t* X, int64_t T, int64_t r,
                                float s, int64_t ldy, const float* u_ws, int total_rb, int num_cus,
                                hipStream_t st);
// U[p][t][k] = sum_i X[t][i] A_p[k][i] (fp32) for the n projections of set
hipError_t launch_decode_u(const DecodeSet& set, int64_t in, const uint16_t* X, int64_t T, int64_t r,
                           float* u_ws, hipStream_t st);
// compute units of the current device (cached per device)
int device_cus();

}  // namespace qlora
