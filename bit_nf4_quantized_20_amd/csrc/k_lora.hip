// k_lora.hip -- the rank-r parts of the QLoRA linear (paperclase lesson
// "QLoRA", Parte 4: h = W_hat x + (alpha/r) B A x and its gradients), on MFMA:
//   F1  sU = s X A^T             B1  sV = s dY B
//   B3  dA = (sV)^T X            dB = dY^T (sU)
// sU and sV are kept as bf16 pairs hi + lo (hi = bf16(v), lo = bf16(v - hi)),
// so products with them carry ~16 bits of the fp32 value; all accumulation is
// fp32.  Also the zero-padding / transposition of the small LoRA matrices
// into the layouts the GEMM's extra K-steps read.
#include <type_traits>

#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

typedef float f32x4v __attribute__((ext_vector_type(4)));

namespace {
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// LoRA dropout: eight bf16 (one 16-byte piece) with the eight keep bits of
// byte b (bit e for element e); dropped elements become +0.
__device__ __forceinline__ u32x4 keep_bf16x8(u32x4 v, uint32_t b) {
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = ((b >> (2 * d)) & 1u) ? 0x0000ffffu : 0u;
    const uint32_t hi = ((b >> (2 * d + 1)) & 1u) ? 0xffff0000u : 0u;
    o[d] = v[d] & (lo | hi);
  }
  return o;
}
}  // namespace

// ---------------------------------------------------------------------------
// lora_down: sU = scale * in P^T for in [T][K] (X or dY) and P [r][K] (A or
// B^T), written as bf16 hi/lo pairs.  A skinny GEMM (r <= 256 columns) bound
// by streaming `in` once, so the work is split in two dimensions: a
// workgroup takes 128 tokens x 64 ranks x one K-chunk, so P is re-read only
// once per 128 tokens and the grid still has ~256 workgroups.  Each writes
// its fp32 partial tile; k_lora_down_fin adds the K-chunks in a fixed order
// (deterministic), scales, splits hi/lo and writes the padded / transposed
// layouts.
//
// Partial kernel: 4 waves (2 x 2; 64 tokens x 32 ranks each), K-step 64,
// tiles through registers into a double-buffered swizzled LDS stage (one
// barrier per step), v_mfma_f32_32x32x16_bf16 with the rank rows as the A
// operand, so a lane holds 16 ranks of one token and stores them as four
// 16-byte writes.
// ---------------------------------------------------------------------------
constexpr int kDownTok = 128;   // tokens per workgroup
constexpr int kDownRanks = 64;  // ranks per workgroup
constexpr uint32_t kDownPastEnd = 0x80000000u;  // past every buffer (all < 2^31 bytes)
constexpr int kDownBufWord3 = 0x00020000;

namespace {
__device__ __forceinline__ int down_swz(int row, int chunk) { return chunk ^ ((row & 7) ^ ((row >> 3) & 1)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t down_rsrc(const uint16_t* base, int64_t ld, int64_t row0,
                                                            int64_t nrows) {
  const uint64_t bytes = static_cast<uint64_t>(nrows > row0 ? nrows - row0 : 0) * ld * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + row0 * ld), 0,
                                           static_cast<int>(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                           kDownBufWord3);
}
}  // namespace

// part[kc][t][p rp + j] (fp32, [KC][T][nP rp]) = sum over chunk kc of
// in[t][k] P_p[j][k], for the nP rank factors P_p (one per projection).
// kMask: in[t][k] counts only where bit k % 8 of keep[t * ldk + k / 8] is set.
template <bool kMask>
__global__ __launch_bounds__(256) void k_lora_down_part(const uint16_t* __restrict__ in, int64_t ldin,
                                                        int64_t T, int64_t K, DownFactors P,
                                                        int r, int rp, int64_t kch,
                                                        float* __restrict__ part,
                                                        const uint8_t* __restrict__ keep, int64_t ldk) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kDownTok * 64];
  __shared__ __attribute__((aligned(16))) uint16_t s_p[2][kDownRanks * 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kDownTok;
  const int64_t kc = blockIdx.y;
  const int tiles_per_p = rp / kDownRanks;
  const int pj = static_cast<int>(blockIdx.z) / tiles_per_p;           // projection
  const int j0 = (static_cast<int>(blockIdx.z) % tiles_per_p) * kDownRanks;
  const int npr = static_cast<int>(gridDim.z) * kDownRanks;            // nP * rp
  const int64_t kbeg = kc * kch;
  const int64_t kend = kbeg + kch < K ? kbeg + kch : K;
  const int nsteps = static_cast<int>((kend - kbeg) / 64);

  // rows past T (tokens) or r (ranks) read as zero
  const __amdgpu_buffer_rsrc_t rs_x = down_rsrc(in, ldin, t0, T);
  const __amdgpu_buffer_rsrc_t rs_p = down_rsrc(P.p[pj], K, j0, r);
  uint32_t xoff[4], poff[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i, row = id >> 3, q = id & 7;
    xoff[i] = static_cast<uint32_t>((row * ldin + q * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = tid + 256 * i, row = id >> 3, q = id & 7;
    poff[i] = static_cast<uint32_t>((row * K + q * 8) * 2);
  }
  // two register sets (steps alternate): two steps' loads in flight while a
  // third is computed
  u32x4 xv[2][4], pv[2][2];
  uint32_t kb[2][4];
  // keep bytes of this workgroup's token rows (rows past T read zero)
  const uint64_t kbytes = kMask ? static_cast<uint64_t>(T > t0 ? T - t0 : 0) * ldk : 0;
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(kMask ? keep + t0 * ldk : keep), 0,
      static_cast<int>(kbytes < 0x7fffffffu ? kbytes : 0x7fffffffu), kDownBufWord3);
  uint32_t koff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i, row = id >> 3, q = id & 7;
    koff[i] = static_cast<uint32_t>(row * ldk + q);
  }
  // Steps past the chunk (the loop runs an even number) read zeros through
  // past-the-end offsets and add nothing.
  auto load = [&](int st, auto setc) {
    constexpr int S = decltype(setc)::value;
    const uint32_t pe = st < nsteps ? 0u : kDownPastEnd;  // uniform
    const int so = static_cast<int>((kbeg + 64 * static_cast<int64_t>(st < nsteps ? st : 0)) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xv[S][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, xoff[i] | pe, so, 0));
    if constexpr (kMask) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kb[S][i] = __builtin_amdgcn_raw_buffer_load_b8(rs_k, koff[i] | pe, static_cast<int>(so / 16), 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
      pv[S][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_p, poff[i] | pe, so, 0));
  };
  auto store = [&](int b, auto setc) {
    constexpr int S = decltype(setc)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, row = id >> 3, q = id & 7;
      u32x4 v = xv[S][i];
      if constexpr (kMask) v = keep_bf16x8(v, kb[S][i]);
      *reinterpret_cast<u32x4*>(&s_x[b][row * 64 + down_swz(row, q) * 8]) = v;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + 256 * i, row = id >> 3, q = id & 7;
      *reinterpret_cast<u32x4*>(&s_p[b][row * 64 + down_swz(row, q) * 8]) = pv[S][i];
    }
  };
  auto frag = [&](const uint16_t* base, int row, int chunk) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(base + row * 64 + down_swz(row, chunk) * 8));
  };

  f32x16 acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  load(0, I0{});
  store(0, I0{});
  load(1, I1{});
  load(2, I0{});
  // step st: stage st % 2 holds step st; register set (st + 1) % 2 holds
  // step st + 1, goes to the other stage and is reloaded with step st + 3
  auto body = [&](int st, auto bc) {
    constexpr int b = decltype(bc)::value;
    using Next = std::integral_constant<int, b ^ 1>;
    __syncthreads();  // stage b complete, stage b ^ 1 free
    store(b ^ 1, Next{});
    load(st + 3, Next{});
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int chunk = 2 * j + h;
      const bf16x8 fp = frag(s_p[b], wn * 32 + r32, chunk);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp, frag(s_x[b], wm * 64 + c * 32 + r32, chunk), acc[c], 0, 0, 0);
    }
  };
  int sbeg = 0;
  __asm__ volatile("" : "+s"(sbeg));  // opaque start: no differently ordered peeled first pass
  for (int st = sbeg; st < nsteps; st += 2) {
    body(st, I0{});
    body(st + 1, I1{});
  }
  // D[rank][token]: lane holds token r32 of tile c, ranks 8 (e/4) + 4 h + e%4
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t t = t0 + wm * 64 + c * 32 + r32;
    if (t >= T) continue;
    float* dst = part + (kc * T + t) * npr + pj * rp + j0 + wn * 32 + 4 * h;
    // ranks >= r are zero and k_lora_down_fin does not read them: a store
    // whose four ranks all lie there is skipped
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (j0 + wn * 32 + 4 * h + 8 * g < r)
        *reinterpret_cast<f32x4v*>(dst + 8 * g) =
            f32x4v{acc[c][4 * g], acc[c][4 * g + 1], acc[c][4 * g + 2], acc[c][4 * g + 3]};
  }
}

// Sums the KC (<= kDownMaxKC) partials in order, scales and writes sU as
// bf16 hi/lo pairs:
//   pad    [T][2 rp]      hi in columns [0, rp), lo in [rp, 2 rp)
//   hilo_t [2 rp][ldt]    transposed; tokens [T, ldt) are zero
// One workgroup per 16 tokens x 64 ranks (4 per thread, the KC loads of one
// value issued together); the transposed copy goes through an LDS tile so
// both stores are coalesced.  Ranks r .. rp - 1 are written as zeros without
// reading the partials (k_lora_down_part leaves them unwritten).
constexpr int kDownMaxKC = 16;
__global__ __launch_bounds__(256) void k_lora_down_fin(const float* __restrict__ part, int64_t T, int KC,
                                                       int nP, int r, int rp, float scale,
                                                       uint16_t* __restrict__ pad,
                                                       int64_t ldpad, uint16_t* __restrict__ hilo_t,
                                                       int64_t ldt) {
  __shared__ uint32_t s_t[64][17];  // [rank][token] hi | lo << 16
  const int tid = threadIdx.x;
  const int64_t tb = static_cast<int64_t>(blockIdx.x) * 16;
  const int jb = static_cast<int>(blockIdx.y) * 64;
  // phase 1: thread -> rank jb + tid % 64, tokens tb + tid / 64 + 4 i
  const int jl = tid & 63;
  const int npr = nP * rp;
  // rank columns of this workgroup: projection pj, ranks jj .. jj + 63 (rp % 64 == 0)
  const int pj = jb / rp, jj = jb % rp;
  const bool live_rank = jj + jl < r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tl = (tid >> 6) + 4 * i;
    const int64_t t = tb + tl;
    const bool ok = t < T;
    float pv[kDownMaxKC];
#pragma unroll
    for (int q = 0; q < kDownMaxKC; ++q)
      pv[q] = (ok && live_rank && q < KC) ? part[(static_cast<int64_t>(q) * T + t) * npr + jb + jl] : 0.f;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kDownMaxKC; ++q) v += pv[q];
    v *= scale;
    const uint32_t hb = pack_bf16x2(v, 0.f) & 0xffffu;
    const float hi = __builtin_bit_cast(float, hb << 16);
    const uint32_t lb = pack_bf16x2(v - hi, 0.f) & 0xffffu;
    if (ok && pad != nullptr) {
      uint16_t* row = pad + t * ldpad + pj * 2 * rp + jj + jl;
      row[0] = static_cast<uint16_t>(hb);
      row[rp] = static_cast<uint16_t>(lb);
    }
    s_t[jl][tl] = hb | (lb << 16);  // tokens >= T hold zero
  }
  if (hilo_t == nullptr) return;
  __syncthreads();
  // phase 2: thread -> token tb + tid % 16, ranks jb + tid / 16 + 16 i
  const int tl = tid & 15;
  const int64_t t = tb + tl;
  if (t >= ldt) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = (tid >> 4) + 16 * i;
    const uint32_t v = s_t[j][tl];
    uint16_t* blk = hilo_t + static_cast<int64_t>(pj) * 2 * rp * ldt;  // projection pj's [2 rp][ldt]
    blk[static_cast<int64_t>(jj + j) * ldt + t] = static_cast<uint16_t>(v & 0xffffu);
    blk[static_cast<int64_t>(rp + jj + j) * ldt + t] = static_cast<uint16_t>(v >> 16);
  }
}

namespace {
// K-chunk length (a multiple of 64) for about 256 partial workgroups (at
// most kDownMaxKC chunks)
int64_t down_chunk(int64_t T, int64_t K, int64_t rp) {
  const int64_t tiles = ceil_div(T, kDownTok) * ceil_div(rp, kDownRanks);
  if (tiles <= 0 || K <= 0) return 64;  // no tokens: nothing is launched
  int64_t kc = ceil_div(256, tiles);
  const int64_t steps = K / 64;
  if (kc > kDownMaxKC) kc = kDownMaxKC;
  if (kc > steps) kc = steps;
  if (kc < 1) kc = 1;
  return ceil_div(steps, kc) * 64;
}
}  // namespace

size_t lora_down_part_bytes(int64_t T, int64_t K, int64_t nprp) {
  const int64_t kch = down_chunk(T, K, nprp);
  return static_cast<size_t>(ceil_div(K, kch) * T * nprp * 4);
}

hipError_t launch_lora_down(const uint16_t* in, int64_t ldin, int64_t T, int64_t K,
                            const uint16_t* const* P, int nP, int64_t r, float scale, uint16_t* pad,
                            int64_t ldpad, uint16_t* hilo_t, int64_t ldt, int64_t rp, float* part,
                            hipStream_t s, const uint8_t* keep, int64_t ldk) {
  if (T <= 0) return hipSuccess;
  if (nP < 1 || nP > kMaxProj) return hipErrorInvalidValue;
  // 32-bit buffer offsets: one tile's rows of `in` and P stay under 2^31 bytes
  if (kDownTok * ldin * 2 >= (int64_t(1) << 31) || kDownRanks * K * 2 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  DownFactors f{};
  for (int i = 0; i < nP; ++i) f.p[i] = P[i];
  const int64_t kch = down_chunk(T, K, nP * rp);
  const int64_t KC = ceil_div(K, kch);
  const dim3 grid(static_cast<uint32_t>(ceil_div(T, kDownTok)), static_cast<uint32_t>(KC),
                  static_cast<uint32_t>(nP * rp / kDownRanks));
  if (keep != nullptr) {
    if (kDownTok * ldk >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_lora_down_part<true>, grid, dim3(256), 0, s, in, ldin, T, K, f,
                       static_cast<int>(r), static_cast<int>(rp), kch, part, keep, ldk);
  } else {
    hipLaunchKernelGGL(k_lora_down_part<false>, grid, dim3(256), 0, s, in, ldin, T, K, f,
                       static_cast<int>(r), static_cast<int>(rp), kch, part, keep, ldk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tt = hilo_t != nullptr ? (ldt > T ? ldt : T) : T;
  const dim3 fgrid(static_cast<uint32_t>(ceil_div(tt, 16)), static_cast<uint32_t>(nP * rp / 64));
  hipLaunchKernelGGL(k_lora_down_fin, fgrid, dim3(256), 0, s, part, T, static_cast<int>(KC), nP,
                     static_cast<int>(r), static_cast<int>(rp), scale, pad, ldpad, hilo_t, ldt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// lora_grad: G[j][c] = sum_t Pt[j][t] Q[t][c] + sum_t Pt[rp+j][t] Q[t][c]
// (the hi and lo halves of the transposed rank factor) for ranks
// [j0, j0 + 32*JT), 128 columns per workgroup and a slice of tokens; slices
// add into the zeroed fp32 output with atomics.  Bound by streaming Q (dY or
// X) from HBM once.
//
// Per 64-token step the Q tile [64 t][128 c] and the Pt tile [64*JT rows][64 t]
// are loaded contiguously into registers one step ahead and written into a
// double-buffered LDS stage.  Q is transposed on the way: a thread holds two
// token rows of 8 columns, pairs them with v_perm and writes one dword
// (Q[2w][c], Q[2w+1][c]) per column; dword w of column c sits at
// 36c + (w ^ 4((c >> 4) & 7)), which makes both these writes and the MFMA
// fragment reads (8 tokens of one column) free of bank conflicts.  Wave w
// owns columns [32w, 32w + 32) and all JT rank tiles:
// v_mfma_f32_32x32x16_bf16 with Pt rows as A operand and Q columns as B.
// ---------------------------------------------------------------------------
constexpr int kGradCT = 128;    // columns per workgroup
constexpr int kGradPitch = 36;  // dwords per LDS row: 64 tokens + 8 padding
constexpr int kGradMaxJT = 4;   // rank tiles per launch (128 ranks)
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kPastEnd = 0x80000000u;

namespace {
__device__ __forceinline__ int grad_qslot(int c, int w) { return kGradPitch * c + (w ^ (4 * ((c >> 4) & 7))); }
}  // namespace

// kJC: output out[j*C + c] (else out[c*r + j]).  The MFMA orientation
// follows it, so a wave's 32 lanes always add to 32 consecutive floats.
// kMask: Q[t][c] counts only where bit c % 8 of keep[t * ldk + c / 8] is set;
// every output sum is multiplied by oscale.
// The workgroup of token slice y writes its sums (times oscale) to slice y of
// `part` ([slices][r * C] floats, each element written once per slice); a
// second launch adds the slices in order (k_sum_slices).
template <int JT, bool kJC, bool kMask>
__global__ __launch_bounds__(256) void k_lora_grad(const uint16_t* __restrict__ Pt, int64_t T,
                                                   int64_t ldt, int rp, const uint16_t* __restrict__ Q,
                                                   int64_t C, int64_t ldq, int r, int j0, int rproj,
                                                   float* __restrict__ part, int64_t TS,
                                                   const uint8_t* __restrict__ keep, int64_t ldk,
                                                   float oscale) {
  constexpr int kPRows = 64 * JT;  // hi rows [0, 32JT), lo rows [32JT, 64JT)
  __shared__ uint32_t s_q[2][kGradCT * kGradPitch];
  __shared__ uint32_t s_p[2][kPRows * kGradPitch];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kGradCT;
  const int64_t ts = static_cast<int64_t>(blockIdx.y) * TS;
  const int64_t te = ts + TS < T ? ts + TS : T;
  const int nsteps = static_cast<int>((te - ts + 63) / 64);

  // Q resource starts at this slice and ends at row T (or 2^31 - 1 bytes;
  // the host keeps a slice under 2^30 bytes)
  const uint64_t q_bytes = static_cast<uint64_t>(T - ts) * ldq * 2;
  const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Q + ts * ldq), 0, static_cast<int>(q_bytes < 0x7fffffffu ? q_bytes : 0x7fffffffu),
      kBufferWord3);
  // Pt holds ceil(r / rproj) stacked projections of 2 rp rows each
  const int nproj = (r + rproj - 1) / rproj;
  const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Pt), 0, static_cast<int>(static_cast<uint64_t>(nproj) * 2 * rp * ldt * 2),
      kBufferWord3);
  // Rank J of the call is rank J % rproj of projection J / rproj, whose hi and
  // lo rows are i 2rp + J % rproj and i 2rp + rp + J % rproj; ranks past r read zeros.
  int64_t prow_base[2 * JT];
#pragma unroll
  for (int i = 0; i < 2 * JT; ++i) {
    const int prow = (tid + 256 * i) >> 3;
    const int J = j0 + (prow < 32 * JT ? prow : prow - 32 * JT);
    const int pi = J / rproj, jl = J - pi * rproj;
    prow_base[i] = J < r ? static_cast<int64_t>(pi) * 2 * rp + jl + (prow < 32 * JT ? 0 : rp) : -1;
  }

  // Q staging items: column group cg (8 columns), token pairs tp and tp + 16
  const int cg = tid & 15, tp0 = tid >> 4;
  const bool col_ok = c0 + 8 * cg < C;
  // two register sets: the loads of step e go to set e % 2, so two steps'
  // loads are in flight while a third is computed
  u32x4 qv[2][4];
  uint32_t kb[2][4];
  u32x4 pv[2][2 * JT];
  const uint64_t kbytes = kMask ? static_cast<uint64_t>(T - ts) * ldk : 0;
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(kMask ? keep + ts * ldk : keep), 0,
      static_cast<int>(kbytes < 0x7fffffffu ? kbytes : 0x7fffffffu), kBufferWord3);
  // Every step issues its loads unconditionally; a step past the slice
  // (the loop runs an even number of steps) reads zeros and adds nothing.
  auto load = [&](int step, auto setc) {
    constexpr int S = decltype(setc)::value;
    const uint32_t pe = step < nsteps ? 0u : kPastEnd;  // uniform
    const int64_t t0 = ts + 64 * static_cast<int64_t>(step);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 - ts + 2 * (tp0 + 16 * (i >> 1)) + (i & 1);  // rows past T read as zero
      const uint32_t off = col_ok ? static_cast<uint32_t>((t * ldq + c0 + 8 * cg) * 2) | pe : kPastEnd;
      qv[S][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_q, off, 0, 0));
      if constexpr (kMask) {
        const uint32_t koff = col_ok ? static_cast<uint32_t>(t * ldk + (c0 + 8 * cg) / 8) | pe : kPastEnd;
        kb[S][i] = __builtin_amdgcn_raw_buffer_load_b8(rs_k, koff, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * JT; ++i) {
      const int id = tid + 256 * i, q = id & 7;
      const int64_t grow = prow_base[i];
      const int64_t tk = t0 + 8 * q;  // tokens in [T, ldt) are zero in Pt
      const uint32_t off = (tk < ldt && grow >= 0) ? static_cast<uint32_t>((grow * ldt + tk) * 2) | pe : kPastEnd;
      pv[S][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_p, off, 0, 0));
    }
  };
  auto store = [&](int buf, auto setc) {
    constexpr int S = decltype(setc)::value;
    if constexpr (kMask) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[S][i] = keep_bf16x8(qv[S][i], kb[S][i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 a = qv[S][2 * i], b = qv[S][2 * i + 1];
      const int w = tp0 + 16 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_q[buf][grad_qslot(8 * cg + 2 * e, w)] = perm(b[e], a[e], 0x05040100u);
        s_q[buf][grad_qslot(8 * cg + 2 * e + 1, w)] = perm(b[e], a[e], 0x07060302u);
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * JT; ++i) {
      const int id = tid + 256 * i, prow = id >> 3, q = id & 7;
      *reinterpret_cast<u32x4*>(&s_p[buf][kGradPitch * prow + 4 * q]) = pv[S][i];
    }
  };

  f32x16 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[jt][e] = 0.f;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  load(0, I0{});
  store(0, I0{});
  load(1, I1{});
  load(2, I0{});
  const int c = 32 * wv + r32;
  // step e: stage e % 2 holds step e; registers of set (e + 1) % 2 hold step
  // e + 1, are stored to the other stage and then reloaded with step e + 3
  auto body = [&](int step, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    using Next = std::integral_constant<int, buf ^ 1>;
    __syncthreads();  // stage buf complete, stage buf ^ 1 free
    store(buf ^ 1, Next{});
    load(step + 3, Next{});
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int w0 = 8 * s4 + 4 * h;
      const u32x4 qf = *reinterpret_cast<const u32x4*>(&s_q[buf][grad_qslot(c, w0)]);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 ph = *reinterpret_cast<const u32x4*>(&s_p[buf][kGradPitch * (32 * jt + r32) + w0]);
        const u32x4 pl = *reinterpret_cast<const u32x4*>(&s_p[buf][kGradPitch * (32 * JT + 32 * jt + r32) + w0]);
        if constexpr (kJC) {  // D[j][c]
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ph), as_bf16x8(qf), acc[jt], 0, 0, 0);
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pl), as_bf16x8(qf), acc[jt], 0, 0, 0);
        } else {  // D[c][j]
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qf), as_bf16x8(ph), acc[jt], 0, 0, 0);
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qf), as_bf16x8(pl), acc[jt], 0, 0, 0);
        }
      }
    }
  };
  int sbeg = 0;
  __asm__ volatile("" : "+s"(sbeg));  // opaque start: no differently ordered peeled first pass
  for (int step = sbeg; step < nsteps; step += 2) {
    body(step, I0{});
    body(step + 1, I1{});
  }
  float* const out = part + static_cast<int64_t>(blockIdx.y) * r * C;  // this slice's sums
  if constexpr (kJC) {
    // D[j][c]: lane holds column c, rows j = 8*(e/4) + 4*h + e%4
    const int64_t cc = c0 + c;
    if (cc >= C) return;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + 32 * jt + 8 * (e >> 2) + 4 * h + (e & 3);
        if (j < r) out[static_cast<int64_t>(j) * C + cc] = acc[jt][e] * oscale;
      }
  } else {
    // D[c][j]: lane holds rank j, rows c = 8*(e/4) + 4*h + e%4 of the wave's tile
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const int j = j0 + 32 * jt + r32;
      if (j >= r) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t cc = c0 + 32 * wv + 8 * (e >> 2) + 4 * h + (e & 3);
        if (cc < C) out[cc * r + j] = acc[jt][e] * oscale;
      }
    }
  }
}

// Token slices (multiples of 64 tokens) for about one workgroup per CU: more
// slices shorten each workgroup's stream but add partial sums (measured on
// the 8B-MLP shapes: 256-450 workgroups are fastest, 560 were 35% slower for
// 14336 columns, 512 were 30% slower for 4096).  The count depends on the
// shape only.
namespace {
int64_t grad_slice_tokens(int64_t T, int64_t C, int64_t ldq) {
  const int64_t ctiles = ceil_div(C, kGradCT);
  int64_t slices = ceil_div(256, ctiles);
  const int64_t max_slices = ceil_div(T, 64);
  if (slices > max_slices) slices = max_slices;
  if (slices < 1) slices = 1;
  // 32-bit buffer offsets: a slice of Q stays under 2^30 bytes
  const int64_t min_slices = ceil_div(T * ldq * 2, int64_t(1) << 30);
  if (slices < min_slices) slices = min_slices;
  return round_up(ceil_div(T, slices), 64);
}
}  // namespace

int64_t lora_grad_slices(int64_t T, int64_t C, int64_t ldq) {
  return T > 0 ? ceil_div(T, grad_slice_tokens(T, C, ldq)) : 0;
}

hipError_t launch_lora_grad(const uint16_t* Pt, int64_t T, int64_t ldt, int64_t rp, const uint16_t* Q,
                            int64_t C, int64_t ldq, int64_t r, float* part, bool out_jc, hipStream_t s,
                            const uint8_t* keep, int64_t ldk, float oscale, int64_t rproj) {
  if (T <= 0) return hipSuccess;
  if (rproj <= 0) rproj = r;
  if (ceil_div(r, rproj) * 2 * rp * ldt * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;  // Pt under 2^31 bytes
  if (keep != nullptr && T * ldk >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const int64_t TS = grad_slice_tokens(T, C, ldq);
  const int64_t slices = ceil_div(T, TS);
  const int64_t ctiles = ceil_div(C, kGradCT);
  const dim3 grid(static_cast<uint32_t>(ctiles), static_cast<uint32_t>(slices));
  const int irp = static_cast<int>(rp), ir = static_cast<int>(r);
  for (int64_t j0 = 0; j0 < r; j0 += 32 * kGradMaxJT) {
    const int64_t left = r - j0;
    const int jt = static_cast<int>(ceil_div(left < 32 * kGradMaxJT ? left : 32 * kGradMaxJT, 32));
    const int ij0 = static_cast<int>(j0);
#define QLORA_GRAD(JTV, JC, MK)                                                                      \
  hipLaunchKernelGGL((k_lora_grad<JTV, JC, MK>), grid, dim3(256), 0, s, Pt, T, ldt, irp, Q, C, ldq, ir, ij0, \
                     static_cast<int>(rproj), part, TS, keep, ldk, oscale)
    if (keep != nullptr) {  // the masked operand is X: dA, out_jc
      if (jt <= 1) QLORA_GRAD(1, true, true);
      else if (jt <= 2) QLORA_GRAD(2, true, true);
      else QLORA_GRAD(4, true, true);
    } else if (out_jc) {
      if (jt <= 1) QLORA_GRAD(1, true, false);
      else if (jt <= 2) QLORA_GRAD(2, true, false);
      else QLORA_GRAD(4, true, false);
    } else {
      if (jt <= 1) QLORA_GRAD(1, false, false);
      else if (jt <= 2) QLORA_GRAD(2, false, false);
      else QLORA_GRAD(4, false, false);
    }
#undef QLORA_GRAD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
namespace {
// dst row i = [src row i zero-padded to Cp | the same again] (src transposed
// when `transpose`: row i of src^T is column i of src [C][R]); element idx of R * Cp
__device__ __forceinline__ void pad_elem(int64_t idx, const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                         int transpose, uint16_t* __restrict__ dst, int64_t Cp, int64_t ldd) {
  if (idx >= R * Cp) return;
  const int64_t i = idx / Cp, j = idx % Cp;
  uint16_t v = 0;
  if (j < C) v = transpose ? src[j * R + i] : src[i * C + j];
  dst[i * ldd + j] = v;
  dst[i * ldd + Cp + j] = v;
}

// dst[c][r] = src[r][c] for src [R][C]; element idx of R * C
__device__ __forceinline__ void transpose_elem(int64_t idx, const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                               uint16_t* __restrict__ dst) {
  if (idx >= R * C) return;
  const int64_t c = idx / R, rr = idx % R;
  dst[idx] = src[rr * C + c];
}
}  // namespace

__global__ __launch_bounds__(256) void k_pad_bf16(const uint16_t* __restrict__ src, int64_t R,
                                                  int64_t C, int transpose,
                                                  uint16_t* __restrict__ dst, int64_t Cp, int64_t ldd) {
  pad_elem(static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x, src, R, C, transpose, dst, Cp, ldd);
}

hipError_t launch_pad_bf16(const uint16_t* src, int64_t R, int64_t C, bool transpose, uint16_t* dst,
                           int64_t Cp, int64_t ldd, hipStream_t s) {
  hipLaunchKernelGGL(k_pad_bf16, dim3(static_cast<uint32_t>(ceil_div(R * Cp, 256))), dim3(256), 0,
                     s, src, R, C, transpose ? 1 : 0, dst, Cp, ldd);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src, int64_t R,
                                                        int64_t C, uint16_t* __restrict__ dst) {
  transpose_elem(static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x, src, R, C, dst);
}

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst,
                                 hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_bf16, dim3(static_cast<uint32_t>(ceil_div(R * C, 256))), dim3(256),
                     0, s, src, R, C, dst);
  return hipGetLastError();
}

// launch_pad_bf16 (not transposed) for up to kMaxProj sources in one launch:
// job i takes blocks [blk0[i], blk0[i + 1])
struct PadJobs {
  const uint16_t* src[kMaxProj];
  uint16_t* dst[kMaxProj];
  int64_t R[kMaxProj];
  int64_t blk0[kMaxProj + 1];
  int n;
};

__global__ __launch_bounds__(256) void k_pad_many(PadJobs J, int64_t C, int64_t Cp, int64_t ldd) {
  const int64_t blk = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int q = 1; q < kMaxProj; ++q)
    if (q < J.n && blk >= J.blk0[q]) i = q;
  pad_elem((blk - J.blk0[i]) * 256 + threadIdx.x, J.src[i], J.R[i], C, 0, J.dst[i], Cp, ldd);
}

hipError_t launch_pad_many(const uint16_t* const* src, const int64_t* R, uint16_t* const* dst, int n, int64_t C,
                           int64_t Cp, int64_t ldd, hipStream_t s) {
  if (n < 1 || n > kMaxProj) return hipErrorInvalidValue;
  if (n == 1) return launch_pad_bf16(src[0], R[0], C, false, dst[0], Cp, ldd, s);
  PadJobs J{};
  J.n = n;
  J.blk0[0] = 0;
  for (int i = 0; i < n; ++i) {
    J.src[i] = src[i];
    J.dst[i] = dst[i];
    J.R[i] = R[i];
    J.blk0[i + 1] = J.blk0[i] + ceil_div(R[i] * Cp, 256);
  }
  if (J.blk0[n] == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pad_many, dim3(static_cast<uint32_t>(J.blk0[n])), dim3(256), 0, s, J, C, Cp, ldd);
  return hipGetLastError();
}

// The backward's two rank-factor copies in one launch: the first tb blocks
// transpose B [out][r] into bt [r][out], the rest pad A [r][in] transposed
// into a_t_pad [in][ldd] (A^T | A^T, each zero-padded to rp columns).
__global__ __launch_bounds__(256) void k_factor_prep(const uint16_t* __restrict__ B, int64_t out, int64_t r,
                                                     uint16_t* __restrict__ bt, int64_t tb,
                                                     const uint16_t* __restrict__ A, int64_t in,
                                                     uint16_t* __restrict__ a_t_pad, int64_t rp, int64_t ldd) {
  const int64_t blk = blockIdx.x;
  if (blk < tb)
    transpose_elem(blk * 256 + threadIdx.x, B, out, r, bt);
  else
    pad_elem((blk - tb) * 256 + threadIdx.x, A, in, r, 1, a_t_pad, rp, ldd);
}

hipError_t launch_factor_prep(const uint16_t* B, int64_t out, int64_t r, uint16_t* bt, const uint16_t* A,
                              int64_t in, uint16_t* a_t_pad, int64_t rp, int64_t ldd, hipStream_t s) {
  const int64_t tb = ceil_div(out * r, 256), pb = ceil_div(in * rp, 256);
  hipLaunchKernelGGL(k_factor_prep, dim3(static_cast<uint32_t>(tb + pb)), dim3(256), 0, s, B, out, r, bt, tb, A,
                     in, a_t_pad, rp, ldd);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ dst, int64_t n, float v) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx < n) dst[idx] = v;
}

hipError_t launch_fill_f32(float* dst, int64_t n, float v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_f32, dim3(static_cast<uint32_t>(ceil_div(n, 256))), dim3(256), 0, s,
                     dst, n, v);
  return hipGetLastError();
}

// Several buffers set to v in one launch (a small kernel costs its launch
// more than its work): buffer b covers workgroups [first[b], first[b + 1]).
struct FillList {
  float* dst[kMaxFill];
  int64_t n[kMaxFill];
  int64_t first[kMaxFill + 1];
  int count;
};

__global__ __launch_bounds__(256) void k_fill_many_f32(FillList L, float v) {
  const int64_t wg = blockIdx.x;
  int b = 0;
#pragma unroll
  for (int i = 1; i < kMaxFill; ++i)
    if (i < L.count && wg >= L.first[i]) b = i;
  const int64_t idx = (wg - L.first[b]) * 256 + threadIdx.x;
  if (idx < L.n[b]) L.dst[b][idx] = v;
}

hipError_t launch_fill_many_f32(float* const* dst, const int64_t* n, int count, float v, hipStream_t s) {
  if (count < 1 || count > kMaxFill) return hipErrorInvalidValue;
  FillList L{};
  L.count = count;
  int64_t wgs = 0;
  for (int i = 0; i < count; ++i) {
    L.dst[i] = dst[i];
    L.n[i] = n[i];
    L.first[i] = wgs;
    wgs += ceil_div(n[i], 256);
  }
  L.first[count] = wgs;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_many_f32, dim3(static_cast<uint32_t>(wgs)), dim3(256), 0, s, L, v);
  return hipGetLastError();
}

// out_b[i] = sum over z = 0, 1, ... of part_b[z * stride_b + i] for each job b,
// the slices added in order (bit-reproducible); 4 floats per thread, n_b % 4 == 0.
struct SumList {
  const float* part[kMaxFill];
  float* out[kMaxFill];
  int64_t n[kMaxFill];
  int64_t stride[kMaxFill];  // elements between consecutive slices
  int64_t first[kMaxFill + 1];
  int slices[kMaxFill];
  int count;
};

__global__ __launch_bounds__(256) void k_sum_slices(SumList L) {
  const int64_t wg = blockIdx.x;
  int b = 0;
#pragma unroll
  for (int i = 1; i < kMaxFill; ++i)
    if (i < L.count && wg >= L.first[i]) b = i;
  const float* part = L.part[0];
  float* out = L.out[0];
  int64_t n = L.n[0], first = L.first[0], stride = L.stride[0];
  int S = L.slices[0];
#pragma unroll
  for (int i = 1; i < kMaxFill; ++i)
    if (i == b) {
      part = L.part[i]; out = L.out[i]; n = L.n[i]; first = L.first[i]; S = L.slices[i]; stride = L.stride[i];
    }
  const int64_t idx = ((wg - first) * 256 + threadIdx.x) * 4;
  if (idx >= n) return;
  // eight slices' loads in flight at a time, added in slice order
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < S; z0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = z0 + u < S ? *reinterpret_cast<const f32x4*>(part + (z0 + u) * stride + idx) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < S) acc += v[u];
  }
  *reinterpret_cast<f32x4*>(out + idx) = acc;
}

hipError_t launch_sum_slices(const float* const* part, const int* slices, const int64_t* n, float* const* out,
                             int count, hipStream_t s, const int64_t* stride) {
  if (count < 1 || count > kMaxFill) return hipErrorInvalidValue;
  SumList L{};
  L.count = count;
  int64_t wgs = 0;
  for (int i = 0; i < count; ++i) {
    if (n[i] % 4 != 0 || slices[i] < 1) return hipErrorInvalidValue;
    L.part[i] = part[i];
    L.out[i] = out[i];
    L.n[i] = n[i];
    L.stride[i] = stride != nullptr ? stride[i] : n[i];
    if (L.stride[i] % 4 != 0 || L.stride[i] < n[i]) return hipErrorInvalidValue;
    L.slices[i] = slices[i];
    L.first[i] = wgs;
    wgs += ceil_div(n[i], 1024);
  }
  L.first[count] = wgs;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sum_slices, dim3(static_cast<uint32_t>(wgs)), dim3(256), 0, s, L);
  return hipGetLastError();
}

}  // namespace qlora
