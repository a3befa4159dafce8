// k_decode.hip -- fused QLoRA linear forward for small token counts
// (T <= 16, r <= 64), bound by the packed-nibble weight stream.
//
//   Y = X W_hat^T + s (X A^T) B^T     (paperclase lesson "QLoRA", Parte 4)
//
// Decomposition.  Workgroup b owns the 16 output rows [16b, 16b + 16) over
// the whole reduction dimension, so its part of Y is finished inside the
// workgroup: no partial sums and no synchronisation cross workgroups.  With
// out = 4096 the grid is 256 workgroups, one per CU, each streaming 16 rows x
// in of codes.  Up to one workgroup per CU (and r <= 16) every workgroup
// computes the small U = X A^T itself from X and A, which stay resident in
// L2, and the call is one launch with no workspace.  With more workgroups, or
// r > 16, reading all of A in every workgroup costs more than a second
// launch: k_decode_u computes U once into the workspace first.
//
// Eight waves split the 64-weight blocks of the 16 rows into contiguous
// ranges, walked in chunks of four blocks (256 k).  In a chunk, lane
// (n = l%16, g = l/16) owns block 4c+g of row n: 32 code bytes, the block's
// 16-entry bf16 table, then 8 dwords of codes through the v_perm lookup into
// the A operand of v_mfma_f32_16x16x32_bf16 (16 rows x 16 tokens x 32 k).
// The B operand is token n's matching 8 activations.  The same activation
// fragments also meet A's rows in a second MFMA (16 ranks x 16 tokens),
// which accumulates this wave's share of U.
//
// Activations and A rows are 16 rows at a large stride; loading MFMA
// fragments straight from memory puts 16 rows at one offset into every
// instruction, which the memory pipeline serves several times slower than
// contiguous requests.  So each wave loads its chunk of X (T tokens x 512 B)
// and of A (16 ranks x 512 B) contiguously, two rows per instruction, into
// a private LDS tile, then reads the fragments back (padded rows, below).
// Two chunks' global loads (codes, X, A) are in flight at a time.
//
// Epilogue: the eight waves' fp32 accumulators of the base product and of U
// meet in LDS; Y = base + s U B^T is rounded to bf16 once.
#include <type_traits>

#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 16;
constexpr int kCodeSlots = 16 * 8;   // 16 rows x 8 pieces: one chunk of codes (2 KB)
// Split kernel tiles: rows of 32 pieces padded to 33, so piece p of row t
// sits at slot 33 t + p.  A fragment read (16 rows at one piece) then falls
// on 16 distinct 4-bank groups, and every lane's slots differ by constants,
// which the LDS instructions take as immediate offsets.
constexpr int kPitch = 33;
constexpr int kPadSlots = 16 * kPitch;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource, 32-bit data format
constexpr int kStream = 2;               // cache policy nt: streamed once
constexpr uint32_t kPastEnd = 0x80000000u;  // past every buffer (all < 2^31 bytes)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// This lane's block of codes in one chunk, with its absmax code and scale.
struct CodeStage {
  u32x4 c0, c1;
  uint32_t q;
  float sc;
};
}  // namespace

// ---------------------------------------------------------------------------
// r <= 16: the same decomposition with the two kinds of work on different
// waves.  Waves 0-3 stream codes and run the dequantize + base MFMA (vector
// ALU bound); waves 4-7 load X and A and run the U MFMA (bound by the
// load-address unit).  Wave w and wave w + 4 share a quarter of the blocks
// of each row and sit on the same SIMD, so the hardware overlaps one pair
// member's address-unit stalls with the other's vector arithmetic.  The X
// tile of a chunk is written by the U wave and read by both, double-buffered
// by chunk parity with one workgroup barrier per chunk.
//
// Two chunks' loads are in flight per wave.  That only holds if the wait
// counts the compiler derives at each consumer allow the younger chunk to
// stay outstanding, which needs one fixed issue order:
//   - every load of a chunk step is issued unconditionally (offsets of rows,
//     pieces or chunks that do not exist are pushed past the buffer end and
//     read zeros without touching memory), so no branch decides whether a
//     load exists;
//   - the steps run from chunk -2: the first two only issue loads, so each
//     register set is filled by the same instructions every time;
//   - with NS > 0 the step sequence is fully unrolled (NS steps, compile-time
//     register sets, no loop-carried copies that would force a full wait);
//     NS = 0 keeps a loop whose start is hidden from the optimizer so the
//     loading steps are not peeled off into a differently ordered prologue.
// XP = token-row pairs of the X tile (T <= 2 XP).  kFull: every wave's
// block range is whole chunks (in % 1024 == 0), so no load needs a per-lane
// range test; a step past the range reads through an empty buffer resource.
// Each load's per-lane offset (row and piece) is fixed for the whole kernel
// and the chunk's position goes into the scalar offset.
// ---------------------------------------------------------------------------
// Several projections that share X (q|k|v) run as one launch: workgroups
// [wg0[p], wg0[p + 1]) take projection p's rows, written to columns
// [col0[p], col0[p] + out[p]) of Y.
// kPreU: U = X A^T of every projection was computed beforehand
// (k_decode_u, fp32 [n][T][r] at Upre, r <= 64): the U waves then only
// stage X, and no workgroup reads A.  Otherwise r <= 16 and each workgroup
// computes U itself.
template <int XP, int NS, bool kFull, bool kPreU>
__global__ __launch_bounds__(kThreads) void k_decode_fwd_split(DecodeSet P, int64_t in,
                                                               const uint16_t* __restrict__ X, int T, int r,
                                                               float s, int64_t ldy,
                                                               const float* __restrict__ Upre) {
  // this workgroup's projection (uniform)
  int pj = 0;
#pragma unroll
  for (int i = 1; i < kMaxProj; ++i)
    if (i < P.n && static_cast<int>(blockIdx.x) >= P.wg0[i]) pj = i;
  const uint8_t* __restrict__ codes = P.proj[pj].codes;
  const uint8_t* __restrict__ absmax_q = P.proj[pj].absmax_q;
  const float* __restrict__ scale = P.proj[pj].scale;
  const uint16_t* __restrict__ A = P.proj[pj].A;
  const uint16_t* __restrict__ B = P.proj[pj].B;
  const int64_t out = P.proj[pj].out;
  uint16_t* __restrict__ Y = P.Y + P.col0[pj];
  const int wg = static_cast<int>(blockIdx.x) - P.wg0[pj];  // row block within the projection
  constexpr int kPairs = kWaves / 2;
  __shared__ u32x4 s_x[kPairs][2][kPadSlots];    // X tiles by chunk parity
  __shared__ u32x4 s_a[kPairs][kPadSlots];       // A tile of each U wave
  __shared__ u32x4 s_codes[kPairs][kCodeSlots];  // codes of each dequantize wave
  // The epilogue's arrays reuse the X tiles' memory once the chunk steps
  // are done, which keeps the kPreU kernel under half the CU's LDS (two
  // workgroups per CU).
  constexpr int kRU = kPreU ? 64 : 16;  // ranks held by the epilogue
  static_assert(sizeof(f32x4) * kWaves * 64 + sizeof(float) * (kRows + 16) * (kRU + 1) <= sizeof(s_x));
  f32x4(*s_acc)[64] = reinterpret_cast<f32x4(*)[64]>(&s_x[0][0][0]);
  float(*s_b)[kRU + 1] = reinterpret_cast<float(*)[kRU + 1]>(&s_acc[kWaves][0]);
  float(*s_u)[kRU + 1] = s_b + kRows;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar wave index
  const bool dq_wave = wv < kPairs;
  const int qtr = dq_wave ? wv : wv - kPairs;
  const int n = lane & 15, g = lane >> 4;
  const int half = lane >> 5, piece = lane & 31;
  const int64_t r0 = static_cast<int64_t>(wg) * kRows;
  const int64_t nb = in / 64;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  const int bw0 = static_cast<int>(nb * qtr / kPairs), bw1 = static_cast<int>(nb * (qtr + 1) / kPairs);
  const int nch = (bw1 - bw0 + 3) / 4;
  // steps every wave runs (the same count for all: one barrier each), even
  const int nsteps = NS > 0 ? NS : static_cast<int>(round_up((ceil_div(nb, kPairs) + 3) / 4, 2));
  const uint32_t row = static_cast<uint32_t>(r0) + n;
  const uint32_t inu = static_cast<uint32_t>(in), nbu = static_cast<uint32_t>(nb);

  const uint32_t wbytes = static_cast<uint32_t>(static_cast<uint64_t>(out) * in / 2);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B), 0, static_cast<int>(static_cast<uint32_t>(out) * r * 2), kBufferWord3);

  // B rows of this workgroup (16 x kRU values, ranks >= r zero), converted
  // in the epilogue; every thread loads (past the end where there is no
  // value), so no branch makes the compiler wait for this load before the
  // main loop
  constexpr int kBLoads = kRows * kRU / kThreads > 0 ? kRows * kRU / kThreads : 1;
  uint32_t braw[kBLoads];
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int idx = tid + kThreads * i, rr = idx / kRU, j = idx % kRU;
    const uint32_t off = (rr < kRows && j < r) ? ((static_cast<uint32_t>(r0) + rr) * r + j) * 2 : kPastEnd;
    braw[i] = __builtin_amdgcn_raw_buffer_load_b16(rs_b, off, 0, 0);
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // runs step(c, d) for c = -2 .. nsteps - 1, d = c & 1 a compile-time index
  auto run_steps = [&](auto&& step) {
    if constexpr (NS > 0) {
      // With 8 or more token rows the U waves' loads (X and A, L2 resident)
      // go out first: the dequantize waves issue their codes (HBM) once the
      // U waves have issued their first two chunks.
      if constexpr (XP >= 4) {
        if (dq_wave) __syncthreads();
      }
      step(-2, std::integral_constant<int, 0>{});
      step(-1, std::integral_constant<int, 1>{});
      if constexpr (XP >= 4) {
        if (!dq_wave) __syncthreads();
      }
#pragma unroll
      for (int c = 0; c < NS; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        step(c + 1, std::integral_constant<int, 1>{});
      }
    } else {
      int cstart = -2;
      __asm__ volatile("" : "+s"(cstart));  // opaque start: the loading steps stay in the loop
      for (int c = cstart; c < nsteps; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        step(c + 1, std::integral_constant<int, 1>{});
      }
    }
  };

  if (dq_wave) {
    // ------------------------------------------------ dequantize waves
    // the vector-ALU-bound waves issue ahead of the U wave on their SIMD
    __builtin_amdgcn_s_setprio(1);
    u32x4* tc = s_codes[qtr];
    CodeStage cs[2];
    // Per-lane offsets of the code rows and absmax bytes.  With whole
    // chunks the chunk's position is a scalar offset (every byte a live step
    // reads lies in its row, so the per-lane offset alone keeps the bounds
    // check meaningful) and a step past the range reads through empty buffer
    // resources.  Otherwise a partial last chunk reads past its row's end,
    // so the whole offset stays per lane.
    const uint32_t rl = static_cast<uint32_t>(r0) + (lane >> 3);
    const uint32_t cvo0 = rl * (inu / 2) + 16 * (lane & 7), cvo1 = cvo0 + 8 * (inu / 2);
    const uint32_t qvo = row * nbu + static_cast<uint32_t>(g);
    const int cbytes = static_cast<int>(wbytes), qbytes = static_cast<int>(wbytes / 32);
    const int sbytes = static_cast<int>((wbytes + 8191) / 8192 * 4);
    auto load_codes = [&](CodeStage& st, int c) {
      const int blk0 = bw0 + 4 * c;  // the chunk's first block in the row (uniform)
      if constexpr (kFull) {
        const bool live = c < nch;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(codes), 0, live ? cbytes : 0, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(absmax_q), 0, live ? qbytes : 0, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(scale), 0, live ? sbytes : 0, kBufferWord3);
        st.c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, cvo0, 32 * blk0, kStream));
        st.c1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, cvo1, 32 * blk0, kStream));
        st.q = __builtin_amdgcn_raw_buffer_load_b8(rq, qvo, blk0, 0);
        const uint32_t bi = qvo + static_cast<uint32_t>(blk0);
        st.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, (bi >> 8) * 4, 0, 0));
      } else {
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(codes), 0, cbytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(absmax_q), 0, qbytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(scale), 0, sbytes, kBufferWord3);
        const uint32_t pe = c < nch ? 0u : kPastEnd;  // uniform, OR-ed into the offsets
        const uint32_t cb = 32 * static_cast<uint32_t>(blk0);
        st.c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, (cvo0 + cb) | pe, 0, kStream));
        st.c1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, (cvo1 + cb) | pe, 0, kStream));
        const uint32_t bi = qvo + static_cast<uint32_t>(blk0);
        st.q = __builtin_amdgcn_raw_buffer_load_b8(rq, bi | pe, 0, 0);
        st.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, ((bi >> 8) * 4) | pe, 0, 0));
      }
    };
    auto step = [&](int c, auto d) {
      CodeStage& st = cs[decltype(d)::value];
      u32x4 cc0 = zero4, cc1 = zero4;
      float ah = 0.f;
      if (c >= 0) {
        // codes to their owners: row n, block g = pieces 2g, 2g + 1
        const int m = lane >> 3, pc = lane & 7;
        tc[8 * m + (pc ^ ((m >> 1) & 7))] = st.c0;
        tc[8 * (m + 8) + (pc ^ (((m + 8) >> 1) & 7))] = st.c1;
        cc0 = tc[8 * n + ((2 * g) ^ ((n >> 1) & 7))];
        cc1 = tc[8 * n + ((2 * g + 1) ^ ((n >> 1) & 7))];
        ah = dq_absmax(st.q, st.sc);
      }
      load_codes(st, c + 2);
      if (c >= 0) {
        __syncthreads();  // X(c) is in its tile
        const u32x4* tx = s_x[qtr][decltype(d)::value] + kPitch * n + 8 * g;
        const Nf4Table tab = make_table(ah);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4 xf = tx[j];
          const uint32_t cw = j < 4 ? cc0[j] : cc1[j - 4];
          uint32_t w[4];
          lookup8(tab, cw, w);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}),
                                                        as_bf16x8(xf), acc, 0, 0, 0);
        }
      }
    };
    run_steps(step);
  } else {
    // ------------------------------------------------ U waves
    u32x4* ta = s_a[qtr];
    u32x4 xs[2][XP], as[2][8];
    // lane (half, piece) of row pair i loads piece `piece` (16 B) of row
    // 2 i + half of the chunk; rows >= T (X) or >= r (A) lie past the buffer
    uint32_t voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) voff[i] = ((2 * i + half) * inu + 8 * piece) * 2;
    auto load_rows = [&](auto& reg, const uint16_t* base, uint32_t bytes, auto npairs, int c) {
      const int kb = (bw0 + 4 * c) * 128;  // the chunk's first byte in a row (uniform)
      if constexpr (kFull) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base), 0, c < nch ? static_cast<int>(bytes) : 0, kBufferWord3);
#pragma unroll
        for (int i = 0; i < decltype(npairs)::value; ++i)
          reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], kb, 0));
      } else {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base), 0, static_cast<int>(bytes), kBufferWord3);
        // valid k of this chunk: 256, fewer in a partial last chunk, none past the range
        const int lim = c < nch ? min((bw1 - bw0 - 4 * c) * 64, 256) : 0;
#pragma unroll
        for (int i = 0; i < decltype(npairs)::value; ++i) {
          const uint32_t off = 8 * piece < lim ? voff[i] : kPastEnd;
          reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, kb, 0));
        }
      }
    };
    const uint32_t xbytes = static_cast<uint32_t>(T) * inu * 2, abytes = static_cast<uint32_t>(r) * inu * 2;
    const int wslot = kPitch * half + piece;  // + 2 kPitch i for row pair i
    // token rows that no chunk writes stay zero in both X tiles
#pragma unroll
    for (int i = XP; i < 8; ++i) {
      s_x[qtr][0][wslot + 2 * kPitch * i] = zero4;
      s_x[qtr][1][wslot + 2 * kPitch * i] = zero4;
    }
    auto step = [&](int c, auto d) {
      constexpr int kD = decltype(d)::value;
      u32x4* tx = s_x[qtr][kD];
      if (c >= 0) {
#pragma unroll
        for (int i = 0; i < XP; ++i) tx[wslot + 2 * kPitch * i] = xs[kD][i];
        if constexpr (!kPreU) {
#pragma unroll
          for (int i = 0; i < 8; ++i) ta[wslot + 2 * kPitch * i] = as[kD][i];
        }
      }
      load_rows(xs[kD], X, xbytes, std::integral_constant<int, XP>{}, c + 2);
      if constexpr (!kPreU)
        load_rows(as[kD], A, abytes, std::integral_constant<int, 8>{}, c + 2);  // ranks >= r read zeros
      if constexpr (kPreU) {
        if (c >= 0) __syncthreads();  // X(c) is in tx for the partner
      } else if (c >= 0) {
        __syncthreads();  // X(c) is in tx for the partner
        const u32x4* fx = tx + kPitch * n + 8 * g;
        const u32x4* fa = ta + kPitch * n + 8 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4 xf = fx[j];
          const u32x4 af = fa[j];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(xf), acc, 0, 0, 0);
        }
      }
    };
    run_steps(step);
  }

  // ---------------- epilogue: waves 0-3 hold D[row][token], 4-7 D[rank][token]
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();  // every wave is done with the X tiles
  s_acc[wv][lane] = acc;
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int idx = tid + kThreads * i;
    if (idx < kRows * kRU) s_b[idx / kRU][idx % kRU] = __builtin_bit_cast(float, braw[i] << 16);
  }
  if constexpr (kPreU) {
    const float* __restrict__ up = Upre + static_cast<int64_t>(pj) * T * r;
    for (int idx = tid; idx < 16 * kRU; idx += kThreads) {
      const int t = idx / kRU, j = idx % kRU;
      s_u[t][j] = (t < T && j < r) ? up[t * r + j] : 0.f;
    }
  }
  __syncthreads();
  // Y = base + s U B^T in wave 0: B rows x (s U)^T as bf16 hi + lo on MFMA
  // (32 ranks per pair of MFMAs; ranks >= r are zero in U and B), added to
  // the dequantize waves' partials of the same four outputs in a fixed
  // order; lane (n, g) holds rows 4 g .. + 3 of token n
  if (wv == 0) {
    // U[t][j]: up front in s_u, or the U waves' partials D[j][t] (lane
    // 16 (j / 4) + t, element j % 4 of each), added in a fixed order
    auto u_at = [&](int t, int j) {
      if constexpr (kPreU) {
        return s_u[t][j];
      } else {
        float u = 0.f;
#pragma unroll
        for (int w = kPairs; w < kWaves; ++w) u += s_acc[w][16 * (j >> 2) + t][j & 3];
        return u;
      }
    };
    f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < (kRU + 31) / 32; ++ks) {
      const int j0 = 32 * ks + 8 * g;
      uint32_t bq[4] = {0u, 0u, 0u, 0u}, hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
      if (j0 < kRU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // B values are bf16 held as fp32: their top halves are exact
          bq[e] = (__builtin_bit_cast(uint32_t, s_b[n][j0 + 2 * e]) >> 16) |
                  (__builtin_bit_cast(uint32_t, s_b[n][j0 + 2 * e + 1]) & 0xffff0000u);
          const float u0 = s * u_at(n, j0 + 2 * e), u1 = s * u_at(n, j0 + 2 * e + 1);
          hi[e] = pack_bf16x2(u0, u1);
          lo[e] = pack_bf16x2(u0 - __builtin_bit_cast(float, hi[e] << 16),
                              u1 - __builtin_bit_cast(float, hi[e] & 0xffff0000u));
        }
      }
      const bf16x8 fb = as_bf16x8(u32x4{bq[0], bq[1], bq[2], bq[3]});
      lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, as_bf16x8(u32x4{hi[0], hi[1], hi[2], hi[3]}), lsum, 0, 0, 0);
      lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]}), lsum, 0, 0, 0);
    }
    f32x4 base = s_acc[0][lane];
#pragma unroll
    for (int w = 1; w < kPairs; ++w) {
      const f32x4 pw = s_acc[w][lane];
      base = f32x4{base[0] + pw[0], base[1] + pw[1], base[2] + pw[2], base[3] + pw[3]};
    }
    if (n < T)
      *reinterpret_cast<u32x2*>(Y + static_cast<int64_t>(n) * ldy + r0 + 4 * g) =
          u32x2{pack_bf16x2(base[0] + lsum[0], base[1] + lsum[1]), pack_bf16x2(base[2] + lsum[2], base[3] + lsum[3])};
  }
}

// U = X A^T for the small-token forward, computed once per call instead of
// by every workgroup: U[p][t][k] = sum_i X[t][i] A_p[k][i] in fp32 (the
// scale s is applied by the consumer).  One workgroup per (rank k, token t,
// projection p); its 256 threads each take 16-byte pieces of the two rows at
// a stride of 4 KB, then the partial sums meet in LDS.
__global__ __launch_bounds__(256) void k_decode_u(DecodeSet P, int64_t in, const uint16_t* __restrict__ X,
                                                  int T, int r, float* __restrict__ U) {
  const int k = blockIdx.x, t = blockIdx.y, pj = blockIdx.z;
  const u32x4* __restrict__ xr = reinterpret_cast<const u32x4*>(X + static_cast<int64_t>(t) * in);
  const u32x4* __restrict__ ar = reinterpret_cast<const u32x4*>(P.proj[pj].A + static_cast<int64_t>(k) * in);
  const int npieces = static_cast<int>(in / 8);
  float sum = 0.f;
  for (int i = threadIdx.x; i < npieces; i += 256) {
    const u32x4 xv = xr[i], av = ar[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sum = fmaf(__builtin_bit_cast(float, xv[e] << 16), __builtin_bit_cast(float, av[e] << 16), sum);
      sum = fmaf(__builtin_bit_cast(float, xv[e] & 0xffff0000u), __builtin_bit_cast(float, av[e] & 0xffff0000u), sum);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  __shared__ float s_part[4];
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0)
    U[(static_cast<int64_t>(pj) * T + t) * r + k] = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
}

bool decode_fits(int64_t T, int64_t in, int64_t out, int64_t r) {
  // 32-bit buffer offsets: codes and every row of X and A stay below 2^31 bytes
  return T >= 1 && T <= kDecodeMaxT && r >= 1 && r <= kDecodeMaxRank && out % kRows == 0 &&
         in % 64 == 0 && in <= (int64_t(1) << 24) && out * in < (int64_t(1) << 32);
}

bool decode_pre_u(int n, const int64_t* outs, int64_t r) {
  int64_t rows = 0;
  for (int i = 0; i < n; ++i) rows += outs[i];
  return r > 16 || rows / kRows > kDecodeFusedMaxWgs;
}

hipError_t launch_decode_u(const DecodeSet& set, int64_t in, const uint16_t* X, int64_t T, int64_t r,
                           float* u_ws, hipStream_t st) {
  hipLaunchKernelGGL(k_decode_u, dim3(static_cast<uint32_t>(r), static_cast<uint32_t>(T), set.n), dim3(256), 0,
                     st, set, in, X, static_cast<int>(T), static_cast<int>(r), u_ws);
  return hipGetLastError();
}

int device_cus() {
  constexpr int kMaxDevices = 64;
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = cus;
  }
  return cached[dev];
}

hipError_t launch_decode_fwd(int n, const DecodeProj* proj, int64_t in, const uint16_t* X, int64_t T,
                             int64_t r, float s, uint16_t* Y, int64_t ldy, float* u_ws, hipStream_t st) {
  if (n < 1 || n > kMaxProj) return hipErrorInvalidValue;
  int64_t outs[kMaxProj];
  for (int i = 0; i < n; ++i) {
    if (!decode_fits(T, in, proj[i].out, r)) return hipErrorInvalidValue;
    outs[i] = proj[i].out;
  }
  // all projections in one launch
  DecodeSet set{};
  set.n = n;
  set.Y = Y;
  int64_t wgs = 0, col = 0;
  for (int i = 0; i < n; ++i) {
    set.proj[i] = proj[i];
    set.wg0[i] = static_cast<int>(wgs);
    set.col0[i] = col;
    wgs += proj[i].out / kRows;
    col += proj[i].out;
  }
  // With a workspace for U, the shapes the weight-stream kernel takes go
  // there: U = X A^T first, then the stream.
  const int cus = device_cus();
  if (u_ws != nullptr && cus > 0 && stream_fits(n, outs, in, T, r, cus)) {
    hipError_t e = launch_decode_u(set, in, X, T, r, u_ws, st);
    if (e == hipSuccess)
      e = launch_decode_stream(set, in, X, T, r, s, ldy, u_ws, static_cast<int>(wgs), cus, st);
    return e;
  }
  const bool pre_u = decode_pre_u(n, outs, r);
  if (pre_u && u_ws == nullptr) return hipErrorInvalidValue;
  const dim3 block(kThreads);
  const int iT = static_cast<int>(T), ir = static_cast<int>(r);
  if (pre_u) {
    const hipError_t e = launch_decode_u(set, in, X, T, r, u_ws, st);
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<uint32_t>(wgs));
  // chunk steps per wave: fully unrolled when they number 4 (in <= 4096)
  // or 8 (in <= 8192), a loop otherwise
  const int64_t steps = round_up((ceil_div(in / 64, 4) + 3) / 4, 2);
  const int ns = steps == 4 ? 4 : steps == 8 ? 8 : 0;
  const int xp = T <= 2 ? 1 : T <= 4 ? 2 : T <= 8 ? 4 : 8;
  // whole chunks in every wave's block range: 16 | in / 64
  const bool full = (in / 64) % 16 == 0;
  const float* upre = u_ws;
#define QLORA_SPLIT(XPV, NSV, FV)                                                                        \
  do {                                                                                                   \
    if (pre_u)                                                                                           \
      hipLaunchKernelGGL((k_decode_fwd_split<XPV, NSV, FV, true>), grid, block, 0, st, set, in, X, iT, ir, \
                         s, ldy, upre);                                                                  \
    else                                                                                                 \
      hipLaunchKernelGGL((k_decode_fwd_split<XPV, NSV, FV, false>), grid, block, 0, st, set, in, X, iT,   \
                         ir, s, ldy, upre);                                                              \
  } while (0)
#define QLORA_SPLIT_NS(XPV)                                  \
  do {                                                       \
    if (full) {                                              \
      if (ns == 4) QLORA_SPLIT(XPV, 4, true);                \
      else if (ns == 8) QLORA_SPLIT(XPV, 8, true);           \
      else QLORA_SPLIT(XPV, 0, true);                        \
    } else {                                                 \
      if (ns == 4) QLORA_SPLIT(XPV, 4, false);               \
      else if (ns == 8) QLORA_SPLIT(XPV, 8, false);          \
      else QLORA_SPLIT(XPV, 0, false);                       \
    }                                                        \
  } while (0)
  if (xp == 1) QLORA_SPLIT_NS(1);
  else if (xp == 2) QLORA_SPLIT_NS(2);
  else if (xp == 4) QLORA_SPLIT_NS(4);
  else QLORA_SPLIT_NS(8);
#undef QLORA_SPLIT_NS
#undef QLORA_SPLIT
  return hipGetLastError();
}

}  // namespace qlora
