// k_decode_stream.hip -- small-token QLoRA forward (T <= 16) as a
// persistent weight stream over all waves of the chip.
//
//   Y = X W_hat^T + s U B^T,  U = X A^T computed beforehand   (paperclase
//   lesson "QLoRA", Parte 4, h = W_hat x + (alpha/r) B A x; the weight is
//   dequantized to bf16 right before the matrix cores use it: ultralytics
//   glossary "QLoRA", "Como funciona a QLoRA")
//
// At these token counts the kernel is bound by streaming the packed codes
// and by the vector-ALU work of dequantizing them (about 3 instructions per
// weight), so the design keeps every SIMD dequantizing and every wave's
// next code loads in flight:
//
//   * grid: one workgroup per CU (at most 256), each owning a contiguous
//     range of 16-row blocks ("row blocks", up to kMaxRb of them);
//   * the 8 waves of a workgroup split the reduction dimension: wave w owns
//     blocks [w nb/8, (w+1) nb/8) of every row (nb = in/64, a multiple of
//     32), walked in chunks of 4 blocks; per chunk, lane (n, g) dequantizes
//     block g of row n (32 code bytes, one 16-entry table) straight into the
//     A operand of v_mfma_f32_16x16x32_bf16, whose B operand is token n's
//     matching activations;
//   * each wave stages its own slice of X (all T tokens, its in/8 columns)
//     once, in LDS, in the element order the table lookup produces, so the
//     lookups skip the four re-interleaving permutes per 8 weights; the
//     slice is private to the wave, so the stream needs no barrier;
//   * the steps (row block, chunk) form one flat sequence per wave with
//     kDepth steps of code loads in flight; every load of a step is issued
//     unconditionally (steps past the end read through an empty buffer
//     resource), so the compiler's wait counts keep the younger steps
//     outstanding;
//   * at the end of a row block every wave parks its 16 x 16 fp32 partial
//     in LDS; after one barrier the workgroup adds the 8 partials in a fixed
//     order, adds s U B^T and rounds Y to bf16 once (bit-reproducible).
//
// U = X A^T (fp32, [n][T][r]) is computed by k_decode_u before this launch;
// the B rows of all of a workgroup's row blocks are loaded at the start.
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxRb = 8;              // row blocks per workgroup
constexpr int kXPad = 16;              // bytes after each token row of a wave's slice
constexpr int kXBytes = 2 * kStreamMaxTokElems + kWaves * 16 * kXPad;
constexpr int kRU = 64;                // ranks held by the epilogue (r <= 64)
constexpr int kBufferWord3 = 0x00020000;
constexpr int kStream = 2;             // nt: streamed once
constexpr uint32_t kPastEnd = 0x80000000u;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kBufferWord3);
}

struct Codes {
  u32x4 c0, c1;   // this lane's 32 code bytes of the step
  uint32_t q;     // its 8-bit absmax code
  float sc;       // its group scale
};

// projection owning row block R (uniform)
__device__ __forceinline__ int proj_of(const DecodeSet& P, int R) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < kMaxProj; ++i)
    if (i < P.n && R >= P.wg0[i]) p = i;
  return p;
}

// What the stream needs of one projection, read from the kernel arguments
// once at entry: a workgroup's row blocks lie in at most two projections, so
// every later use picks one of two register-resident copies with a scalar
// select instead of walking the argument block again (each walk is a chain
// of dependent scalar-memory round trips).
struct Slot {
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* scale;
  const uint16_t* B;
  uint16_t* Y;          // the projection's first output column
  uint32_t wbytes;      // code bytes: out * in / 2
  int out, wg0;         // rows, first row block
};

__device__ __forceinline__ Slot load_slot(const DecodeSet& P, int p, int in) {
  Slot s;
  s.codes = P.proj[p].codes;
  s.absmax_q = P.proj[p].absmax_q;
  s.scale = P.proj[p].scale;
  s.B = P.proj[p].B;
  s.Y = P.Y + P.col0[p];
  s.out = static_cast<int>(P.proj[p].out);
  s.wbytes = static_cast<uint32_t>(P.proj[p].out * in / 2);
  s.wg0 = P.wg0[p];
  return s;
}

// (uniform) the slot of row block R
__device__ __forceinline__ Slot pick(int R, const Slot& a, const Slot& b) {
  const bool second = __builtin_amdgcn_readfirstlane(R >= b.wg0 ? 1 : 0) != 0;
  Slot s;
  s.codes = second ? b.codes : a.codes;
  s.absmax_q = second ? b.absmax_q : a.absmax_q;
  s.scale = second ? b.scale : a.scale;
  s.B = second ? b.B : a.B;
  s.Y = second ? b.Y : a.Y;
  s.wbytes = second ? b.wbytes : a.wbytes;
  s.out = second ? b.out : a.out;
  s.wg0 = second ? b.wg0 : a.wg0;
  return s;
}
}  // namespace

// kDepth: chunk steps of code loads in flight per wave (2 or 4); it divides
// the chunk steps of a row block (in / 2048), so every row block starts at
// register set 0 and the loop over a row block's steps unrolls in groups of
// kDepth with the epilogue after them (one copy of its code).  kSingle: one
// projection (its fields sit at fixed offsets of the argument block, so they
// are read in the first batch of scalar loads rather than after the
// projection lookup).
//
// The prologue is straight-line code whose uniform branches fall through on
// the common path: a kernel's first instructions are fetched cold by every
// CU at once, and each taken jump into code not yet fetched costs a full
// instruction-fetch round trip.
template <int kDepth, bool kSingle>
__global__ __launch_bounds__(kThreads) void k_decode_stream(DecodeSet P, int in, const uint16_t* __restrict__ X,
                                                            int T, int r, float s, int64_t ldy,
                                                            const float* __restrict__ U, int total_rb) {
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kXBytes];
  __shared__ f32x4 s_part[2][kWaves][64];
  __shared__ uint16_t s_b[2][16][kRU];
  __shared__ float s_u[2][16][kRU];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int G = gridDim.x, wg = blockIdx.x;
  // (readfirstlane: the values are uniform; it keeps them in scalar registers
  // so that the buffer descriptors built from them need no per-lane loop)
  const int rb0 = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(total_rb * wg) / G));
  const int rb1 =
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(total_rb * (wg + 1)) / G));
  const int nrb = rb1 - rb0;
  const int nb = in / 64;
  const int nbw = nb / kWaves;        // blocks of each row in this wave's slice
  const int nch = nbw / 4;            // chunk steps per row block
  const int kb0 = wv * nbw;           // first block of the slice
  const int p_first = kSingle ? 0 : proj_of(P, rb0), p_last = kSingle ? 0 : proj_of(P, rb1 - 1);
  const Slot sl0 = load_slot(P, p_first, in), sl1 = kSingle ? sl0 : load_slot(P, p_last, in);
  // every argument the prologue needs, read before any load is issued: the
  // empty asm takes them as scalar operands, so their loads from the argument
  // block leave in one batch here instead of one round trip at each first use
  const int np = P.n;
  __asm__ volatile("" ::"s"(in), "s"(T), "s"(r), "s"(s), "s"(ldy), "s"(total_rb), "s"(np), "s"(X), "s"(U));
  __asm__ volatile("" ::"s"(sl0.codes), "s"(sl0.absmax_q), "s"(sl0.scale), "s"(sl0.B), "s"(sl0.Y), "s"(sl0.wbytes),
                   "s"(sl0.out), "s"(sl0.wg0));
  if constexpr (!kSingle)
    __asm__ volatile("" ::"s"(sl1.codes), "s"(sl1.absmax_q), "s"(sl1.scale), "s"(sl1.B), "s"(sl1.Y),
                     "s"(sl1.wbytes), "s"(sl1.out), "s"(sl1.wg0));
  const __amdgpu_buffer_rsrc_t rs_u = rsrc(U, static_cast<uint32_t>(np * T * r * 4));
  const __amdgpu_buffer_rsrc_t rs_x = rsrc(X, static_cast<uint32_t>(T) * in * 2);
  // per-lane parts of the code and absmax offsets (row n, block g of a
  // chunk), computed before any load is in flight
  const uint32_t vo_code = __umul24(n, in / 2) + 32 * g;
  const uint32_t vo_q = __umul24(n, nb) + g;

  // ---------------------------------------------------------- code stream
  int l_rbl = 0, l_c = 0;  // next step to load
  auto issue = [&](Codes& cs) {
    const bool live = l_rbl < nrb;
    const int R = __builtin_amdgcn_readfirstlane(rb0 + (live ? l_rbl : 0));
    const Slot sl = kSingle ? sl0 : pick(R, sl0, sl1);
    const int rbp = R - sl.wg0;
    const uint32_t wbytes = __builtin_amdgcn_readfirstlane(live ? sl.wbytes : 0u);
    const __amdgpu_buffer_rsrc_t rc = rsrc(sl.codes, wbytes);
    const __amdgpu_buffer_rsrc_t rq = rsrc(sl.absmax_q, wbytes / 32);
    const __amdgpu_buffer_rsrc_t rsc = rsrc(sl.scale, (wbytes + 8191) / 8192 * 4);
    const int blk = kb0 + 4 * l_c;
    const int soff = rbp * 16 * (in / 2) + 32 * blk;
    cs.c0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, vo_code, soff, kStream));
    cs.c1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, vo_code + 16, soff, kStream));
    const uint32_t bi = vo_q + static_cast<uint32_t>(rbp * 16 * nb + blk);
    cs.q = __builtin_amdgcn_raw_buffer_load_b8(rq, bi, 0, 0);
    cs.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, (bi >> 8) * 4, 0, 0));
    if (++l_c == nch) {
      l_c = 0;
      ++l_rbl;
    }
  };
  Codes cs[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(cs[d]);

  // ------------------------------------------------------ loads at the start
  // Element idx = tid + 512 i of the two [16][64] U slots (first and last
  // projection of the range): slot i / 2, token wv + 8 (i % 2), rank lane --
  // the token is uniform per wave, so each load is one scalar offset plus the
  // lane's rank (ranks >= r and tokens >= T read zero)
  const uint32_t vo_rank4 = lane < r ? static_cast<uint32_t>(lane * 4) : kPastEnd;
  float ureg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = wv + 8 * (i & 1), p = i < 2 ? p_first : p_last;
    const uint32_t so = t < T ? static_cast<uint32_t>((p * T + t) * r * 4) : kPastEnd;
    ureg[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_u, vo_rank4, so, 0));
  }

  // This wave's X slice: T token rows of in / 8 columns, PR = in / 64 pieces
  // of 16 bytes each, PR a multiple of 64: load i takes token t_i, pieces
  // pc_i + lane (one scalar offset plus the lane's 16 bytes); loads stop at T.
  const int PR = nb;
  const int pitch = PR * 16 + kXPad;  // bytes per token row in LDS
  uint8_t* xw = s_x + wv * T * pitch;
  const int nx = T * (PR >> 6);       // loads of this wave (<= 16)
  u32x4 xv[16];
  {
    int t = 0, pc0 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nx)  // uniform
        xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs_x, 16 * lane, (t * in + kb0 * 64 + 8 * pc0) * 2, 0));
      pc0 += 64;
      if (pc0 == PR) {
        pc0 = 0;
        ++t;
      }
    }
  }

  // B rows of every row block of the range: element idx = tid + 512 e of a
  // block's [16][64] (row wv + 8 e, uniform per wave; rank lane, ranks >= r
  // read zero)
  const uint32_t vo_rank2 = lane < r ? static_cast<uint32_t>(lane * 2) : kPastEnd;
  uint32_t braw[kMaxRb][2];
#pragma unroll
  for (int k = 0; k < kMaxRb; ++k) {
    braw[k][0] = braw[k][1] = 0u;
    if (k < nrb) {  // uniform
      const int R = rb0 + k;
      const Slot sl = kSingle ? sl0 : pick(R, sl0, sl1);
      const __amdgpu_buffer_rsrc_t rs_b = rsrc(sl.B, static_cast<uint32_t>(sl.out * r * 2));
      const int rbp = R - sl.wg0;
#pragma unroll
      for (int e = 0; e < 2; ++e)
        braw[k][e] = __builtin_amdgcn_raw_buffer_load_b16(rs_b, vo_rank2, (16 * rbp + wv + 8 * e) * r * 2, 0);
    }
  }

  // U into LDS, then the X slice in the lookup's element order
#pragma unroll
  for (int i = 0; i < 4; ++i) s_u[i >> 1][wv + 8 * (i & 1)][lane] = ureg[i];
  {
    int t = 0, pc0 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nx) {  // uniform
        const uint32_t in4[4] = {xv[i][0], xv[i][1], xv[i][2], xv[i][3]};
        uint32_t o[4];
        to_split_order(in4, o);
        *reinterpret_cast<u32x4*>(xw + t * pitch + 16 * (pc0 + lane)) = u32x4{o[0], o[1], o[2], o[3]};
      }
      pc0 += 64;
      if (pc0 == PR) {
        pc0 = 0;
        ++t;
      }
    }
  }

  // lane (n, g) feeds token n's activations into MFMA column n; columns
  // n >= T are discarded, so their lanes read token T - 1's row, which keeps
  // every read inside this wave's slice
  const uint8_t* xr = xw + (n < T ? n : T - 1) * pitch + 128 * g;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  // one chunk step: lane (n, g) dequantizes block g of row n straight into the
  // MFMA's A operand, against its activations in the B operand
  auto compute = [&](const Codes& st, int c) {
    // the step's 8 activation fragments first: their LDS latency passes
    // while the table is built
    const uint8_t* xc = xr + 512 * c;
    u32x4 xf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xf[j] = *reinterpret_cast<const u32x4*>(xc + 16 * j);
    const Nf4Table tab = make_table(dq_absmax(st.q, st.sc));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w[4];
      lookup8_split(tab, j < 4 ? st.c0[j] : st.c1[j - 4], w);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}), as_bf16x8(xf[j]),
                                                    acc, 0, 0, 0);
    }
  };

  for (int rbl = 0; rbl < nrb; ++rbl) {
    for (int c = 0; c < nch; c += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        // keep each step's instructions together: the scheduler would
        // otherwise hoist the next step's table build (and so the wait for
        // its loads) into this one, shortening the prefetch by a step
        __builtin_amdgcn_sched_barrier(0);
        compute(cs[d], c + d);
        issue(cs[d]);
      }
    }
    // ---- epilogue of the row block: the 8 waves' partials meet in LDS;
    // wave 0 adds s U B^T with four MFMAs (the block's 16 B rows x (s U)^T
    // as bf16 hi + lo, 2 x 32 ranks) and stores Y, rounded to bf16 once.
    // The other waves go on with the next row block.
    const int buf = rbl & 1;
    s_part[buf][wv][lane] = acc;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    // this block's B values: an and/or mask over the registers (a select
    // chain would be turned into a dynamically indexed array in scratch)
    uint32_t b0 = 0, b1 = 0;
#pragma unroll
    for (int k = 0; k < kMaxRb; ++k) {
      const uint32_t mk = 0u - static_cast<uint32_t>(rbl == k);
      b0 |= braw[k][0] & mk;
      b1 |= braw[k][1] & mk;
    }
    (&s_b[buf][0][0])[tid] = static_cast<uint16_t>(b0);
    (&s_b[buf][0][0])[tid + kThreads] = static_cast<uint16_t>(b1);
    __syncthreads();
    if (wv == 0) {
      const int R = __builtin_amdgcn_readfirstlane(rb0 + rbl);
      const Slot sl = kSingle ? sl0 : pick(R, sl0, sl1);
      const int rbp = R - sl.wg0;
      const int slot = R >= sl1.wg0 ? 1 : 0;  // U of the first or second projection
      // D[row 4 g + e][token n] = sum_j B[row][j] (s U)[n][j]: lane (n, g)
      // holds B row n's and token n's ranks 32 ks + 8 g .. + 7
      f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kRU / 32; ++ks) {
        const u32x4 bf = *reinterpret_cast<const u32x4*>(&s_b[buf][n][32 * ks + 8 * g]);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float u0 = s * s_u[slot][n][32 * ks + 8 * g + 2 * e];
          const float u1 = s * s_u[slot][n][32 * ks + 8 * g + 2 * e + 1];
          hi[e] = pack_bf16x2(u0, u1);
          lo[e] = pack_bf16x2(u0 - __builtin_bit_cast(float, hi[e] << 16),
                              u1 - __builtin_bit_cast(float, hi[e] & 0xffff0000u));
        }
        lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bf), as_bf16x8(u32x4{hi[0], hi[1], hi[2], hi[3]}),
                                                       lsum, 0, 0, 0);
        lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bf), as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]}),
                                                       lsum, 0, 0, 0);
      }
      // the waves' partials of the same four outputs, in a fixed order
      f32x4 base = s_part[buf][0][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const f32x4 pw = s_part[buf][w][lane];
        base = f32x4{base[0] + pw[0], base[1] + pw[1], base[2] + pw[2], base[3] + pw[3]};
      }
      if (n < T) {
        uint16_t* __restrict__ Y = sl.Y + static_cast<int64_t>(n) * ldy + 16 * rbp + 4 * g;
        *reinterpret_cast<u32x2*>(Y) = u32x2{pack_bf16x2(base[0] + lsum[0], base[1] + lsum[1]),
                                             pack_bf16x2(base[2] + lsum[2], base[3] + lsum[3])};
      }
    }
  }
}

bool stream_fits(int n, const int64_t* outs, int64_t in, int64_t T, int64_t r, int num_cus) {
  if (T < 1 || T > kDecodeMaxT || r < 1 || r > kRU || n < 1 || n > kMaxProj) return false;
  if (in % 4096 != 0 || T * in > kStreamMaxTokElems) return false;
  int64_t total = 0;
  int64_t first[kMaxProj + 1];
  for (int i = 0; i < n; ++i) {
    if (outs[i] % 16 != 0 || outs[i] * in >= (int64_t(1) << 31)) return false;
    first[i] = total;
    total += outs[i] / 16;
  }
  first[n] = total;
  // At most one 16-row block per CU the single-launch kernel (k_decode.hip),
  // which computes U itself, is faster: this kernel needs U from a separate
  // launch first.  From two blocks per CU on it wins (measured on the MLP
  // weights at 1 and 16 tokens).
  if (total < 2 * static_cast<int64_t>(num_cus)) return false;
  const int64_t G = num_cus;
  if ((total + G - 1) / G > kMaxRb) return false;
  // every workgroup's row blocks lie in at most two projections
  for (int64_t w = 0; w < G; ++w) {
    const int64_t a = total * w / G, b = total * (w + 1) / G - 1;
    int pa = 0, pb = 0;
    for (int i = 0; i < n; ++i) {
      if (a >= first[i]) pa = i;
      if (b >= first[i]) pb = i;
    }
    if (pb - pa > 1) return false;
  }
  return true;
}

hipError_t launch_decode_stream(const DecodeSet& set, int64_t in, const uint16_t* X, int64_t T, int64_t r,
                                float s, int64_t ldy, const float* u_ws, int total_rb, int num_cus,
                                hipStream_t st) {
  const int G = total_rb < num_cus ? total_rb : num_cus;
  // steps in flight: 4 where they divide a row block's in / 2048 chunk steps, else 2
  const int depth = (in / 2048) % 4 == 0 ? 4 : 2;
  const bool single = set.n == 1;
#define QLORA_STREAM(D, S1)                                                                                 \
  hipLaunchKernelGGL((k_decode_stream<D, S1>), dim3(static_cast<uint32_t>(G)), dim3(kThreads), 0, st, set, \
                     static_cast<int>(in), X, static_cast<int>(T), static_cast<int>(r), s, ldy, u_ws, total_rb)
  if (single) {
    if (depth == 4) QLORA_STREAM(4, true);
    else QLORA_STREAM(2, true);
  } else {
    if (depth == 4) QLORA_STREAM(4, false);
    else QLORA_STREAM(2, false);
  }
#undef QLORA_STREAM
  return hipGetLastError();
}

}  // namespace qlora
