// k_gemm.hip -- bf16 MFMA GEMM for gfx950 with fp32 accumulation and one
// rounding to bf16 at the end:
//   C[M][N] = sum_k act0[m][k] wt0[n][k]  +  sum_k act1[m][k] wt1[n][k]
// The main segment's weight operand is either a bf16 matrix or an NF4 weight
// (codes + double-quantized absmax) that is dequantized while it is staged
// into LDS: each thread turns packed codes of one 64-weight block into bf16
// with the block's v_perm table and writes them straight into the swizzled
// LDS tile, so W_hat never exists in HBM (ultralytics glossary "QLoRA": the
// frozen weight is dequantized to bfloat16 right before the matmul;
// paperclase lesson "QLoRA", Parte 4: W_hat is built, used and discarded).
// The second segment carries the LoRA term as extra K-steps (act1 = s*U or
// s*V as a bf16 hi/lo pair, wt1 = B or A^T padded to match), so base and
// adapter products share one fp32 accumulator and Y / dX are rounded once.
//
// Two kernels, both v_mfma_f32_32x32x16_bf16 with the weight tile as the
// MFMA A operand (rows n) and the activation tile as B (rows m), so each lane
// ends up holding 4 consecutive n of one output row m (one 8-byte store):
//
// k_gemm_big (grids of >= 256 tiles): 256 x 256 x 64 tiles, 8 waves (2 x 4,
// 128 x 64 each, two per SIMD).  bf16 tiles go from global memory straight
// into LDS (buffer_load ... lds: one 1 KB block of 8 rows per wave
// instruction, the swizzle applied on the global side), so they take no
// registers and no LDS-write instructions.  Two LDS stages, each a separate
// __shared__ array and the stage index a compile-time constant in the
// unrolled loop, so the compiler can see that the copies into one stage do
// not alias the fragment reads of the other and does not make every LDS
// read wait for the copies in flight.  Step e: copy step e+1 into the other
// stage, compute step e (fragments of sub-step j+1 read during sub-step j),
// one barrier at the end.  An NF4 weight is loaded into registers three
// steps ahead (three register sets) and dequantized into the other stage a
// quarter per sub-step, between the MFMAs; the barrier waits only for the
// copies, not for those code loads.
//
// k_gemm (smaller grids): 128 x 128 x 64 tiles, 4 waves, tiles staged
// through two register sets (three K-steps of loads in flight) and two LDS
// stages, one barrier per K-step.  Below one workgroup per CU it splits K
// (blockIdx.z) into fp32 partials that k_split_sum adds in order.
//
// For dX = dY W_hat the weight is read transposed (K runs along W's rows):
// the NF4 tile is dequantized into LDS K-row-major and the MFMA fragments
// are read with gfx950's transposing LDS loads (Nf4TileT, lds_frag_tr).
#include <type_traits>

#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

namespace {

constexpr int kBK = 64;

// main-segment weight operand of the GEMM kernels
constexpr int kWBf16 = 0;  // bf16 matrix [N][K]
constexpr int kWNf4 = 1;   // NF4 weight [N][K], dequantized while staged
constexpr int kWNf4T = 2;  // NF4 weight [K][N] (dX), dequantized and transposed while staged

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
  static_assert(kTPR == 1 || kTPR == 2 || kTPR == 4, "unsupported tile");
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
    if constexpr (kDw == 8) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff, static_cast<int>(k0 / 2), kStream));
      const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff + 16, static_cast<int>(k0 / 2), kStream));
      r.cw[0] = v[0]; r.cw[1] = v[1]; r.cw[2] = v[2]; r.cw[3] = v[3];
      r.cw[4] = w[0]; r.cw[5] = w[1]; r.cw[6] = w[2]; r.cw[7] = w[3];
    } else if constexpr (kDw == 4) {
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
  // The same in pieces: the block's table once, then code dword d -> one
  // 16-byte chunk of the LDS tile.
  __device__ __forceinline__ static Nf4Table table(const Regs& r) { return make_table(dq_absmax(r.q, r.sg)); }
  __device__ __forceinline__ static void store_part(const Regs& r, const Nf4Table& tab, uint16_t* lds, int tid, int d) {
    const int row = tid / kTPR, part = tid % kTPR;
    uint32_t o[4];
    lookup8(tab, r.cw[d], o);
    const int chunk = part * kDw + d;
    *reinterpret_cast<u32x4*>(lds + row * kBK + swz(row, chunk) * 8) = u32x4{o[0], o[1], o[2], o[3]};
  }
};

// bf16 tile rows [ROWS][64] of a K-contiguous matrix copied straight into
// LDS by NW waves: ROWS/8 blocks of 1 KB, one wave instruction each.  Lane L
// of a block lands at LDS byte 16 L of the block, i.e. row 8 blk + L/8,
// position L % 8, so it loads the global chunk that the swizzle puts there
// (the XOR swizzle is its own inverse).  Rows past the matrix read as zero.
template <int ROWS, int NW>
struct DtlTile {
  static constexpr int kPerWave = ROWS / 8 / NW;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[kPerWave];
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int64_t row0, int64_t nrows, int wv, int lane) {
    rs = rows_rsrc(base, ld, row0, nrows, 2);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int row = (i * NW + wv) * 8 + (lane >> 3);
      voff[i] = static_cast<uint32_t>((row * ld + swz(row, lane & 7) * 8) * 2);
    }
  }
  __device__ __forceinline__ void load(uint16_t* lds, int wv, int64_t k0) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + (i * NW + wv) * 512), 16, voff[i],
          static_cast<int>(k0 * 2), 0, 0);
  }
};

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* lds, int row, int chunk) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * kBK + swz(row, chunk) * 8);
  return __builtin_bit_cast(bf16x8, v);
}
// Transposed NF4 weight tiles (the dX GEMM) are stored K-row-major: row k
// of W (a K index) holds the tile's BN columns, 16-byte chunk c of row k at
// chunk c ^ tswz(k).  tswz(k) = 4 (k % 4) + (k / 4) % 4 keeps both accesses
// conflict-free on the 64-bank LDS: a dequantize write (16 lanes, 16
// consecutive rows, one chunk) lands in 16 distinct chunk slots, and a
// transposed fragment read (32 lanes: 4 consecutive rows x 4 consecutive
// chunks, 8 bytes per lane) covers 16 distinct slots.
__device__ __forceinline__ int tswz(int k) { return 4 * (k & 3) + ((k >> 2) & 3); }

// MFMA operand fragment of rows n = n0 .. n0 + 31 (n0 wave-uniform), K
// sub-step j, from a transposed tile of BN columns: lane l holds n = n0 + l % 32
// and k = 16 j + 8 (l / 32) + 0..7.  ds_read_b64_tr_b16 hands each group of
// 16 lanes a 16 x 4 block transposed: lane i of the group supplies the address
// of row i / 4 (of four consecutive rows) at columns 4 (i % 4) .. + 3, and
// receives column i of the four rows.  Two such reads give the eight k.
template <int BN>
__device__ __forceinline__ bf16x8 lds_frag_tr(const uint16_t* lds, int n0, int j) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const int l = threadIdx.x & 63, i = l & 15, G = l >> 4;
  const int n = n0 + 16 * (G & 1) + 4 * (i & 3);
  v4s v[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int k = 16 * j + 8 * (G >> 1) + 4 * s2 + (i >> 2);
    const int e = k * BN + (((n >> 3) ^ tswz(k)) << 3) + (n & 4);
    v[s2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(const_cast<uint16_t*>(lds) + e));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}
// A weight fragment of the main segment (kTr: a transposed NF4 tile of BN
// columns) or of the LoRA segment (always the swizzled N-row-major tile);
// row = n0 + lane % 32, chunk = 2 j + lane / 32.
template <bool kTr, int BN>
__device__ __forceinline__ bf16x8 wt_frag(const uint16_t* lds, int n0, int row, int j, int chunk) {
  if constexpr (kTr) return lds_frag_tr<BN>(lds, n0, j);
  else return lds_frag(lds, row, chunk);
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

// One projection of an NF4 main segment: its rows [n0, n0 + rows) of C, its
// storage and its LoRA activation block (act1 of the extension segment).
struct Nf4Seg {
  const uint8_t* codes; const uint8_t* absmax_q; const float* scale;
  int64_t n0, rows;
  const uint16_t* act1;
};

struct GemmArgs {
  int64_t M, N;
  // main segment activation and weight: a bf16 weight (wt0), or NF4
  // projections stacked along N (nseg >= 1; no tile straddles two)
  const uint16_t* act0; int64_t lda0;
  const uint16_t* wt0; int64_t ldw0;
  int nseg;
  Nf4Seg seg[kMaxProj];
  int64_t K0;
  // LoRA extension segment (with nseg > 0, act1 comes from the tile's seg[])
  const uint16_t* act1; int64_t lda1;
  const uint16_t* wt1; int64_t ldw1;
  int64_t K1;
  uint16_t* C; int64_t ldc;
  // LoRA dropout (null: none): the extension segment runs first and its
  // product is multiplied element-wise by keep_scale * keep[m][n] before the
  // main segment adds to the same accumulator (bit n % 8 of byte
  // keep[m * ldk + n / 8])
  const uint8_t* keep; int64_t ldk; float keep_scale;
  // split-K (k_gemm only; part == nullptr: none): workgroup z = blockIdx.z of
  // gridDim.z takes main-segment K-steps [z ks, min((z + 1) ks, K0 / 64)),
  // split 0 also the LoRA segment, and writes fp32 partials
  // part[z][m][n] (row stride N) instead of C
  float* part; int64_t ks;
};

// acc[a][c][e] holds C[m][n] with m = m_base + 32 c + r32 and
// n = n_base + 32 a + 8 (e / 4) + 4 half + e % 4 (the layout of
// v_mfma_f32_32x32x16_bf16 as these kernels use it).  Multiplies each
// element by keep_scale where its keep bit is set, by 0 elsewhere.
template <int FN, int FM>
__device__ __forceinline__ void apply_keep(f32x16 (&acc)[FN][FM], const GemmArgs& p, int64_t m_base,
                                           int64_t n_base, int r32, int half) {
  const uint64_t kbytes = static_cast<uint64_t>(p.M) * p.ldk;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.keep), 0, static_cast<int>(kbytes < 0x7fffffffu ? kbytes : 0x7fffffffu),
      0x00020000);
#pragma unroll
  for (int c = 0; c < FM; ++c) {
    const int64_t m = m_base + 32 * c + r32;
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n_base + 32 * a + 8 * g;  // a multiple of 8: one byte
        // rows past M and columns past N are never stored: read nothing for them
        const uint32_t off = (m < p.M && n < p.N) ? static_cast<uint32_t>(m * p.ldk + n / 8) : 0x80000000u;
        const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0) >> (4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[a][c][4 * g + i] *= ((bits >> i) & 1u) ? p.keep_scale : 0.f;
      }
  }
}

// The projection holding output column n0 (uniform; constant indices only,
// so the table stays in scalar registers).
__device__ __forceinline__ Nf4Seg seg_of(const GemmArgs& p, int64_t n0) {
  Nf4Seg sg = p.seg[0];
#pragma unroll
  for (int i = 1; i < kMaxProj; ++i)
    if (i < p.nseg && n0 >= p.seg[i].n0) sg = p.seg[i];
  return sg;
}

// Register set of a weight tile staged through registers (none for tiles
// copied straight into LDS).
struct NoRegs {};
template <class T, bool kReg>
struct RegsOf { using type = NoRegs; };
template <class T>
struct RegsOf<T, true> { using type = typename T::Regs; };

// NF4 weights for dX = dY W_hat: the tile holds W_hat^T rows [n0, n0 + ROWS)
// -- columns of W -- by 64 K, and K runs along W's rows (over several
// projections, the projections' rows one after another: each K-step picks its
// projection from the table).  The 64-weight blocks run along W's rows, so
// wave g takes the 32 columns [n0 + 32 g, n0 + 32 g + 32) and lane k row k of
// each K-step: its 16 code bytes (half a block), the block's absmax code and
// group scale.  At store time the lane expands its 32 weights with the block's
// table and writes them as four 16-byte chunks of row k, so the stage holds
// the tile K-row-major (swizzled by tswz) and the MFMA fragments are read
// with transposing loads (lds_frag_tr).
template <int ROWS, int NT>
struct Nf4TileT {
  static_assert(NT == 2 * ROWS, "one wave per 32 columns");
  static constexpr int kDw = 4;  // code dwords (8 weights each) per thread
  struct Regs {
    uint32_t cw[kDw];
    uint32_t q;
    float sg;
  };
  const GemmArgs* p;  // projection table: seg[i].n0 = first K row, .rows = rows
  int64_t in;
  uint32_t coff, qoff;  // this lane's code byte / absmax code in row 0 of a projection
  uint32_t bcol;        // its column block
  uint32_t wofs[kDw];   // LDS element offsets of its four 16-byte chunks

  // the tile's first column n0 (columns past `in` load valid data that is never stored)
  __device__ __forceinline__ void init(const GemmArgs& args, int64_t n0, int tid) {
    const int k = tid & 63, g = tid >> 6;
    p = &args;
    in = args.N;
    int64_t c0 = n0 + 32 * g;
    if (c0 >= in) c0 = in - 32;
    coff = static_cast<uint32_t>(k * (in / 2) + c0 / 2);
    qoff = static_cast<uint32_t>(k * (in / 64) + c0 / 64);
    bcol = static_cast<uint32_t>(c0 / 64);
#pragma unroll
    for (int d = 0; d < kDw; ++d) wofs[d] = static_cast<uint32_t>(k * ROWS + (((4 * g + d) ^ tswz(k)) << 3));
  }
  // K-step starting at row k0 of the stacked projections
  __device__ __forceinline__ void load(Regs& r, int64_t k0) const {
    const Nf4Seg sg = seg_of(*p, k0);
    const int64_t kr = k0 - sg.n0;  // first row of the step within its projection
    const __amdgpu_buffer_rsrc_t rc = rows_rsrc(sg.codes, in / 2, 0, sg.rows, 1);
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(sg.absmax_q, in / 64, 0, sg.rows, 1);
    const u32x4 v = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff, static_cast<int>(kr * (in / 2)), kStream));
    r.cw[0] = v[0]; r.cw[1] = v[1]; r.cw[2] = v[2]; r.cw[3] = v[3];
    r.q = __builtin_amdgcn_raw_buffer_load_b8(rq, qoff, static_cast<int>(kr * (in / 64)), 0);
    const int k = static_cast<int>(threadIdx.x & 63);
    r.sg = sg.scale[((kr + k) * (in / 64) + bcol) >> 8];
  }
  __device__ __forceinline__ static Nf4Table table(const Regs& r) { return make_table(dq_absmax(r.q, r.sg)); }
  // code dword d: the lane's columns 8 d .. 8 d + 7, one 16-byte chunk
  __device__ __forceinline__ void store_part(const Regs& r, const Nf4Table& tab, uint16_t* lds, int, int d) const {
    uint32_t o[4];
    lookup8(tab, r.cw[d], o);
    *reinterpret_cast<u32x4*>(lds + wofs[d]) = u32x4{o[0], o[1], o[2], o[3]};
  }
  __device__ __forceinline__ void store(const Regs& r, uint16_t* lds, int tid) const {
    const Nf4Table tab = table(r);
#pragma unroll
    for (int d = 0; d < kDw; ++d) store_part(r, tab, lds, tid, d);
  }
};

}  // namespace

// WAVES_M x WAVES_N waves; each computes a (BM/WAVES_M) x (BN/WAVES_N) sub-tile.
//
// Step st: barrier (LDS stage st % 2 complete; stage (st + 1) % 2 free), write
// step st + 1's tiles from register set (st + 1) % 2 into LDS (NF4 weights
// are dequantized here), load step st + 3's tiles into that register set,
// compute step st.  The main and LoRA segments run this pipeline one after
// the other, each with register sets of its own operand types.
template <int BM, int BN, int WAVES_M, int WAVES_N, int kW>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm(GemmArgs p) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, FM = WM / 32, FN = WN / 32;
  __shared__ __attribute__((aligned(16))) uint16_t s_act[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_wt[2][BN * kBK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % WAVES_M, wn = wv / WAVES_M;
  // NF4: waves 4-7 (sharing SIMDs with waves 0-3) dequantize after computing
  const bool late = kW != kWBf16 && wv >= 4;
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

  auto compute = [&](int b, auto tr) {
    constexpr bool P = decltype(tr)::value;
    const uint16_t* sa = s_act[b];
    const uint16_t* sw = s_wt[b];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int chunk = 2 * j + half;
      bf16x8 fw[FN], fa[FM];
#pragma unroll
      for (int a = 0; a < FN; ++a) fw[a] = wt_frag<P, BN>(sw, wn * WN + a * 32, wn * WN + a * 32 + r32, j, chunk);
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
  auto segment = [&](auto& r0, auto& r1, int64_t first, int64_t last, auto fetch, auto stash, auto tr) {
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
      compute(static_cast<int>((first + e) & 1), tr);
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

  const bool split = p.part != nullptr;
  const int z = split ? static_cast<int>(blockIdx.z) : 0;
  int64_t kb = 0, s0 = p.K0 / kBK;  // this workgroup's main-segment K-steps [kb, kb + s0)
  if (split) {
    kb = z * p.ks;
    const int64_t end = kb + p.ks < s0 ? kb + p.ks : s0;
    s0 = end > kb ? end - kb : 0;
  }
  const int64_t s1 = z == 0 ? p.K1 / kBK : 0;
  using TA = Bf16Tile<BM, NT>;
  using TW = Bf16Tile<BN, NT>;
  // main segment over global steps [first, first + s0)
  auto main_seg = [&](int64_t first) {
    if constexpr (kW == kWNf4T) {
      using TQ = Nf4TileT<BN, NT>;
      TA ta;
      TQ tq;
      ta.init(p.act0, p.lda0, m0, p.M, tid);
      tq.init(p, n0, tid);
      struct R { typename TA::Regs a; typename TQ::Regs w; };
      R r0, r1;
      segment(r0, r1, first, first + s0,
              [&](R& r, int64_t e) {
                ta.load(r.a, (kb + e) * kBK);
                tq.load(r.w, (kb + e) * kBK);
              },
              [&](const R& r, int b) {
                TA::store(r.a, s_act[b], tid);
                tq.store(r.w, s_wt[b], tid);
              }, std::true_type{});
    } else if constexpr (kW == kWNf4) {
      using TQ = Nf4Tile<BN, NT>;
      TA ta;
      TQ tq;
      ta.init(p.act0, p.lda0, m0, p.M, tid);
      const Nf4Seg sg = seg_of(p, n0);
      tq.init(sg.codes, sg.absmax_q, sg.scale, p.K0, n0 - sg.n0, sg.rows, tid);
      struct R { typename TA::Regs a; typename TQ::Regs w; };
      R r0, r1;
      segment(r0, r1, first, first + s0,
              [&](R& r, int64_t e) {
                ta.load(r.a, (kb + e) * kBK);
                tq.load(r.w, (kb + e) * kBK);
              },
              [&](const R& r, int b) {
                TA::store(r.a, s_act[b], tid);
                TQ::store(r.w, s_wt[b], tid);
              }, std::false_type{});
    } else {
      TA ta;
      TW tw;
      ta.init(p.act0, p.lda0, m0, p.M, tid);
      tw.init(p.wt0, p.ldw0, n0, p.N, tid);
      struct R { typename TA::Regs a; typename TW::Regs w; };
      R r0, r1;
      segment(r0, r1, first, first + s0,
              [&](R& r, int64_t e) {
                ta.load(r.a, (kb + e) * kBK);
                tw.load(r.w, (kb + e) * kBK);
              },
              [&](const R& r, int b) {
                TA::store(r.a, s_act[b], tid);
                TW::store(r.w, s_wt[b], tid);
              }, std::false_type{});
    }
  };
  // LoRA extension segment over global steps [first, first + s1)
  auto lora_seg = [&](int64_t first) {
    if (s1 <= 0) return;
    TA ta;
    TW tw;
    ta.init(p.nseg > 0 ? seg_of(p, n0).act1 : p.act1, p.lda1, m0, p.M, tid);
    tw.init(p.wt1, p.ldw1, n0, p.N, tid);
    struct R { typename TA::Regs a; typename TW::Regs w; };
    R r0, r1;
    segment(r0, r1, first, first + s1,
            [&](R& r, int64_t e) {
              ta.load(r.a, e * kBK);
              tw.load(r.w, e * kBK);
            },
            [&](const R& r, int b) {
              TA::store(r.a, s_act[b], tid);
              TW::store(r.w, s_wt[b], tid);
            }, std::false_type{});
  };
  if (p.keep != nullptr) {
    // dropout: the adapter product alone, masked, then the base on top
    lora_seg(0);
    apply_keep<FN, FM>(acc, p, m0 + wm * WM, n0 + wn * WN, r32, half);
    main_seg(s1);
  } else {
    main_seg(0);
    lora_seg(s0);
  }

  // epilogue: D[n][m] -> C[m][n] (or the split's fp32 partial); lane holds
  // m = r32, n = 8*(e/4) + 4*half + e%4
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
          if (split) {
            *reinterpret_cast<f32x4*>(p.part + (static_cast<int64_t>(z) * p.M + m) * p.N + n) =
                f32x4{acc[a][c][4 * g + 0], acc[a][c][4 * g + 1], acc[a][c][4 * g + 2], acc[a][c][4 * g + 3]};
          } else {
            const uint32_t p0 = pack_bf16x2(acc[a][c][4 * g + 0], acc[a][c][4 * g + 1]);
            const uint32_t p1 = pack_bf16x2(acc[a][c][4 * g + 2], acc[a][c][4 * g + 3]);
            *reinterpret_cast<u32x2*>(p.C + m * p.ldc + n) = u32x2{p0, p1};
          }
        }
      }
    }
  }
}

// C[m][n] = bf16(sum over z = 0, 1, ... of part[z][m][n]), the splits added
// in order (bit-reproducible), one rounding.  Thread: 8 consecutive columns
// of one row; N % 8 == 0.
__global__ __launch_bounds__(256) void k_split_sum(const float* part, int S, int64_t M, int64_t N,
                                                   int64_t ldp, uint16_t* C, int64_t ldc) {
  const int64_t groups = N / 8;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= M * groups) return;
  const int64_t m = id / groups, n = (id % groups) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int z = 0; z < S; ++z) {
    const float* src = part + (static_cast<int64_t>(z) * M + m) * ldp + n;
    const f32x4 u = *reinterpret_cast<const f32x4*>(src);
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += u[e];
      acc[4 + e] += v[e];
    }
  }
  *reinterpret_cast<u32x4*>(C + m * ldc + n) =
      u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
            pack_bf16x2(acc[6], acc[7])};
}

// BM x 256 tiles (BM = 256 or 128), 8 waves (see the file comment).
// Launch: 512 threads.
template <int kW, int BM>
__global__ __launch_bounds__(512, 1) void k_gemm_big(GemmArgs p) {
  static_assert(BM == 256 || BM == 128, "tile rows");
  constexpr int NW = 8, NT = 64 * NW, BN = 256;
  constexpr int FN = 2, WN = 64, FM = BM / 64, WM = BM / 2;  // wave tile BM/2 (m) x 64 (n)
  __shared__ __attribute__((aligned(1024))) uint16_t s_act0[BM * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t s_act1[BM * kBK];
  constexpr bool kTrW = kW == kWNf4T;  // main-segment weight tile K-row-major (transposed reads)
  constexpr int kWtElems = BN * kBK;
  __shared__ __attribute__((aligned(1024))) uint16_t s_wt0[kWtElems];
  __shared__ __attribute__((aligned(1024))) uint16_t s_wt1[kWtElems];
  uint16_t* const s_act[2] = {s_act0, s_act1};
  uint16_t* const s_wt[2] = {s_wt0, s_wt1};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;
  int64_t mt, nt;
  xcd_tile(gridDim.x, gridDim.y, mt, nt);
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int r32 = lane & 31, half = lane >> 5;

  f32x16 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int c = 0; c < FM; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.f;

  typedef bf16x8 Frags[FN + FM];  // [0, FN) weight rows, [FN, FN + FM) activation rows
  // tr: the weight stage holds a transposed NF4 tile (K-row-major)
  auto read_frags = [&](Frags& f, const uint16_t* sw, const uint16_t* sa, int j, auto tr) {
    constexpr bool P = decltype(tr)::value;
    const int chunk = 2 * j + half;
#pragma unroll
    for (int a = 0; a < FN; ++a) f[a] = wt_frag<P, BN>(sw, wn * WN + a * 32, wn * WN + a * 32 + r32, j, chunk);
#pragma unroll
    for (int c = 0; c < FM; ++c) f[FN + c] = lds_frag(sa, wm * WM + c * 32 + r32, chunk);
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int c = 0; c < FM; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[a], f[FN + c], acc[a][c], 0, 0, 0);
  };
  // scheduling hint for one sub-step: each MFMA followed by at most one LDS
  // read, one LDS write, one global load and eight vector-ALU instructions
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < FN * FM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using TrMain = std::integral_constant<bool, kTrW>;
  using NoTr = std::integral_constant<bool, false>;

  // Main segment.  TW: DtlTile (bf16 weight), Nf4Tile or Nf4TileT (codes in registers).
  auto main_loop = [&](DtlTile<BM, NW>& ta, auto& tw, int64_t steps) {
    using TW = std::remove_reference_t<decltype(tw)>;
    constexpr bool kRegW = !std::is_same_v<TW, DtlTile<BN, NW>>;
    using WRegs = typename RegsOf<TW, kRegW>::type;
    const int64_t last = steps - 1;
    WRegs wr[3];
    auto wfetch = [&](WRegs& r, int64_t e) {  // steps past the end re-read the last one
      if constexpr (kRegW) tw.load(r, (e < last ? e : last) * kBK);
    };
    auto copy = [&](int64_t e, uint16_t* sa, uint16_t* sw) {
      const int64_t k = (e < last ? e : last) * kBK;
      ta.load(sa, wv, k);
      if constexpr (!kRegW) tw.load(sw, wv, k);
    };
    wfetch(wr[0], 0);
    wfetch(wr[1], 1);
    wfetch(wr[2], 2);
    copy(0, s_act0, s_wt0);
    if constexpr (kRegW) tw.store(wr[0], s_wt0, tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Frags f0, f1;
    read_frags(f0, s_wt0, s_act0, 0, TrMain{});
    // Step e: stage B holds step e; code set (C + 1) % 3 holds step e + 1 and
    // set C (step e's, consumed) takes step e + 3.
    auto step = [&](int64_t e, auto bc, auto cc) {
      constexpr int B = decltype(bc)::value, C = decltype(cc)::value;
      uint16_t* const sa = s_act[B];
      uint16_t* const sw = s_wt[B];
      uint16_t* const na = s_act[B ^ 1];
      uint16_t* const nw = s_wt[B ^ 1];
      WRegs& nxt = wr[(C + 1) % 3];
      Nf4Table tab{};
      auto part = [&](int d) {  // a quarter of step e+1's weight tile
        if constexpr (kRegW) {
          if constexpr (TW::kDw == 4) {
            tw.store_part(nxt, tab, nw, tid, d);
          } else {
            tw.store_part(nxt, tab, nw, tid, 2 * d);
            tw.store_part(nxt, tab, nw, tid, 2 * d + 1);
          }
        }
      };
      copy(e + 1, na, nw);
      wfetch(wr[C], e + 3);
      __builtin_amdgcn_s_setprio(1);  // the MFMA phase issues ahead of the other wave's loads
      if constexpr (kRegW) tab = TW::table(nxt);
      part(0);
      read_frags(f1, sw, sa, 1, TrMain{});
      mfmas(f0);
      interleave();
      part(1);
      read_frags(f0, sw, sa, 2, TrMain{});
      mfmas(f1);
      interleave();
      part(2);
      read_frags(f1, sw, sa, 3, TrMain{});
      mfmas(f0);
      interleave();
      part(3);
      mfmas(f1);
      interleave();
      __builtin_amdgcn_s_setprio(0);
      // stage B^1 complete and stage B free: wait for this wave's copies and
      // LDS writes (the code loads issued after the copies, 3 instructions,
      // may stay in flight), then the barrier
      if constexpr (kRegW) __builtin_amdgcn_s_waitcnt(0x73);  // vmcnt(3) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      read_frags(f0, nw, na, 0, TrMain{});
    };
    int64_t e = 0;
    for (; e + 6 <= steps; e += 6) {
      step(e, I0{}, I0{});
      step(e + 1, I1{}, I1{});
      step(e + 2, I0{}, I2{});
      step(e + 3, I1{}, I0{});
      step(e + 4, I0{}, I1{});
      step(e + 5, I1{}, I2{});
    }
    const int64_t rem = steps - e;
    if (rem > 0) step(e, I0{}, I0{});
    if (rem > 1) step(e + 1, I1{}, I1{});
    if (rem > 2) step(e + 2, I0{}, I2{});
    if (rem > 3) step(e + 3, I1{}, I0{});
    if (rem > 4) step(e + 4, I0{}, I1{});
  };

  const int64_t s0 = p.K0 / kBK, s1 = p.K1 / kBK;
  // LoRA extension segment (a few steps): two steps copied into the two
  // stages at once, one barrier, then both computed
  auto lora_seg = [&]() {
    if (s1 <= 0) return;
    DtlTile<BM, NW> ta1;
    DtlTile<BN, NW> tw1;
    ta1.init(p.nseg > 0 ? seg_of(p, n0).act1 : p.act1, p.lda1, m0, p.M, wv, lane);
    tw1.init(p.wt1, p.ldw1, n0, p.N, wv, lane);
    for (int64_t e = 0; e < s1; e += 2) {
      const bool two = e + 1 < s1;
      __syncthreads();  // every wave is done reading both stages
      ta1.load(s_act0, wv, e * kBK);
      tw1.load(s_wt0, wv, e * kBK);
      if (two) {
        ta1.load(s_act1, wv, (e + 1) * kBK);
        tw1.load(s_wt1, wv, (e + 1) * kBK);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Frags f;
        read_frags(f, s_wt0, s_act0, j, NoTr{});
        mfmas(f);
      }
      if (two) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Frags f;
          read_frags(f, s_wt1, s_act1, j, NoTr{});
          mfmas(f);
        }
      }
    }
  };
  if (p.keep != nullptr) {
    // dropout: the adapter product alone, masked, then the base on top
    lora_seg();
    apply_keep<FN, FM>(acc, p, m0 + wm * WM, n0 + wn * WN, r32, half);
    __syncthreads();  // every wave is done reading stage 0 before the main copies
  }
  if constexpr (kW == kWNf4T) {
    DtlTile<BM, NW> ta;
    ta.init(p.act0, p.lda0, m0, p.M, wv, lane);
    Nf4TileT<BN, NT> tq;
    tq.init(p, n0, tid);
    main_loop(ta, tq, s0);
  } else if constexpr (kW == kWNf4) {
    DtlTile<BM, NW> ta;
    ta.init(p.act0, p.lda0, m0, p.M, wv, lane);
    Nf4Tile<BN, NT> tq;
    const Nf4Seg sg = seg_of(p, n0);
    tq.init(sg.codes, sg.absmax_q, sg.scale, p.K0, n0 - sg.n0, sg.rows, tid);
    main_loop(ta, tq, s0);
  } else {
    DtlTile<BM, NW> ta;
    ta.init(p.act0, p.lda0, m0, p.M, wv, lane);
    DtlTile<BN, NW> tw;
    tw.init(p.wt0, p.ldw0, n0, p.N, wv, lane);
    main_loop(ta, tw, s0);
  }
  if (p.keep == nullptr) lora_seg();

  // Epilogue: D[n][m] -> C[m][n].  A lane holds m = r32 and four
  // consecutive n per (a, c, g): written straight out, every store
  // instruction would put 32 rows' 16-byte pieces into flight.  Instead each
  // wave parks its 128 x 64 bf16 block in LDS (16 KB, rows of eight 16-byte
  // pieces, piece k of row r at slot k ^ (r % 8)) and stores it back eight
  // whole 128-byte rows per instruction.
  __syncthreads();  // every wave is done reading the stages
  uint16_t* const s_c = (wv < 2 ? s_act0 : wv < 4 ? s_act1 : wv < 6 ? s_wt0 : s_wt1) + (wv & 1) * (WM * WN);
#pragma unroll
  for (int c = 0; c < FM; ++c) {
    const int row = c * 32 + r32;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t p0 = pack_bf16x2(acc[a][c][4 * g + 0], acc[a][c][4 * g + 1]);
        const uint32_t p1 = pack_bf16x2(acc[a][c][4 * g + 2], acc[a][c][4 * g + 3]);
        const int piece = 4 * a + g;
        *reinterpret_cast<u32x2*>(s_c + row * WN + ((piece ^ (row & 7)) * 8) + 4 * half) = u32x2{p0, p1};
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's block is in LDS
#pragma unroll
  for (int i = 0; i < WM / 8; ++i) {
    const int row = 8 * i + (lane >> 3), piece = lane & 7;
    const int64_t m = m0 + wm * WM + row;
    const int64_t n = n0 + wn * WN + 8 * piece;
    const u32x4 v = *reinterpret_cast<const u32x4*>(s_c + row * WN + ((piece ^ (row & 7)) * 8));
    if (m < p.M && n < p.N) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p.C + m * p.ldc + n));
  }
}

// (explicit instantiations: the host-side launch stubs of these templates are
// otherwise not always emitted)
template __global__ void k_gemm_big<kWBf16, 256>(GemmArgs);
template __global__ void k_gemm_big<kWNf4, 256>(GemmArgs);
template __global__ void k_gemm_big<kWNf4T, 256>(GemmArgs);
template __global__ void k_gemm_big<kWBf16, 128>(GemmArgs);
template __global__ void k_gemm_big<kWNf4, 128>(GemmArgs);
template __global__ void k_gemm_big<kWNf4T, 128>(GemmArgs);

// Split-K of the 128 x 128 kernel: up to 1024 rows, a grid below one
// workgroup per CU (of a 256-CU part; the count depends on the shape only, so
// workspace sizes do not depend on the device) splits K into up to 8 ranges
// of at least 8 K-steps, one workgroup each, with at most 32 MiB of fp32
// partials.  1: no split.
int gemm_splits(int64_t M, int64_t N, int64_t K) {
  constexpr int64_t kTarget = 256, kMaxSplits = 8, kMinSteps = 8, kMaxRows = 1024;
  constexpr int64_t kMaxPartBytes = int64_t(32) << 20;
  if (M <= 0 || N <= 0 || M > kMaxRows) return 1;
  if (ceil_div(M, 128) * ceil_div(N, 256) >= kTarget) return 1;  // a 256-column kernel
  const int64_t tiles = ceil_div(M, 128) * ceil_div(N, 128);
  int64_t S = kTarget / tiles;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S > K / kBK / kMinSteps) S = K / kBK / kMinSteps;
  if (S > kMaxPartBytes / (M * N * 4)) S = kMaxPartBytes / (M * N * 4);
  return S > 1 ? static_cast<int>(S) : 1;
}

size_t gemm_split_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = gemm_splits(M, N, K);
  return S > 1 ? static_cast<size_t>(S) * M * N * 4 : 0;
}

namespace {
// Tile shape of a launch.  The 8-wave kernel takes 256-column tiles of
// 256 rows when they fill at least one wave of CUs (one tile per CU at a
// time), else of 128 rows when those do (N = 1024 at T = 8192: 128 tiles of
// 256 x 256, 256 of 128 x 256); smaller grids take the 4-wave 128 x 128
// kernel.  (128-row tiles measured slower than 256-row ones also where they
// would fill the last wave better: the 8B MLP's 896 tiles = 3.5 waves.)
struct TileChoice {
  int bm, bn;  // bn 256: k_gemm_big<., bm>; bn 128: k_gemm<128, 128, ...>
};
TileChoice choose_tiles(int64_t M, int64_t N) {
  const int cus0 = device_cus();
  const int64_t cus = cus0 > 0 ? cus0 : 256;
  if (ceil_div(M, 256) * ceil_div(N, 256) >= cus) return {256, 256};
  if (ceil_div(M, 128) * ceil_div(N, 256) >= cus) return {128, 256};
  return {128, 128};
}

template <int kW>
hipError_t launch_tiles(const GemmArgs& a0, hipStream_t s, float* part = nullptr, size_t part_bytes = 0) {
  const TileChoice tc = choose_tiles(a0.M, a0.N);
  GemmArgs a = a0;
  const int S = gemm_splits(a.M, a.N, a.K0);
  if (tc.bn == 128 && S > 1 && part != nullptr && part_bytes >= gemm_split_bytes(a.M, a.N, a.K0)) {
    // split-K: S partial products, then their ordered sum
    a.part = part;
    a.ks = ceil_div(a.K0 / kBK, S);
    const int Sr = static_cast<int>(ceil_div(a.K0 / kBK, a.ks));  // splits that hold K-steps
    dim3 grid(static_cast<uint32_t>(ceil_div(a.M, 128)), static_cast<uint32_t>(ceil_div(a.N, 128)),
              static_cast<uint32_t>(Sr));
    hipLaunchKernelGGL((k_gemm<128, 128, 2, 2, kW>), grid, dim3(256), 0, s, a);
    const int64_t threads = a.M * (a.N / 8);
    hipLaunchKernelGGL(k_split_sum, dim3(static_cast<uint32_t>(ceil_div(threads, 256))), dim3(256), 0, s,
                       static_cast<const float*>(part), Sr, a.M, a.N, a.N, a.C, a.ldc);
    return hipGetLastError();
  }
  a.part = nullptr;
  if (tc.bn == 256) {
    dim3 grid(static_cast<uint32_t>(ceil_div(a.M, tc.bm)), static_cast<uint32_t>(ceil_div(a.N, 256)));
    if (tc.bm == 256) hipLaunchKernelGGL((k_gemm_big<kW, 256>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_gemm_big<kW, 128>), grid, dim3(512), 0, s, a);
  } else {
    dim3 grid(static_cast<uint32_t>(ceil_div(a.M, 128)), static_cast<uint32_t>(ceil_div(a.N, 128)));
    hipLaunchKernelGGL((k_gemm<128, 128, 2, 2, kW>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_nt(int64_t M, int64_t N, const uint16_t* act0, int64_t lda0,
                          const uint16_t* wt0, int64_t ldw0, int64_t K0, const uint16_t* act1,
                          int64_t lda1, const uint16_t* wt1, int64_t ldw1, int64_t K1, uint16_t* C,
                          int64_t ldc, hipStream_t s, const uint8_t* keep, int64_t ldk,
                          float keep_scale, float* part, size_t part_bytes) {
  GemmArgs a{};
  a.M = M; a.N = N; a.act0 = act0; a.lda0 = lda0; a.wt0 = wt0; a.ldw0 = ldw0; a.nseg = 0; a.K0 = K0;
  a.act1 = act1; a.lda1 = lda1; a.wt1 = wt1; a.ldw1 = ldw1; a.K1 = K1; a.C = C; a.ldc = ldc;
  a.keep = keep; a.ldk = ldk; a.keep_scale = keep_scale;
  return launch_tiles<kWBf16>(a, s, part, part_bytes);
}

hipError_t launch_gemm_nt_proj(int64_t M, int nproj, const int64_t* rows, const uint16_t* const* act1,
                               const uint16_t* act0, int64_t lda0, const uint16_t* wt0, int64_t ldw0,
                               int64_t K0, int64_t lda1, const uint16_t* wt1, int64_t ldw1, int64_t K1,
                               uint16_t* C, int64_t ldc, hipStream_t s, float* part, size_t part_bytes) {
  if (nproj < 1 || nproj > kMaxProj) return hipErrorInvalidValue;
  GemmArgs a{};
  a.M = M; a.act0 = act0; a.lda0 = lda0; a.wt0 = wt0; a.ldw0 = ldw0; a.K0 = K0;
  a.lda1 = lda1; a.wt1 = wt1; a.ldw1 = ldw1; a.K1 = K1; a.C = C; a.ldc = ldc;
  int64_t n = 0;
  for (int i = 0; i < nproj; ++i) n += rows[i];
  a.N = n;
  const int64_t tile = choose_tiles(M, n).bn;
  for (int i = 0; i + 1 < nproj; ++i)
    if (rows[i] % tile != 0) return hipErrorInvalidValue;  // a tile would straddle two projections
  a.nseg = nproj;
  int64_t n0 = 0;
  for (int i = 0; i < nproj; ++i) {
    a.seg[i] = Nf4Seg{nullptr, nullptr, nullptr, n0, rows[i], act1[i]};
    n0 += rows[i];
  }
  return launch_tiles<kWBf16>(a, s, part, part_bytes);
}

bool gemm_proj_aligned(int64_t M, int nproj, const int64_t* rows) {
  int64_t n = 0;
  for (int i = 0; i < nproj; ++i) n += rows[i];
  const int64_t tile = choose_tiles(M, n).bn;
  for (int i = 0; i + 1 < nproj; ++i)
    if (rows[i] % tile != 0) return false;
  return true;
}

hipError_t launch_gemm_nf4(int64_t M, int nproj, const Nf4Proj* proj, const uint16_t* act0,
                           int64_t lda0, int64_t K0, int64_t lda1, const uint16_t* wt1,
                           int64_t ldw1, int64_t K1, uint16_t* C, int64_t ldc, hipStream_t s,
                           float* part, size_t part_bytes) {
  if (nproj < 1 || nproj > kMaxProj) return hipErrorInvalidValue;
  GemmArgs a{};
  a.M = M; a.act0 = act0; a.lda0 = lda0; a.K0 = K0; a.lda1 = lda1; a.wt1 = wt1; a.ldw1 = ldw1;
  a.K1 = K1; a.ldc = ldc;
  int64_t n = 0;
  for (int i = 0; i < nproj; ++i) n += proj[i].rows;
  a.N = n;
  // one launch when no tile straddles two projections, else one per projection
  const int64_t tile = choose_tiles(M, n).bn;
  bool aligned = true;
  for (int i = 0; i + 1 < nproj; ++i) aligned = aligned && (proj[i].rows % tile == 0);
  if (aligned) {
    a.nseg = nproj;
    int64_t n0 = 0;
    for (int i = 0; i < nproj; ++i) {
      a.seg[i] = Nf4Seg{proj[i].codes, proj[i].absmax_q, proj[i].scale, n0, proj[i].rows, proj[i].act1};
      n0 += proj[i].rows;
    }
    a.C = C;
    return launch_tiles<kWNf4>(a, s, part, part_bytes);
  }
  int64_t n0 = 0;
  for (int i = 0; i < nproj; ++i) {
    GemmArgs b = a;
    b.N = proj[i].rows;
    b.nseg = 1;
    b.seg[0] = Nf4Seg{proj[i].codes, proj[i].absmax_q, proj[i].scale, 0, proj[i].rows, proj[i].act1};
    b.wt1 = wt1 + n0 * ldw1;
    b.C = C + n0;
    const hipError_t e = launch_tiles<kWNf4>(b, s);
    if (e != hipSuccess) return e;
    n0 += proj[i].rows;
  }
  return hipSuccess;
}

hipError_t launch_gemm_nf4t(int64_t M, int64_t N, int nproj, const Nf4Proj* proj, const uint16_t* act0,
                            int64_t lda0, const uint16_t* act1, int64_t lda1, const uint16_t* wt1,
                            int64_t ldw1, int64_t K1, uint16_t* C, int64_t ldc, hipStream_t s,
                            const uint8_t* keep, int64_t ldk, float keep_scale, float* part,
                            size_t part_bytes) {
  if (nproj < 1 || nproj > kMaxProj) return hipErrorInvalidValue;
  GemmArgs a{};
  a.M = M; a.N = N; a.act0 = act0; a.lda0 = lda0; a.nseg = nproj;
  int64_t k = 0;
  for (int i = 0; i < nproj; ++i) {
    if (proj[i].rows <= 0 || proj[i].rows % kBK != 0 || !nf4t_fits(proj[i].rows, N)) return hipErrorInvalidValue;
    a.seg[i] = Nf4Seg{proj[i].codes, proj[i].absmax_q, proj[i].scale, k, proj[i].rows, act1};
    k += proj[i].rows;
  }
  a.K0 = k;
  a.act1 = act1; a.lda1 = lda1; a.wt1 = wt1; a.ldw1 = ldw1; a.K1 = K1;
  a.C = C; a.ldc = ldc;
  a.keep = keep; a.ldk = ldk; a.keep_scale = keep_scale;
  return launch_tiles<kWNf4T>(a, s, part, part_bytes);
}

bool nf4t_fits(int64_t rows, int64_t in) { return rows * (in / 2) <= 0x7fffffff; }

}  // namespace qlora
