// nf4_format.hpp -- constants of the NF4 + double-quant format and the
// register-level dequantization primitives shared by the gfx950 kernels.
//
// Format (ultralytics glossary "QLoRA", "Como funciona a QLoRA", NF4 and
// double-quantization bullets; paperclase lesson "QLoRA", Partes 2-4):
//   block  = 64 consecutive weights of the row-major flattening, one absmax
//   group  = 256 consecutive blocks, one fp32 scale; absmax stored as 8 bits
//   code   = 4-bit index into 16 ascending levels, code 7 = exact zero
//   packed = element 2i in the low nibble of byte i, element 2i+1 in the high
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;
constexpr int kGroup = 256;
constexpr int kGroupElems = kBlock * kGroup;  // 16384 weights per scale

// The 16 NF4 levels as fp32 bit patterns: the quantile construction of the
// ultralytics "QLoRA" listing (normal quantiles at evenly spaced
// probabilities from 0.9677083 to 0.5, 8 positive and 7 negative, an exact
// zero, sorted, divided by the largest) evaluated in IEEE fp32.
constexpr uint32_t kLevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24du, 0xbe3d353fu,
    0xbdba7870u, 0x00000000u, 0x3da2faffu, 0x3e24cae3u, 0x3e7c04ddu, 0x3ead033au,
    0x3ee1a4b8u, 0x3f1007aau, 0x3f3913b3u, 0x3f800000u};

__host__ __device__ constexpr float level(int j) { return __builtin_bit_cast(float, kLevelBits[j]); }

// ---------------------------------------------------------------------------
// Code thresholds, derived at compile time from the levels.
//
// The code of x is the first index minimising |fl32(x - L_j)| (paperclase
// "QLoRA", Parte 4: argmin of the distance).  Both fl32(x - L_j) and
// fl32(L_{j+1} - x) are monotone in x, and a non-neighbouring level is never
// within an fp32 rounding of the nearest one (the smallest level gap, 0.08, is
// far above an ulp), so the code is a step function of x:
//   code(x) = #{ j : x > t_j },
// with t_j the largest fp32 x in [L_j, L_{j+1}) for which L_j still wins
// (ties go to the lower index).  t_j is found by bisection over the ordered
// fp32 bit patterns of that interval.
// ---------------------------------------------------------------------------
namespace detail {
constexpr float cabs(float v) { return v < 0.0f ? -v : v; }
constexpr int32_t ordered(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? -static_cast<int32_t>(u & 0x7fffffffu) : static_cast<int32_t>(u);
}
constexpr float from_ordered(int32_t o) {
  return o >= 0 ? __builtin_bit_cast(float, static_cast<uint32_t>(o))
                : __builtin_bit_cast(float, static_cast<uint32_t>(-o) | 0x80000000u);
}
constexpr bool lower_wins(float x, int j) { return cabs(x - level(j)) <= cabs(x - level(j + 1)); }
constexpr float threshold(int j) {
  int32_t lo = ordered(level(j));      // L_j itself: lower level wins
  int32_t hi = ordered(level(j + 1));  // L_{j+1}: upper level wins
  while (hi - lo > 1) {
    const int32_t mid = lo + (hi - lo) / 2;
    if (lower_wins(from_ordered(mid), j)) lo = mid; else hi = mid;
  }
  return from_ordered(lo);
}
struct Thresholds { float t[15]; };
constexpr Thresholds make_thresholds() {
  Thresholds r{};
  for (int j = 0; j < 15; ++j) r.t[j] = threshold(j);
  return r;
}
}  // namespace detail

constexpr detail::Thresholds kThresholds = detail::make_thresholds();

static_assert(kThresholds.t[6] < 0.0f && kThresholds.t[7] > 0.0f, "zero must be code 7");
static_assert(__builtin_bit_cast(uint32_t, kThresholds.t[0]) == 0xbf591cd9u, "t0");
static_assert(__builtin_bit_cast(uint32_t, kThresholds.t[14]) == 0x3f5c89d9u, "t14");

// ---------------------------------------------------------------------------
// The quantizer's per-weight arithmetic without a division or 15 comparisons.
//
// Quotient.  The code depends on x = fl32(w / a) only through comparisons
// with the thresholds, so the kernel needs x exactly.  It works on
// X = fl32(w / b) with b = a / 16, which is 16 x exactly (scaling by a power
// of two commutes with rounding away from underflow), and with the block's
// y = fl32(1 / b), one IEEE division per block:
//   q0 = fl(w y) is within 1.5 ulp of w / b;
//   q1 = fl(q0 + fl(w - b q0) y) is then a faithful quotient;
//   with y correctly rounded and q1 faithful, w - b q1 is exact (one fma)
//   and fl(q1 + (w - b q1) y) is the correctly rounded w / b (Markstein's
//   theorem on division by fused multiply-add, as given in Muller et al.,
//   Handbook of Floating-Point Arithmetic, chapter on FMA-based division).
// The theorem needs y normal and the remainder representable: for
// 2^-90 <= a <= 2^120 and |X| >= 1/2 (all thresholds lie beyond 0.63 in X)
// the remainder is a multiple of 2^-141, exact even if subnormal; smaller |X|
// is code 7 whatever its last bits.  Blocks outside that range (far from
// any real weight block) divide directly.
//
// Lookup.  code(X) = #{j : X > 16 t_j}.  The thresholds are at least 0.08
// apart, more than the 1/16 that one unit of X spans, so each interval
// [k, k + 1), k = -16..16, holds at most one scaled threshold: with base_k
// the number below the interval and thr_k the one inside it (+inf if none),
// code(X) = base_k + (X > thr_k), k = floor(X).  X = 16 (the block maximum)
// falls in k = 16.
// ---------------------------------------------------------------------------
constexpr float kFastAbsmaxMin = 0x1p-90f;
constexpr float kFastAbsmaxMax = 0x1p120f;

// fl32(w / b) from y = fl32(1 / b), for b and w as above
__host__ __device__ inline float div_by_reciprocal(float w, float b, float y) {
  float q = w * y;
  float r = __builtin_fmaf(-b, q, w);
  q = __builtin_fmaf(r, y, q);
  r = __builtin_fmaf(-b, q, w);
  return __builtin_fmaf(r, y, q);
}

constexpr int kBuckets = 33;  // k = -16..16 at index k + 16
struct BucketTable {
  uint32_t word[2 * kBuckets];  // entry i: word[2i] = fp32 bits of thr, word[2i + 1] = base
};

namespace detail {
constexpr float scaled_threshold(int j) { return 16.0f * kThresholds.t[j]; }
constexpr BucketTable make_buckets() {
  BucketTable tb{};
  for (int i = 0; i < kBuckets; ++i) {
    const float lo = static_cast<float>(i - 16), hi = lo + 1.0f;
    uint32_t base = 0;
    float thr = __builtin_inff();
    for (int j = 0; j < 15; ++j) {
      const float T = scaled_threshold(j);
      if (T < lo) ++base;
      else if (T < hi) thr = T;
    }
    tb.word[2 * i] = __builtin_bit_cast(uint32_t, thr);
    tb.word[2 * i + 1] = base;
  }
  return tb;
}
// at most one scaled threshold per unit interval, and scaling by 16 exact
constexpr bool buckets_hold_one_threshold() {
  for (int j = 0; j < 15; ++j) {
    if (j > 0 && scaled_threshold(j) - scaled_threshold(j - 1) <= 1.0f) return false;
    if (scaled_threshold(j) / 16.0f != kThresholds.t[j]) return false;
  }
  return true;
}
}  // namespace detail

static_assert(detail::buckets_hold_one_threshold(), "bucket lookup needs thresholds > 1/16 apart");
constexpr BucketTable kBucketTable = detail::make_buckets();
static_assert(kBucketTable.word[2 * 32 + 1] == 15 && kBucketTable.word[2 * 16 + 1] == 7, "bucket bases");

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __builtin_bit_cast(float, p & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Double-quantized absmax: a_hat = fl32(fl32(q / 255) * s).
// fl32(q / 255) without a division: r0 = fl32(q * c) with c = fl32(1/255),
// then one FMA correction r0 + fl32(q - 255 r0) * c.  For every q in 0..255
// this equals the correctly rounded quotient (checked exhaustively on the
// host in the tests, and on the GPU by dequantizing all 256 codes); it costs
// three instructions instead of the ~10 of an IEEE division.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dq_absmax(uint32_t q, float s) {
  constexpr float kInv255 = 0x1.010102p-8f;  // fl32(1 / 255)
  const float qf = static_cast<float>(q);
  const float r0 = __fmul_rn(qf, kInv255);
  const float e = __builtin_fmaf(-r0, 255.0f, qf);
  const float ratio = __builtin_fmaf(e, kInv255, r0);
  return __fmul_rn(ratio, s);
}

// ---------------------------------------------------------------------------
// Per-block product table and 8-codes-at-a-time lookup with v_perm_b32.
//
// For one block, entry j is bf16_rne(fl32(L_j * a_hat)).  The 16 entries are
// kept as two byte planes of 16 bytes: lo[] holds the low bytes, hi[] the high
// bytes, entry 4i..4i+3 in dword i.  v_perm_b32(S0, S1, sel) picks each output
// byte from the 8 bytes {S1 = bytes 0..3, S0 = bytes 4..7}, so one perm looks
// up 4 codes in an 8-entry half-plane; a second perm does the other half and
// a third picks per byte by bit 3 of the code.
// ---------------------------------------------------------------------------
struct Nf4Table {
  uint32_t lo[4];
  uint32_t hi[4];
};

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

__device__ __forceinline__ Nf4Table make_table(float ahat) {
  uint32_t d[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float p0 = level(2 * k) * ahat;
    const float p1 = level(2 * k + 1) * ahat;
    d[k] = pack_bf16x2(p0, p1);  // entry 2k in bits 0-15, 2k+1 in bits 16-31
  }
  Nf4Table t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.lo[i] = perm(d[2 * i + 1], d[2 * i], 0x06040200u);
    t.hi[i] = perm(d[2 * i + 1], d[2 * i], 0x07050301u);
  }
  return t;
}

// Looks up 4 codes, one per byte of `sel` (values 0..7 after masking) with
// `pick` = 0x03020100 | (bit3 of each code << 2) per byte.  The pick is one
// v_bitop3 ((x & 0x04040404) | 0x03020100, truth table 0xEA) on the shifted
// codes instead of an and + or.
__device__ __forceinline__ uint32_t lookup_plane(const uint32_t (&plane)[4], uint32_t sel, uint32_t pick) {
  const uint32_t a = perm(plane[1], plane[0], sel);
  const uint32_t b = perm(plane[3], plane[2], sel);
  return perm(b, a, pick);
}

// 8 codes (one packed dword, element e in nibble e) -> bf16 values.
// Output order "split": out[0] = (w0, w2), out[1] = (w4, w6), out[2] = (w1, w3),
// out[3] = (w5, w7) -- each dword is two bf16, lower element in bits 0-15.
__device__ __forceinline__ void lookup8_split(const Nf4Table& t, uint32_t c, uint32_t out[4]) {
  const uint32_t sel_e = c & 0x07070707u;
  const uint32_t pick_e = __builtin_amdgcn_bitop3_b32(c >> 1, 0x04040404u, 0x03020100u, 0xEA);
  const uint32_t sel_o = (c >> 4) & 0x07070707u;
  const uint32_t pick_o = __builtin_amdgcn_bitop3_b32(c >> 5, 0x04040404u, 0x03020100u, 0xEA);
  const uint32_t el = lookup_plane(t.lo, sel_e, pick_e);  // byte i = lo(w_{2i})
  const uint32_t eh = lookup_plane(t.hi, sel_e, pick_e);
  const uint32_t ol = lookup_plane(t.lo, sel_o, pick_o);  // byte i = lo(w_{2i+1})
  const uint32_t oh = lookup_plane(t.hi, sel_o, pick_o);
  out[0] = perm(eh, el, 0x05010400u);  // (w0, w2)
  out[1] = perm(eh, el, 0x07030602u);  // (w4, w6)
  out[2] = perm(oh, ol, 0x05010400u);  // (w1, w3)
  out[3] = perm(oh, ol, 0x07030602u);  // (w5, w7)
}

// Same, natural order: out[k] = (w_{2k}, w_{2k+1}).
__device__ __forceinline__ void lookup8(const Nf4Table& t, uint32_t c, uint32_t out[4]) {
  uint32_t s[4];
  lookup8_split(t, c, s);
  out[0] = perm(s[2], s[0], 0x05040100u);  // (w0, w1)
  out[1] = perm(s[2], s[0], 0x07060302u);  // (w2, w3)
  out[2] = perm(s[3], s[1], 0x05040100u);  // (w4, w5)
  out[3] = perm(s[3], s[1], 0x07060302u);  // (w6, w7)
}

// The element order lookup8_split produces within each aligned group of 8:
// position p of the 8 output bf16 holds element kSplitOrder[p].
constexpr int kSplitOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};

// Reorders 8 bf16 (as 4 dwords, natural order) into the split order, so an
// activation fragment lines up with lookup8_split output.
__device__ __forceinline__ void to_split_order(const uint32_t in[4], uint32_t out[4]) {
  out[0] = perm(in[1], in[0], 0x05040100u);  // (x0, x2)
  out[1] = perm(in[3], in[2], 0x05040100u);  // (x4, x6)
  out[2] = perm(in[1], in[0], 0x07060302u);  // (x1, x3)
  out[3] = perm(in[3], in[2], 0x07060302u);  // (x5, x7)
}

}  // namespace qlora
