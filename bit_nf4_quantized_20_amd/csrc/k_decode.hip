// k_decode.hip -- fused QLoRA linear forward for small token counts
// (T <= 16), HBM-bound on the packed-nibble weight stream.
//
//   Y = X W_hat^T + s (X A^T) B^T     (paperclase lesson "QLoRA", Parte 4)
//
// Decomposition.  Workgroup (g, k) owns R = 128 output rows (8 tiles of 16)
// and one K slice of whole 256-wide units; the slices of a row group are
// spread over workgroups so the grid fills the chip while each workgroup
// reads only its slice of X and A (the activation traffic is what limits a
// small-token GEMV, not the 0.52 B/weight of codes).  Because the LoRA term
// is linear in U = X A^T, each slice adds s * U_slice B^T to its own partial,
// and the row group's result is the sum of its slices' partials.
//
// Inside a workgroup: the X slice [T][KS] and A slice [r][KS] are staged in
// LDS once, already in MFMA-fragment order.  Wave w owns row tile w; in unit
// u its lane (n = l%16, g = l/16) owns block 4u+g of row n: 32 code bytes, the
// block's 16-entry bf16 table, then 8 dwords of codes through the v_perm
// lookup straight into the A operand of v_mfma_f32_16x16x32_bf16 (16 rows x
// 16 tokens x 32 k) with the activation fragment as B operand.  Waves
// 0..units-1 also compute the unit's U partial (A rows as MFMA A operand).
//
// Cross-workgroup reduction, deterministic: each workgroup stores its fp32
// partial [T][R] to the workspace slot of its slice (device-coherent stores),
// then takes a ticket from the row group's counter with one fetch-add.  The
// workgroup holding the last ticket sums the slices in slice order, rounds to
// bf16 once, writes Y and returns the counter to zero, so the counter region
// must be zero when a call starts and is zero again when it ends.
#include "common.hpp"
#include "nf4_format.hpp"

namespace qlora {

typedef float f32x4v __attribute__((ext_vector_type(4)));

namespace {
constexpr int kWaves = 8;
constexpr int kR = 128;           // rows per row group (8 tiles of 16)
// 256-wide units per slice, bounded so the staged A fragments fit in LDS
constexpr int max_ups(int rt) { return rt <= 1 ? 4 : (rt == 2 ? 2 : 1); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

struct DecodeGeom {
  int64_t units;      // ceil(in / 256)
  int ups;            // units per slice
  int slices;         // slices per row group
};

DecodeGeom decode_geom(int64_t in, int64_t out, int64_t r) {
  DecodeGeom d;
  d.units = ceil_div(in, 256);
  const int kMaxUps = max_ups(static_cast<int>(ceil_div(r, 16)));
  const int64_t groups = ceil_div(out, kR);
  int64_t want = ceil_div(256, groups);  // slices per group for ~256 workgroups
  if (want < 1) want = 1;
  int64_t ups = ceil_div(d.units, want);
  if (ups > kMaxUps) ups = kMaxUps;
  if (ups < 1) ups = 1;
  d.ups = static_cast<int>(ups);
  d.slices = static_cast<int>(ceil_div(d.units, ups));
  return d;
}
}  // namespace

size_t decode_workspace_bytes(int64_t in, int64_t out, int64_t r) {
  const DecodeGeom d = decode_geom(in, out, r);
  return static_cast<size_t>(d.slices) * 16 * static_cast<size_t>(out) * 4;  // fp32 partials
}

int64_t decode_counter_count(int64_t out) { return ceil_div(out, kR); }

template <int RT>  // rank tiles of 16 (r <= 16 * RT)
__global__ __launch_bounds__(kWaves * 64) void k_decode_fwd(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ absmax_q,
    const float* __restrict__ scale, int64_t in, const uint16_t* __restrict__ X, int T,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r, float s,
    uint16_t* __restrict__ Y, int64_t out, int ups, int slices, float* __restrict__ partials,
    uint32_t* __restrict__ counters) {
  constexpr int kMaxUps = max_ups(RT);
  // activation / A fragments: [unit][step j][lane] x 16 B
  __shared__ u32x4 s_x[kMaxUps][8][64];
  __shared__ u32x4 s_a[kMaxUps][RT][8][64];
  __shared__ f32x4v s_u[kMaxUps][RT][64];
  __shared__ float s_uf[RT * 16][17];        // U_slice^T [j][t]
  __shared__ float s_b[kR][RT * 16 + 1];     // B rows of the group, fp32
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t grp = blockIdx.x, slc = blockIdx.y;
  const int64_t r0 = grp * kR;
  const int64_t units = ceil_div(in, 256);
  const int64_t u0 = slc * ups;
  const int nu = static_cast<int>(u0 + ups <= units ? ups : units - u0);
  const int64_t kblocks = in / 64;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  // the last row group may hold only 64 rows (out % 128 == 64)
  const int rows_valid = static_cast<int>(out - r0 < kR ? out - r0 : kR);
  const bool tile_ok = 16 * wv < rows_valid;

  // -- 1. the HBM stream first: this wave's codes for all units of the slice
  const int64_t row = r0 + 16 * wv + n;
  u32x4 c[kMaxUps][2];
  uint32_t qv[kMaxUps];
  float sv[kMaxUps];
  bool okv[kMaxUps];
#pragma unroll
  for (int i = 0; i < kMaxUps; ++i) {
    const int64_t kb = 4 * (u0 + i) + g;
    okv[i] = tile_ok && i < nu && kb < kblocks;
    if (okv[i]) {
      const u32x4* src = reinterpret_cast<const u32x4*>(codes + ((row * in + kb * 64) >> 1));
      c[i][0] = __builtin_nontemporal_load(src);
      c[i][1] = __builtin_nontemporal_load(src + 1);
      const int64_t bi = (row * in) / 64 + kb;
      qv[i] = absmax_q[bi];
      sv[i] = scale[bi >> 8];
    } else {
      c[i][0] = c[i][1] = zero4;
      qv[i] = 0u;
      sv[i] = 0.f;
    }
  }

  // -- 2. stage X and A slices in fragment order, and the group's B rows.
  // Fragment (u, j, lane l) = 8 bf16 at k = 256u + 64*(l/16) + 8j of token /
  // rank row l%16.
  for (int idx = tid; idx < nu * 8 * 64; idx += kWaves * 64) {
    const int u = idx / 512, rem = idx % 512, j = rem / 64, l = rem % 64;
    const int t = l & 15;
    const int64_t k = (u0 + u) * 256 + 64 * (l >> 4) + 8 * j;
    u32x4 v = zero4;
    if (t < T && k < in) v = *reinterpret_cast<const u32x4*>(X + static_cast<int64_t>(t) * in + k);
    s_x[u][j][l] = v;
  }
  for (int idx = tid; idx < nu * RT * 8 * 64; idx += kWaves * 64) {
    const int u = idx / (RT * 512), rem = idx % (RT * 512);
    const int rt = rem / 512, rem2 = rem % 512, j = rem2 / 64, l = rem2 % 64;
    const int jr = rt * 16 + (l & 15);
    const int64_t k = (u0 + u) * 256 + 64 * (l >> 4) + 8 * j;
    u32x4 v = zero4;
    if (jr < r && k < in) v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(jr) * in + k);
    s_a[u][rt][j][l] = v;
  }
  for (int idx = tid; idx < kR * RT * 16; idx += kWaves * 64) {
    const int rr = idx / (RT * 16), j = idx % (RT * 16);
    float v = 0.f;
    if (j < r && rr < rows_valid)
      v = __builtin_bit_cast(float, static_cast<uint32_t>(B[(r0 + rr) * r + j]) << 16);
    s_b[rr][j] = v;
  }
  __syncthreads();

  // -- 3. base product of this wave's row tile, and U of unit wv
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMaxUps; ++i) {
    if (i >= nu) break;
    const float ahat = okv[i] ? dq_absmax(qv[i], sv[i]) : 0.f;
    const Nf4Table tab = make_table(ahat);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t cw = j < 4 ? c[i][0][j] : c[i][1][j - 4];
      uint32_t w[4];
      lookup8(tab, cw, w);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}),
                                                    as_bf16x8(s_x[i][j][lane]), acc, 0, 0, 0);
    }
  }
  if (wv < nu) {
    f32x4v au[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) au[rt] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8 xb = as_bf16x8(s_x[wv][j][lane]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        au[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s_a[wv][rt][j][lane]), xb, au[rt],
                                                         0, 0, 0);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) s_u[wv][rt][lane] = au[rt];
  }
  __syncthreads();
  // U_slice^T[j][t] = sum over the slice's units; lane holds D[4g+i][n]
  if (wv < RT) {
    f32x4v su = {0.f, 0.f, 0.f, 0.f};
    for (int u = 0; u < nu; ++u) su += s_u[u][wv][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) s_uf[wv * 16 + 4 * g + i][n] = su[i];
  }
  __syncthreads();

  // -- 4. partial of this slice: base + s * U_slice B^T, rows 16*wv + 4g + i
  const int t = n;
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 16 * wv + 4 * g + i;
    float lora = 0.f;
#pragma unroll 8
    for (int j = 0; j < RT * 16; ++j) lora += s_uf[j][t] * s_b[rr][j];
    y[i] = acc[i] + s * lora;
  }
  if (t < T && tile_ok) {
    // device-coherent stores (written through to the coherence point shared
    // by all XCDs), so the reducing workgroup can read them without any
    // cache-wide writeback or invalidate
    uint64_t* dst = reinterpret_cast<uint64_t*>(partials + (slc * 16 + t) * out + r0 + 16 * wv + 4 * g);
    const uint64_t v01 = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, y[0])) |
                         (static_cast<uint64_t>(__builtin_bit_cast(uint32_t, y[1])) << 32);
    const uint64_t v23 = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, y[2])) |
                         (static_cast<uint64_t>(__builtin_bit_cast(uint32_t, y[3])) << 32);
    __hip_atomic_store(dst, v01, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dst + 1, v23, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // -- 5. the last slice to finish reduces the row group.  The stores above
  // are acknowledged (vmcnt 0) before the barrier, hence before the counter
  // update; the reducer reads the partials with device-coherent loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t ticket = __hip_atomic_fetch_add(counters + grp, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == static_cast<uint32_t>(slices - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // T x 128 outputs, 4 consecutive rows per thread
  const int tt = tid >> 5, rq = (tid & 31) * 4;
  if (tt < T && rq < rows_valid) {
    f32x4v sum = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < slices; ++k) {
      uint64_t* src = reinterpret_cast<uint64_t*>(
          partials + (static_cast<int64_t>(k) * 16 + tt) * out + r0 + rq);
      const uint64_t v01 = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t v23 = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sum += f32x4v{__builtin_bit_cast(float, static_cast<uint32_t>(v01)),
                    __builtin_bit_cast(float, static_cast<uint32_t>(v01 >> 32)),
                    __builtin_bit_cast(float, static_cast<uint32_t>(v23)),
                    __builtin_bit_cast(float, static_cast<uint32_t>(v23 >> 32))};
    }
    const uint32_t p0 = pack_bf16x2(sum[0], sum[1]);
    const uint32_t p1 = pack_bf16x2(sum[2], sum[3]);
    *reinterpret_cast<u32x2*>(Y + static_cast<int64_t>(tt) * out + r0 + rq) = u32x2{p0, p1};
  }
  // every slice of this group has taken its ticket: reset for the next call
  if (tid == 0) __hip_atomic_store(counters + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_decode_fwd(const uint8_t* codes, const uint8_t* absmax_q, const float* scale,
                             int64_t in, int64_t out, const uint16_t* X, int64_t T,
                             const uint16_t* A, const uint16_t* B, int64_t r, float s,
                             uint16_t* Y, void* ws, uint32_t* counters, hipStream_t st) {
  const DecodeGeom d = decode_geom(in, out, r);
  const dim3 grid(static_cast<uint32_t>(ceil_div(out, kR)), static_cast<uint32_t>(d.slices));
  const dim3 block(kWaves * 64);
  float* partials = static_cast<float*>(ws);
  const int rt = static_cast<int>(ceil_div(r, 16));
  const int iT = static_cast<int>(T), ir = static_cast<int>(r);
#define QLORA_DEC(RTV)                                                                            \
  hipLaunchKernelGGL((k_decode_fwd<RTV>), grid, block, 0, st, codes, absmax_q, scale, in, X, iT, \
                     A, B, ir, s, Y, out, d.ups, d.slices, partials, counters)
  if (rt <= 1) QLORA_DEC(1);
  else if (rt <= 2) QLORA_DEC(2);
  else if (rt <= 4) QLORA_DEC(4);
  else return hipErrorInvalidValue;
#undef QLORA_DEC
  return hipGetLastError();
}

}  // namespace qlora
