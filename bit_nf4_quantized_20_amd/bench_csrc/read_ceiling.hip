// read_ceiling.hip -- measurement support, not part of the QLoRA library:
// the fastest plain read of a device buffer in one launch, the practical
// ceiling a single small-token forward launch streaming a weight of the
// same size can be held against.
//
// Every thread issues all of its 16-byte loads first (kPer of them, a grid
// stride apart, so each wave instruction reads 1 KB contiguous), then folds
// them with XOR.  The result is stored only if it equals a constant no
// buffer of interest produces, so the loads stay live while the launch
// writes (almost surely) nothing.  Built into its own library
// (libqlora_bench.so) for the bench's calibration leg.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr uint32_t kNever = 0x9E3779B9u;
constexpr int kBufferWord3 = 0x00020000;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int kPer>
__global__ __launch_bounds__(512) void k_read_ceiling(const uint8_t* __restrict__ src, uint32_t bytes,
                                                      uint32_t* __restrict__ sink) {
  // offsets past the end read zero (raw buffer bounds check): no branch
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, static_cast<int>(bytes), kBufferWord3);
  const uint32_t stride = gridDim.x * blockDim.x * 16u;
  const uint32_t first = (blockIdx.x * blockDim.x + threadIdx.x) * 16u;
  u32x4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, first + i * stride, 0, 0));
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  if (acc == kNever) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, below 2^31) of device memory at `src`
// with `threads` (256 or 512) per workgroup and `per` (1, 2, 4 or 8) loads
// per thread, on `stream`.  `sink` must hold one uint32 per launched thread
// (ceil(bytes / (16 * per * threads)) * threads of them); it is written only
// in the practically impossible case above.  Returns 0, or -1 for invalid
// arguments, -2 for a launch error.
int qlora_bench_read_ceiling(const void* src, int64_t bytes, int threads, int per, uint32_t* sink,
                             void* stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 31))
    return -1;
  if (threads != 256 && threads != 512) return -1;
  if (per != 1 && per != 2 && per != 4 && per != 8) return -1;
  const int64_t per_wg = int64_t(16) * per * threads;
  const dim3 grid(static_cast<uint32_t>((bytes + per_wg - 1) / per_wg));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* p = static_cast<const uint8_t*>(src);
  const uint32_t b = static_cast<uint32_t>(bytes);
  switch (per) {
    case 1: hipLaunchKernelGGL(k_read_ceiling<1>, grid, dim3(threads), 0, s, p, b, sink); break;
    case 2: hipLaunchKernelGGL(k_read_ceiling<2>, grid, dim3(threads), 0, s, p, b, sink); break;
    case 4: hipLaunchKernelGGL(k_read_ceiling<4>, grid, dim3(threads), 0, s, p, b, sink); break;
    default: hipLaunchKernelGGL(k_read_ceiling<8>, grid, dim3(threads), 0, s, p, b, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
