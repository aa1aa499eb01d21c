// stream_read.hip -- a pure HBM read stream: the measured ceiling that the
// weight-streaming GEMV kernels are compared against (the blueprint's
// card.json prices every kernel floor at a measured read bandwidth, 249 GB/s
// against the part's 273 GB/s nominal; this is the MI355X counterpart).
//
// Each wavefront reads 4 KiB of contiguous memory with the same 128-bit
// non-temporal loads the GEMV uses for codes (lane l takes bytes 16 l +
// 1024 j, j < 4), folds the words with XOR and writes one word only when the
// fold equals a constant no input is expected to produce, so the loads cannot
// be removed. One wavefront per 4 KiB and no persistence, the launch shape of
// the M = 1 GEMV; a sweep of 4, 8 and 16 KiB per wavefront measured 4 KiB
// fastest from 28 MB to 350 MB.
#include "device.h"
#include "internal.h"

namespace nvfp4 {

namespace {

constexpr int kReadUnroll = 4;            // 1 KiB loads per wavefront
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4_t* __restrict__ p, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  const size_t wave = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t base = wave * (64 * kReadUnroll) + (threadIdx.x & 63);
  u32x4_t v[kReadUnroll];
#pragma unroll
  for (int j = 0; j < kReadUnroll; ++j) {
    const size_t i = base + (size_t)j * 64;
    v[j] = i < n16 ? load_stream(p + i) : u32x4_t{0u, 0u, 0u, 0u};
  }
  u32x4_t acc = v[0];
#pragma unroll
  for (int j = 1; j < kReadUnroll; ++j) acc ^= v[j];
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == kSinkMagic) sink[0] = r;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                              hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t waves = (n16 + 64 * kReadUnroll - 1) / (64 * kReadUnroll);
  const size_t grid = (waves + 3) / 4;
  if (grid > 0x7FFFFFFFu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace nvfp4
