// Pure-read bandwidth probe: the same coalesced dwordx4 buffer loads (with the
// same non-temporal hint) as the GEMV weight streams over a given byte range,
// folded with xor so nothing is elided.
// It measures what the part delivers for a read-once stream of that size.
#include "device.hpp"
#include "launch.hpp"

namespace qgemv {

constexpr int kCeilThreads = 256;
constexpr int kCeilLoads = 8;  // dwordx4 per thread, issued back to back
constexpr int64_t kCeilSpan = (int64_t)kCeilThreads * kCeilLoads * 16;  // bytes per workgroup

__global__ __launch_bounds__(kCeilThreads) void read_ceiling_kernel(const uint8_t* __restrict__ buf,
                                                                    int64_t bytes,
                                                                    float* __restrict__ sink) {
  __shared__ unsigned part[kCeilThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kCeilSpan;
  const int64_t left = bytes - base;
  const auto r = make_rsrc(buf + base, (uint32_t)(left < kCeilSpan ? left : kCeilSpan));
  u32x4 v[kCeilLoads];
#pragma unroll
  for (int u = 0; u < kCeilLoads; ++u)
    v[u] = ld128w(r, (uint32_t)((u * kCeilThreads + threadIdx.x) * 16));
  unsigned acc = 0;
#pragma unroll
  for (int u = 0; u < kCeilLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1)
    acc ^= (unsigned)__builtin_amdgcn_ds_bpermute((__lane_id() ^ s) << 2, (int)acc);
  if (__lane_id() == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
    for (int i = 0; i < kCeilThreads / 64; ++i) t ^= part[i];
    sink[blockIdx.x] = __builtin_bit_cast(float, t);
  }
}

int64_t read_sink_len(int64_t bytes) { return (bytes + kCeilSpan - 1) / kCeilSpan; }

hipError_t launch_read_ceiling(const void* buf, int64_t bytes, float* sink, hipStream_t s) {
  const int64_t grid = read_sink_len(bytes);
  hipLaunchKernelGGL(read_ceiling_kernel, dim3((unsigned)grid), dim3(kCeilThreads), 0, s,
                     (const uint8_t*)buf, bytes, sink);
  return hipGetLastError();
}

}  // namespace qgemv
