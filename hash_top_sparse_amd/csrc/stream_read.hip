// stream_read.hip -- read-only streaming reduction over a device buffer, used
// to measure the HBM read rate this device reaches with a plain kernel (the
// "measured peak" a roofline can be set against besides the published one).
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

constexpr int kStreamBlocks = 1024;  // sink words (grid at most this many workgroups)
constexpr int kStreamUnroll = 16;    // 16-byte loads in flight per thread

// Workgroup b reads the contiguous segment [b*seg, (b+1)*seg) of the buffer
// (in 16-byte units) with streaming loads, kStreamUnroll per thread in
// flight, folds it with XOR and writes one word, so no read can be elided.
__global__ __launch_bounds__(kNT) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          int64_t seg, uint64_t* __restrict__ sink) {
  __shared__ uint32_t part[kNT / 64];
  const int t = threadIdx.x;
  const int64_t beg = (int64_t)blockIdx.x * seg, end = min(n16, beg + seg);
  uint32_t acc = 0;
  int64_t i = beg + t;
  for (; i + (kStreamUnroll - 1) * kNT < end; i += kStreamUnroll * kNT) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = load_stream16(src + i + u * kNT);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kNT) {
    const uint4 v = load_stream16(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // fold the wave, then the workgroup
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((t & 63) == 0) part[t >> 6] = acc;
  __syncthreads();
  if (t == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kNT / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

int stream_read_blocks() { return kStreamBlocks; }

hipError_t launch_stream_read(const void* src, size_t bytes, uint64_t* sink, int blocks, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t seg = (n16 + blocks - 1) / blocks;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kNT), 0, s, static_cast<const uint4*>(src),
                     n16, seg, sink);
  // unused sink words stay as they are; a caller folding sink[0 .. 1024)
  // clears it first
  return hipGetLastError();
}

}  // namespace hata
