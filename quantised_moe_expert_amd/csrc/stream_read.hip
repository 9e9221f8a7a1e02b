// Streaming-read reference kernel, built into a library of its own
// (libsmoe_stream.so) for the benchmark: it reads a buffer once from HBM
// with 16-byte loads and nothing else, so that, timed exactly as the layer
// kernels are (an event pair around each launch, buffers rotated so that no
// launch finds its bytes in the caches), it shows what one launch of the
// same byte count can reach on this GPU. It is no part of the MoE path.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kUnroll = 4;  // independent 16-byte loads in flight per lane

// Workgroup b reads the b-th of gridDim.x contiguous spans (a multiple of
// kThreads * kUnroll 16-byte words each, the last one shorter), so each
// wave streams whole 1 KB lines. One word per workgroup is written to keep
// the loads live.
template <bool NT>
__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4* __restrict__ src,
                                                          uint64_t n16, uint64_t span,
                                                          uint32_t* __restrict__ sink) {
  const uint64_t lo = (uint64_t)blockIdx.x * span;
  const uint64_t hi = lo + span < n16 ? lo + span : n16;
  uint32_t acc = 0;
  uint64_t i = lo + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * kThreads) : src[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kThreads) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // combine across the workgroup only to keep one store per workgroup
  __shared__ uint32_t red[kThreads / 64];
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

extern "C" {

// Reads nbytes at src (16-byte aligned, a multiple of 16) with nwg
// workgroups of 512 threads, with non-temporal loads when nontemporal != 0;
// writes nwg words to sink. Returns 0 or the HIP error code (1 for invalid
// arguments, nothing launched).
int smoe_stream_read(const void* src, uint64_t nbytes, uint32_t* sink, int nwg, int nontemporal,
                     void* hip_stream) {
  if (!src || !sink || nbytes == 0 || nbytes % 16 || (uintptr_t)src % 16 || nwg < 1 ||
      nwg > 65535)
    return 1;
  const uint64_t n16 = nbytes / 16;
  const uint64_t chunk = (uint64_t)kThreads * kUnroll;
  uint64_t span = (n16 + nwg - 1) / nwg;
  span = (span + chunk - 1) / chunk * chunk;
  if (nontemporal)
    hipLaunchKernelGGL(k_stream_read<true>, dim3(nwg), dim3(kThreads), 0,
                       (hipStream_t)hip_stream, (const u32x4*)src, n16, span, sink);
  else
    hipLaunchKernelGGL(k_stream_read<false>, dim3(nwg), dim3(kThreads), 0,
                       (hipStream_t)hip_stream, (const u32x4*)src, n16, span, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
