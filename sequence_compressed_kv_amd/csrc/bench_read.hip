// Streaming-read reference for the benchmark (not part of the library's ABI):
// every byte of a buffer read once with 16-byte loads in a grid-stride loop, one
// value stored per block so the loads are kept.  Its rate is the HBM read rate a
// plain kernel reaches on this GPU, the reference the benchmark quotes fractions
// against beside the 8 TB/s vendor figure.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device memory `p` with `grid` blocks of 256
// threads; `sink` holds `grid` uint32 (device).  Returns a hipError_t.
extern "C" int sckv_bench_stream_read(const void* p, size_t bytes, void* sink, int grid, void* stream) {
  if (!p || !sink || grid < 1 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(p), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}
