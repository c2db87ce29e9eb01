// Read references for the benchmark (not part of the library's ABI):
// - a streaming read: every byte of a buffer read once with 16-byte loads in a
//   grid-stride loop, one value stored per block so the loads are kept.  Its rate
//   is the HBM read rate a plain kernel reaches on this GPU, the reference the
//   benchmark quotes fractions against beside the 8 TB/s vendor figure;
// - a row gather: random 1 KB rows, 32 to a chunk, by blocks of 8 waves, the way
//   decode attention gathers its items, either through the asynchronous
//   global -> LDS copies (four 32-row stages, three chunks in flight, one barrier
//   per chunk) or with plain 16-byte loads into registers (one chunk in flight per
//   block).  No arithmetic: the two rates are what each way of gathering reaches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace {

using namespace sckv;

__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

constexpr int kGRows = 32;                 // rows per chunk
constexpr int kGWaves = 8;
constexpr int kGStages = 4;

// wait until at most n (a multiple of the per-chunk copy count, <= N) copies are outstanding
template <int N>
__device__ __forceinline__ void wait_copies(int n) {
  if constexpr (N == 0) {
    wait_vm_lgkm<0, 0>();
  } else {
    if (n >= N) wait_vm_lgkm<N, 0>();
    else wait_copies<N - 1>(n);
  }
}

template <bool LDS_COPY>
__global__ __launch_bounds__(kGWaves * 64) void gather_rows(const uint8_t* __restrict__ base,
                                                           const int32_t* __restrict__ rows, int nch,
                                                           uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[LDS_COPY ? kGStages * kGRows * 1024 : 16];
  constexpr int RPW = kGRows / kGWaves;
  const int w = wave_id(), l = lane_id();
  const int32_t* my = rows + (int64_t)blockIdx.x * nch * kGRows;
  const gbytes gb = opaque_global(base);
  uint32_t acc = 0;
  if constexpr (LDS_COPY) {
    auto issue = [&](int c) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int rr = __builtin_amdgcn_readfirstlane(my[c * kGRows + w * RPW + i]);
        copy_to_lds16(gb + (int64_t)rr * 1024 + l * 16, &stg[((c % kGStages) * kGRows + w * RPW + i) * 1024]);
      }
    };
    for (int c = 0; c < kGStages - 1 && c < nch; ++c) issue(c);
    for (int c = 0; c < nch; ++c) {
      const int ahead = (nch - 1 - c) < (kGStages - 2) ? (nch - 1 - c) : (kGStages - 2);
      wait_copies<(kGStages - 2) * RPW>(ahead * RPW);
      block_barrier();                                   // chunk c landed; the stage of c - 1 is free
      if (c + kGStages - 1 < nch) issue(c + kGStages - 1);
      acc ^= stg[((c % kGStages) * kGRows + (l & (kGRows - 1))) * 1024 + w];
    }
  } else {
    for (int c = 0; c < nch; ++c) {
      u32x4 v[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int rr = __builtin_amdgcn_readfirstlane(my[c * kGRows + w * RPW + i]);
        v[i] = gload<u32x4>(gb, (int64_t)rr * 1024 + l * 16);
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) acc ^= v[i][0];
    }
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

// Gathers `blocks` x `nch` chunks of 32 rows of 1 KB from `base` (device): chunk c
// of block b reads rows rows[(b * nch + c) * 32 + i] (int32, device, each < the
// number of 1 KB rows at base).  lds_copy != 0 gathers through the asynchronous
// global -> LDS copies, 0 with loads into registers.  `sink` holds `blocks` uint32
// (device).  Returns a hipError_t.
extern "C" int sckv_bench_gather_rows(const void* base, const int32_t* rows, int blocks, int nch, int lds_copy,
                                      void* sink, void* stream) {
  if (!base || !rows || !sink || blocks < 1 || nch < 1) return (int)hipErrorInvalidValue;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* b = static_cast<const uint8_t*>(base);
  auto* k = static_cast<uint32_t*>(sink);
  if (lds_copy) hipLaunchKernelGGL(gather_rows<true>, dim3((unsigned)blocks), dim3(kGWaves * 64), 0, s, b, rows, nch, k);
  else hipLaunchKernelGGL(gather_rows<false>, dim3((unsigned)blocks), dim3(kGWaves * 64), 0, s, b, rows, nch, k);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from device memory `p` with `grid` blocks of 256
// threads; `sink` holds `grid` uint32 (device).  Returns a hipError_t.
extern "C" int sckv_bench_stream_read(const void* p, size_t bytes, void* sink, int grid, void* stream) {
  if (!p || !sink || grid < 1 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(p), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}
