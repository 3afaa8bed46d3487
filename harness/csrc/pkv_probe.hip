// pkv_probe.hip — plain HBM streaming kernels, a yardstick for the decode
// kernel's bandwidth (not part of the attention path).
//
//   pkv_probe_read(x, bytes, sink, stream)   reads every byte of x once
//       (16 B per lane, non-temporal, grid-stride) and writes one word per
//       thread to sink so the loads are kept; bytes must be a multiple of 16.
//   pkv_probe_read_slabs(x, bytes, sink, blocks, stream)  the same read as
//       contiguous 16 KB slabs per workgroup (1 KB per instruction) over
//       `blocks` workgroups of 4 waves (at most the grid above); bytes must be
//       a multiple of 16 KB.
//   pkv_probe_copy(dst, src, bytes, stream)  copies bytes (multiple of 16):
//       a kernel of known traffic for calibrating hardware byte counters.
//   pkv_probe_grid(void)  threads the probes launch (size of sink, in words).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 256 * 8;   // 8 workgroups per compute unit

}  // namespace

__global__ __launch_bounds__(kThreads) void pkv_probe_read_kernel(const u32x4* __restrict__ x, int64_t n,
                                                        uint32_t* __restrict__ sink) {
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(x + i);
    const u32x4 b = __builtin_nontemporal_load(x + i + stride);
    const u32x4 c = __builtin_nontemporal_load(x + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(x + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(x + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[tid] = acc;
}

// Contiguous slabs: each workgroup reads 16 KB slabs (4 KB per wave, 1 KB per
// instruction), two slabs in flight, slabs taken grid-stride.
constexpr int64_t kSlab = 16384;
__global__ __launch_bounds__(kThreads) void pkv_probe_read_slabs_kernel(const uint8_t* __restrict__ x,
                                                              int64_t nslabs,
                                                              uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t off = (int64_t)wave * 4096 + lane * 16;
  uint32_t acc = 0;
  int64_t s = blockIdx.x;
  for (; s + gridDim.x < nslabs; s += 2 * (int64_t)gridDim.x) {
    const uint8_t* a = x + s * kSlab + off;
    const uint8_t* b = x + (s + gridDim.x) * kSlab + off;
    u32x4 r[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a + 1024 * j));
      r[4 + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + 1024 * j));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= r[j][0] ^ r[j][1] ^ r[j][2] ^ r[j][3];
  }
  for (; s < nslabs; s += gridDim.x) {
    const uint8_t* a = x + s * kSlab + off;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a + 1024 * j));
      acc ^= r[0] ^ r[1] ^ r[2] ^ r[3];
    }
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void pkv_probe_copy_kernel(u32x4* __restrict__ dst,
                                                        const u32x4* __restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

extern "C" {

int32_t pkv_probe_grid(void) { return kBlocks * kThreads; }

int32_t pkv_probe_read(const void* x, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!x || !sink || bytes % 16) return 1;
  hipLaunchKernelGGL(pkv_probe_read_kernel, dim3(kBlocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(x),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t pkv_probe_read_slabs(const void* x, uint64_t bytes, uint32_t* sink, int32_t blocks,
                             void* stream) {
  if (!x || !sink || bytes % kSlab || blocks < 1 || blocks > kBlocks) return 1;
  hipLaunchKernelGGL(pkv_probe_read_slabs_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(x),
                     (int64_t)(bytes / kSlab), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t pkv_probe_copy(void* dst, const void* src, uint64_t bytes, void* stream) {
  if (!dst || !src || bytes % 16) return 1;
  hipLaunchKernelGGL(pkv_probe_copy_kernel, dim3(kBlocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
