// HBM stream probe for the benchmark: a measurement aid, not part of the
// method and not part of libkvsel.so.  Plain HBM streams that set the rate a
// call of a given size can reach on this GPU.  READ folds src into one
// 16-byte XOR word per workgroup (so the loads cannot be dropped); COPY copies
// src to dst.  Both use 16-byte non-temporal accesses, four per thread in
// flight, over a fixed grid of KVSEL_PROBE_BLOCKS workgroups with a
// grid-stride loop, so every workgroup moves the same share of the buffer.
//
// C ABI of libkvsel_probe.so (one entry point, asynchronous on `stream`):
//   int kvsel_probe_stream(int32_t mode, const void* src, void* dst,
//                          int64_t bytes, hipStream_t stream);
//   mode 0 (read): dst receives KVSEL_PROBE_BLOCKS 16-byte folds whose XOR is
//          the XOR of all of src's 16-byte words; mode 1 (copy): dst = src.
//   src, dst: device pointers, 16-byte aligned, not overlapping; bytes > 0, a
//   multiple of 16.  Returns 0, or 1 (nothing enqueued) for a bad argument,
//   or 4 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define KVSEL_PROBE_BLOCKS 2048

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeBlocks = KVSEL_PROBE_BLOCKS;

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ fold,
                                                              int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n;
       base += step) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  __shared__ u32x4 part[kThreads];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) part[threadIdx.x] ^= part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) fold[blockIdx.x] = part[0];
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst,
                                                              int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n;
       base += step) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace

extern "C" int kvsel_probe_stream(int32_t mode, const void* src, void* dst, int64_t bytes,
                                  hipStream_t stream) {
  if (mode != 0 && mode != 1) return 1;
  if (!src || !dst || (((uintptr_t)src | (uintptr_t)dst) % 16)) return 1;
  if (bytes <= 0 || bytes % 16) return 1;
  const int64_t n = bytes / 16;
  auto s = static_cast<const u32x4*>(src);
  auto d = static_cast<u32x4*>(dst);
  if (mode == 0)
    probe_read_kernel<<<dim3(kProbeBlocks), dim3(kThreads), 0, stream>>>(s, d, n);
  else
    probe_copy_kernel<<<dim3(kProbeBlocks), dim3(kThreads), 0, stream>>>(s, d, n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
