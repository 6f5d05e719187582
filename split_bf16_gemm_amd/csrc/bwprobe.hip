// bwprobe.hip -- plain streaming kernels that measure the HBM ceiling of the
// device they run on, a copy of known size whose profiler byte counters
// calibrate the counters of the GEMM kernel, and an empty kernel that times
// the fixed cost of a launch.  Not part of the GEMM path.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b reads its own contiguous share of the buffer, four 16-byte
// non-temporal loads in flight per thread, and folds them with xor; one word
// per thread is written so the loads cannot be dropped.  On MI355X this was
// the fastest plain read measured (48 MiB in 9.0 us per launch at 1024
// workgroups; grid-stride and default-policy loads were 5-10 % slower).
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                   uint32_t* __restrict__ sink) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t begin = (size_t)blockIdx.x * per;
  const size_t end = begin + per < n ? begin + per : n;
  u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = x0, x2 = x0, x3 = x0;
  size_t i = begin + threadIdx.x;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    x0 ^= __builtin_nontemporal_load(src + i);
    x1 ^= __builtin_nontemporal_load(src + i + 256);
    x2 ^= __builtin_nontemporal_load(src + i + 2 * 256);
    x3 ^= __builtin_nontemporal_load(src + i + 3 * 256);
  }
  for (; i < end; i += 256) x0 ^= __builtin_nontemporal_load(src + i);
  const u32x4 x = x0 ^ x1 ^ x2 ^ x3;
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

// Does nothing.  Back-to-back launches of it with the GEMM's grid time the
// fixed cost of a launch of that shape (dispatch, workgroup start and end,
// the end-of-kernel release), below which no kernel of that grid can go.
__global__ __launch_bounds__(256) void empty_kernel() {}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from `src` with `blocks` workgroups of 256
// threads; `sink` must hold blocks*256 uint32.  Returns a hipError_t.
int bwprobe_read(const void* src, size_t bytes, void* sink, int blocks, void* stream) {
  if (!src || !sink || bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16) from `src` to `dst`.  Returns a hipError_t.
int bwprobe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

// Launches the empty kernel with `blocks` workgroups of 256 threads.
// Returns a hipError_t.
int bwprobe_empty(int blocks, void* stream) {
  if (blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}

}  // extern "C"
