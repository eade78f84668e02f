// Small utility kernels: initial-state copy for empty sequences and the
// streaming copy used to calibrate hardware byte counters.
#include "../../include/ttt_tuning.h"
#include "ttt_launch.h"

namespace ttt {

__global__ void copy_state_kernel(const float* __restrict__ src, int per_unit, int H, int n,
                                  float* __restrict__ dst) {
  const int u = blockIdx.y;
  const float* s = src + (size_t)(per_unit ? u : u % H) * n;
  float* d = dst + (size_t)u * n;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) d[i] = s[i];
}

hipError_t launch_copy_state(const float* src, int per_unit, int units, int H, int n, float* dst,
                             hipStream_t s) {
  return launch(copy_state_kernel, dim3((n + 255) / 256, units), dim3(256), s, src, per_unit, H, n,
                dst);
}

__global__ void __launch_bounds__(256) stream_copy_kernel(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

}  // namespace ttt

extern "C" ttt_status_t ttt_bench_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return TTT_ERR_NULL;
  if ((bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return TTT_ERR_ALIGN;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (bytes && a < b + bytes && b < a + bytes) return TTT_ERR_ALIAS;
  if (bytes == 0) return TTT_OK;
  const size_t n = bytes / 16;
  size_t blocks = (n + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  const hipError_t e = ttt::launch(ttt::stream_copy_kernel, dim3((unsigned)blocks), dim3(256),
                                   (hipStream_t)stream, (const uint4*)src, (uint4*)dst, n);
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}
