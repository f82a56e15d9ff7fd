// index_kernels.hip -- buffer-pointer operations.
//
// Rollback (explainer, "Cheap speculative decoding rollback"): rejecting the
// last k speculative tokens moves the buffer tail back by k; ring contents
// and checkpoints are not touched.  A request that would move the tail before
// the checkpoint (k > len) or k < 0 is refused and flagged.
#include "common.hpp"
#include "launch.hpp"

namespace rssm {
namespace {

__global__ __launch_bounds__(256) void rollback_kernel(const int64_t* pos, int32_t* len,
                                                       uint32_t* status, const int32_t* n_reject,
                                                       int batch, int cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int32_t n = n_reject[b];
  const int32_t l = len[b];
  if (!indices_valid(l, pos[b], cap))
    raise_status(status, kStatusIndex);
  else if (n < 0 || n > l)
    raise_status(status, kStatusRollback);
  else
    len[b] = l - n;
}

__global__ void clear_status_kernel(uint32_t* status) {
  if (threadIdx.x == 0) status[0] = 0u;
}

}  // namespace

hipError_t launch_rollback(int64_t* pos, int32_t* len, uint32_t* status,
                           const int32_t* n_reject, int batch, int cap, hipStream_t s) {
  const unsigned blocks = (unsigned)((batch + 255) / 256);
  hipLaunchKernelGGL(rollback_kernel, dim3(blocks), dim3(256), 0, s, pos, len, status, n_reject,
                     batch, cap);
  return hipGetLastError();
}

hipError_t launch_clear_status(uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, s, status);
  return hipGetLastError();
}

}  // namespace rssm
