// probe_kernels.hip -- streaming ceilings of this GPU, for context next to the
// roofline fraction of the state kernels: the same workgroup shape and load
// pattern as the replay step (256 threads, 32 KiB per workgroup, 16-byte
// nontemporal lane loads, every load instruction covering consecutive bytes,
// the XCD-aware tile order), with nothing else in the way.
#include "common.hpp"
#include "launch.hpp"

namespace rssm {
namespace {

constexpr int NT = 256;
constexpr int TILE = 32768 / 16;   // 16-byte chunks per workgroup
constexpr int PER = TILE / NT;     // per thread

// Read-only: every workgroup streams its 32 KiB and writes one float (so the
// loads cannot be dropped).
__global__ __launch_bounds__(NT) void probe_read_kernel(const u32x4* src, float* sink) {
  const long t = tile_index();
  const u32x4* p = src + t * TILE + threadIdx.x;
  u32x4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = __builtin_nontemporal_load(p + k * NT);
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  x ^= __float_as_uint(rpartner<32>(__uint_as_float(x)));   // fold the wave's values
  x ^= __float_as_uint(rpartner<16>(__uint_as_float(x)));
  x ^= __float_as_uint(rpartner<8>(__uint_as_float(x)));
  x ^= __float_as_uint(rpartner<4>(__uint_as_float(x)));
  x ^= __float_as_uint(rpartner<2>(__uint_as_float(x)));
  x ^= __float_as_uint(rpartner<1>(__uint_as_float(x)));
  if ((threadIdx.x & 63) == 0) sink[t * (NT / 64) + (threadIdx.x >> 6)] = __uint_as_float(x);
}

// Copy: every workgroup reads its 32 KiB and writes it to the destination.
__global__ __launch_bounds__(NT) void probe_copy_kernel(const u32x4* src, u32x4* dst) {
  const long t = tile_index();
  const u32x4* p = src + t * TILE + threadIdx.x;
  u32x4* q = dst + t * TILE + threadIdx.x;
  u32x4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = __builtin_nontemporal_load(p + k * NT);
#pragma unroll
  for (int k = 0; k < PER; ++k) __builtin_nontemporal_store(v[k], q + k * NT);
}

}  // namespace

hipError_t launch_probe(const void* src, void* dst, float* sink, long tiles, hipStream_t s) {
  if (dst)
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)tiles), dim3(NT), 0, s,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst));
  else
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)tiles), dim3(NT), 0, s,
                       static_cast<const u32x4*>(src), sink);
  return hipGetLastError();
}

}  // namespace rssm
