// probe_kernels.hip -- streaming ceilings of this GPU, for context next to the
// roofline fraction of the state kernels.  Two shapes, both 256 threads per
// workgroup with 16-byte nontemporal lane loads, every load instruction
// covering consecutive bytes, and the XCD-aware tile order:
//   PER = 8: 32 KiB per workgroup, eight loads in flight per thread -- the
//            replay step's shape, with nothing else in the way;
//   PER = 1: 4 KiB per workgroup, one load per thread, so that a wave lives
//            for one memory round trip.  Measured on the MI355X this pure
//            stream moves more bytes per second than the 32 KiB shape; a
//            kernel with a per-workgroup chain before its output (index read,
//            prologue, barriers) cannot take it, which is why it is a
//            ceiling for context, not a target shape.
#include "common.hpp"
#include "launch.hpp"

namespace rssm {
namespace {

constexpr int NT = 256;

// Read-only: every workgroup streams its tile and folds each wave's words by
// XOR.  check != 0: every wave writes its fold to the sink.  check == 0
// (timing): only a wave whose fold equals `key` writes, so the loads cannot be
// dropped while the stream carries (almost) no stores -- with 4 KiB tiles one
// 4-byte store per wave would cost a tenth of the read rate.
constexpr uint32_t kProbeKey = 0x9E3779B9u;

template <int PER>
__global__ __launch_bounds__(NT) void probe_read_kernel(const u32x4* src, float* sink, int check) {
  constexpr int TILE = PER * NT;   // 16-byte chunks per workgroup
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
  if ((threadIdx.x & 63) == 0 && (check || x == kProbeKey))
    sink[t * (NT / 64) + (threadIdx.x >> 6)] = __uint_as_float(x);
}

// Copy: every workgroup reads its tile and writes it to the destination.
template <int PER>
__global__ __launch_bounds__(NT) void probe_copy_kernel(const u32x4* src, u32x4* dst) {
  constexpr int TILE = PER * NT;
  const long t = tile_index();
  const u32x4* p = src + t * TILE + threadIdx.x;
  u32x4* q = dst + t * TILE + threadIdx.x;
  u32x4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = __builtin_nontemporal_load(p + k * NT);
#pragma unroll
  for (int k = 0; k < PER; ++k) __builtin_nontemporal_store(v[k], q + k * NT);
}

template <int PER>
void launch_probe_per(const void* src, void* dst, float* sink, long tiles, int check,
                      hipStream_t s) {
  if (dst)
    hipLaunchKernelGGL((probe_copy_kernel<PER>), dim3((unsigned)tiles), dim3(NT), 0, s,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst));
  else
    hipLaunchKernelGGL((probe_read_kernel<PER>), dim3((unsigned)tiles), dim3(NT), 0, s,
                       static_cast<const u32x4*>(src), sink, check);
}

}  // namespace

hipError_t launch_probe(const void* src, void* dst, float* sink, long tiles, int tile_bytes,
                        int check, hipStream_t s) {
  if (tile_bytes == 4096)
    launch_probe_per<1>(src, dst, sink, tiles, check, s);
  else
    launch_probe_per<8>(src, dst, sink, tiles, check, s);
  return hipGetLastError();
}

}  // namespace rssm
