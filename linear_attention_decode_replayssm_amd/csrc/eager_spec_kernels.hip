// eager_spec_kernels.hip -- the eager comparator for speculative decoding.
//
// Without a checkpoint and an input buffer, verifying n drafts and keeping
// the option to roll back to any of them means materialising the state after
// every draft (Abstract: ReplaySSM verifies drafts from their outputs without
// materialising intermediate states; explainer, "Cheap speculative decoding
// rollback").  This comparator does exactly that, as cheaply as it can: the
// state of a sequence is read once from slot cur[b] of a ring of n + 1 state
// slots, the n drafts are applied in registers with the eager recurrence, and
// the state after draft j is written to slot (cur[b] + 1 + j) % (n + 1), so
// that accepting a drafts is a move of cur[b] by a.  Per round: one state
// read and n state writes, against ReplaySSM's one read and no write.
#include "common.hpp"
#include "launch.hpp"

namespace rssm {
namespace {

constexpr int NT = 256;

// Mamba-2: one workgroup per (sequence, head); thread t owns float4 column
// c4 = t % 32 of state rows r0 + 8k (r0 = t / 32), as the eager kernel.
constexpr int MP = 64, MN = 128, MLPR = MN / 4, MRPL = NT / MLPR, MNLD = MP / MRPL;

__global__ __launch_bounds__(NT) void m2_eager_spec_kernel(M2Args a, float* slots,
                                                           const int32_t* cur) {
  const int tile = tile_index();
  const int b = tile / a.H, h = tile - b * a.H;
  const int g = h / (a.H / a.G);
  const int tid = threadIdx.x, lane = tid & 63, c4 = tid % MLPR, r0 = tid / MLPR;
  const long unit = (long)b * a.H + h, gunit = (long)b * a.G + g;
  const int n = a.n_pos, ns = n + 1;
  const long slot = (long)a.batch * a.H * MP * MN;
  const long sx = (long)a.batch * a.H * MP, sg = (long)a.batch * a.G * MN;
  const long sd = (long)a.batch * a.H;
  const float Ah = a.A[h], Dh = a.D[h];
  const int c = cur[b];
  const bool ok = c >= 0 && c < ns;
  if (!ok) {   // a corrupt slot index: outputs NaN, nothing written
    if (tid < MP)
      for (int j = 0; j < n; ++j) a.y[j * sx + unit * MP + tid] = __builtin_nanf("");
    if (tid == 0 && h == 0) raise_status(a.status, kStatusRollback);
    return;
  }
  const long e0 = unit * (MP * MN) + (long)r0 * MN + c4 * 4;
  f32x4 hv[MNLD];
#pragma unroll
  for (int k = 0; k < MNLD; ++k) hv[k] = ld_nt(slots + c * slot + e0 + (long)k * MRPL * MN);
  for (int j = 0; j < n; ++j) {
    const float dtv = a.dt[j * sd + unit];
    const float dec = expf(dtv * Ah);
    const float* xt = a.x + j * sx + unit * MP;
    const f32x4 bb = ld4(a.B + j * sg + gunit * MN + c4 * 4);
    const f32x4 cc = ld4(a.C + j * sg + gunit * MN + c4 * 4);
    float d[MNLD];
    float* dst = slots + ((c + 1 + j) % ns) * slot + e0;
#pragma unroll
    for (int k = 0; k < MNLD; ++k) {
      hv[k] = dec * hv[k] + (dtv * xt[k * MRPL + r0]) * bb;
      d[k] = dot4(hv[k], cc);
      st_nt(dst + (long)k * MRPL * MN, hv[k]);
    }
    xreduce<MNLD, MLPR>(d, lane);
    using M = XMap<MNLD, MLPR>;
    if (M::writer(lane)) {
      const int p = M::index(lane, 0) * MRPL + r0;
      a.y[j * sx + unit * MP + p] = d[0] + Dh * xt[p];
    }
  }
}

// GDN: one workgroup per half head (64 state rows), thread t owns float4
// column t % 32 of rows r0 + 8k, as the eager kernel.  Per draft and row:
// (S k)_r, S_r <- alpha S_r + beta (v_r - alpha (S k)_r) k^T, o_r = S_r . q.
constexpr int GD = 128, GROWS = 64, GLPR = GD / 4, GRPL = NT / GLPR, GNLD = GROWS / GRPL;

__global__ __launch_bounds__(NT) void gdn_eager_spec_kernel(GdnArgs a, float* slots,
                                                            const int32_t* cur) {
  const int tile = tile_index();
  const int hp = tile / (GD / GROWS), row0 = (tile - hp * (GD / GROWS)) * GROWS;
  const int b = hp / a.H, h = hp - b * a.H;
  const int tid = threadIdx.x, lane = tid & 63, cl = tid % GLPR, r0 = tid / GLPR;
  const long unit = (long)b * a.H + h;
  const int n = a.n_pos, ns = n + 1;
  const long slot = (long)a.batch * a.H * GD * GD;
  const long sk = (long)a.batch * a.H * GD, sd = (long)a.batch * a.H;
  const int c = cur[b];
  if (c < 0 || c >= ns) {   // a corrupt slot index: outputs NaN, nothing written
    if (tid < GROWS)
      for (int j = 0; j < n; ++j) a.o[j * sk + unit * GD + row0 + tid] = __builtin_nanf("");
    if (tid == 0 && h == 0 && row0 == 0) raise_status(a.status, kStatusRollback);
    return;
  }
  const long e0 = unit * (GD * GD) + (long)(row0 + r0) * GD + cl * 4;
  f32x4 hv[GNLD];
#pragma unroll
  for (int k = 0; k < GNLD; ++k) hv[k] = ld_nt(slots + c * slot + e0 + (long)k * GRPL * GD);
  for (int j = 0; j < n; ++j) {
    const f32x4 kv = ld4(a.k + j * sk + unit * GD + cl * 4);
    const f32x4 qv = ld4(a.q + j * sk + unit * GD + cl * 4);
    const float al = a.alpha[j * sd + unit], be = a.beta[j * sd + unit];
    const float* vv = a.v + j * sk + unit * GD + row0;
    float skr[GNLD], d[GNLD];
#pragma unroll
    for (int k = 0; k < GNLD; ++k) skr[k] = dot4(hv[k], kv);
    allreduce<GNLD, GLPR>(skr);
    float* dst = slots + ((c + 1 + j) % ns) * slot + e0;
#pragma unroll
    for (int k = 0; k < GNLD; ++k) {
      const float coef = be * (vv[k * GRPL + r0] - al * skr[k]);
      hv[k] = al * hv[k] + coef * kv;
      d[k] = dot4(hv[k], qv);
      st_nt(dst + (long)k * GRPL * GD, hv[k]);
    }
    xreduce<GNLD, GLPR>(d, lane);
    using M = XMap<GNLD, GLPR>;
    if (M::writer(lane)) {
      const int r = row0 + M::index(lane, 0) * GRPL + r0;
      a.o[j * sk + unit * GD + r] = d[0];
    }
  }
}

// cur[b] += n_accept[b] within the ring of n + 1 slots; a count outside 0..n
// leaves the sequence unchanged and raises RSSM_STATUS_ROLLBACK.
__global__ __launch_bounds__(256) void eager_spec_accept_kernel(int32_t* cur, uint32_t* status,
                                                                const int32_t* n_accept, int n,
                                                                int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int acc = n_accept[b], c = cur[b];
  if (acc < 0 || acc > n || c < 0 || c > n)
    raise_status(status, kStatusRollback);
  else
    cur[b] = (c + acc) % (n + 1);
}

}  // namespace

hipError_t launch_m2_eager_spec(const M2Args& a, float* slots, const int32_t* cur,
                                hipStream_t s) {
  hipLaunchKernelGGL(m2_eager_spec_kernel, dim3((unsigned)(a.batch * a.H)), dim3(NT), 0, s, a,
                     slots, cur);
  return hipGetLastError();
}

hipError_t launch_gdn_eager_spec(const GdnArgs& a, float* slots, const int32_t* cur,
                                 hipStream_t s) {
  hipLaunchKernelGGL(gdn_eager_spec_kernel, dim3((unsigned)(a.batch * a.H * (GD / GROWS))), dim3(NT),
                     0, s, a, slots, cur);
  return hipGetLastError();
}

hipError_t launch_eager_spec_accept(int32_t* cur, uint32_t* status, const int32_t* n_accept,
                                    int n, int batch, hipStream_t s) {
  const int blocks = (batch + 255) / 256;
  hipLaunchKernelGGL(eager_spec_accept_kernel, dim3((unsigned)blocks), dim3(256), 0, s, cur,
                     status, n_accept, n, batch);
  return hipGetLastError();
}

}  // namespace rssm
