// prefill_kernels.hip -- prefill of a prompt into the checkpoint, for gfx950.
//
// The pages describe decode only; prefill is read here as a commit over a
// long buffer (explainer, "Periodically commit a new checkpoint": apply the
// recurrence from the checkpoint across the inputs, store the result): each
// sequence's buffered entries and then the prompt are folded into the state,
// and every prompt token also gets its output.  Unlike decode, a prefill
// keeps the state on chip for the whole prompt: it is read once and written
// once, and the work in between is dense arithmetic, so it runs on the
// matrix cores.
//
// Mamba-2 (one 256-thread workgroup per (sequence, head); wave w owns state
// rows p = 16w .. 16w+15).  The prompt goes in chunks of Q = 16 tokens.  With
// cum_j the chunk's dt prefix sum (token j included), Gamma_j = exp(A cum_j)
// and E[j][i] = C_j . B_i:
//   y_j  = Gamma_j h C_j + sum_{i<=j} exp(A (cum_j - cum_i)) dt_i E[j][i] x_i + D x_j
//   h   <- Gamma_{Q-1} h + sum_i exp(A (cum_{Q-1} - cum_i)) dt_i x_i B_i^T
// which is the eager recurrence regrouped (Mamba-2 replay form, ReplaySSM
// explainer, "Compute outputs without eagerly updating the checkpoint").  All
// three products (E, the outputs, the fold) are v_mfma_f32_16x16x4f32.
//
// MFMA operand layout (16x16x4, fp32; lane l, li = l % 16, lq = l / 16):
// A[i][k] comes from lane (i, k), B[k][j] from lane (j, k), and accumulator
// register r of lane l holds D[4 lq + r][li].  The state is kept transposed in
// accumulators: tile t, register r of lane l holds h[16w + li][16t + 4lq + r].
// The output product contracts over the state's n index, which is the
// accumulator's row index: at the step that uses register r of tile t, lane
// (li, lq) supplies B = its register and A = Gamma_li C_li[16t + 4lq + r], so
// both operands of k-slot lq name the same n and the state never moves.
#include "common.hpp"
#include "launch.hpp"
#include "lp_codec.hpp"

namespace rssm {
namespace {

constexpr int MP = 64;        // Mamba-2 head dim P (state rows)
constexpr int MN = 128;       // Mamba-2 state dim N (state columns)
constexpr int Q = 16;         // prompt tokens per chunk: one MFMA tile edge
constexpr int NT = 256;       // 4 waves, 16 state rows each
constexpr int PAD = 4;        // LDS row padding (floats) against bank conflicts
constexpr int kSchemeF32 = 0, kSchemeDual = 1, kSchemeShared = 2;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One chunk's inputs in flight: thread tid holds x_i[4c..4c+3] for
// i = tid / 16, c = tid % 16, and two float4 of B and C each (flat float4
// index tid + 256u over [Q][N/4]), dt_tid for tid < Q.
struct M2Chunk {
  f32x4 x;
  f32x4 B[2], C[2];
  float dt;
};

struct M2Pre {
  const float *ring_x, *ring_B, *ring_dt, *x, *B, *C, *dt;
  long unit, gunit, sx, sg, sd;
  int cap, slot0, nring, T;
  bool outs;
  // entries of chunk c: c < 0 is the buffer (its nring entries), c >= 0 the
  // prompt tokens c*Q .. ; returns how many are valid
  __device__ int count(int c) const { return c < 0 ? nring : min(Q, T - c * Q); }
  __device__ void fetch(int c, M2Chunk& f) const {
    const int tid = threadIdx.x, n = count(c);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const int i = tid >> 4, c4 = tid & 15;
    f.x = z;
    if (i < n)
      f.x = c < 0 ? ld4(ring_x + (unit * cap + ring_slot(slot0, i, cap)) * MP + 4 * c4)
                  : ld4(x + (long)(c * Q + i) * sx + unit * MP + 4 * c4);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * NT, e = idx >> 5, n4 = idx & 31;
      f.B[u] = z;
      f.C[u] = z;
      if (e < n) {
        f.B[u] = c < 0 ? ld4(ring_B + (gunit * cap + ring_slot(slot0, e, cap)) * MN + 4 * n4)
                       : ld4(B + (long)(c * Q + e) * sg + gunit * MN + 4 * n4);
        if (c >= 0 && outs) f.C[u] = ld4(C + (long)(c * Q + e) * sg + gunit * MN + 4 * n4);
      }
    }
    f.dt = 0.f;
    if (tid < n)
      f.dt = c < 0 ? ring_dt[unit * cap + ring_slot(slot0, tid, cap)]
                   : dt[(long)(c * Q + tid) * sd + unit];
  }
};

template <int SCHEME, int LP>
__global__ __launch_bounds__(NT) void m2_prefill_kernel(M2Args a) {
  const int tile = tile_index();
  const int b = tile / a.H, h = tile - b * a.H;
  if (a.mask && a.mask[b] == 0) return;   // the whole sequence skips: no arrival
  const int g = h / (a.H / a.G);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
  const int p = 16 * w + li;              // this lane's state row
  const int T = a.n_pos;
  const int len = a.len[b];
  const int64_t pos = a.pos[b];
  const float Ah = a.A[h], Dh = a.D[h];
  const long unit = (long)b * a.H + h;
  const long sx = (long)a.batch * a.H * MP;

  M2Pre pre;
  pre.ring_x = a.ring_x;
  pre.ring_B = a.ring_B;
  pre.ring_dt = a.ring_dt;
  pre.x = a.x;
  pre.B = a.B;
  pre.C = a.C;
  pre.dt = a.dt;
  pre.unit = unit;
  pre.gunit = (long)b * a.G + g;
  pre.sx = sx;
  pre.sg = (long)a.batch * a.G * MN;
  pre.sd = (long)a.batch * a.H;
  pre.cap = a.cap;
  pre.slot0 = (int)(pos % a.cap);
  pre.nring = min(max(len, 0), min(a.cap, Q));
  pre.T = T;
  pre.outs = a.y != nullptr;

  const int c0 = pre.nring > 0 ? -1 : 0;
  const int nch = (T + Q - 1) / Q;
  M2Chunk f;
  pre.fetch(c0, f);

  // the state, transposed into 8 accumulator tiles (see the file comment)
  f32x4 acc[8];
  const long e0 = unit * (MP * MN) + (long)p * MN + 4 * lq;   // element of tile 0
  if constexpr (SCHEME == kSchemeShared) {
    if constexpr (LP == kLpBf16) {
      const uint16_t* lp = reinterpret_cast<const uint16_t*>(a.ckpt_lp) + e0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(lp + 16 * t);
        acc[t] = f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
      }
    } else {
      const uint8_t* lp = reinterpret_cast<const uint8_t*>(a.ckpt_lp) + e0;
      const float sc = a.lp_scale[unit];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(lp + 16 * t);
        const f32x2 lo = e4m3_pair(v, false), hi = e4m3_pair(v, true);
        acc[t] = f32x4{lo.x * sc, lo.y * sc, hi.x * sc, hi.y * sc};
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = ld_nt(a.ckpt + e0 + 16 * t);
  }
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, b, len, pos);

  __shared__ __attribute__((aligned(16))) float s_x[Q][MP + PAD];
  __shared__ __attribute__((aligned(16))) float s_B[Q][MN + PAD];
  __shared__ __attribute__((aligned(16))) float s_C[Q][MN + PAD];
  __shared__ float s_dt[Q], s_cum[Q], s_gam[Q], s_fw[Q];
  __shared__ float s_E[4][Q][Q + 1];
  __shared__ float s_W[Q][Q + 1];
  __shared__ float s_red[NT / 64];

  for (int c = c0; c < nch; ++c) {
    st4(&s_x[tid >> 4][4 * (tid & 15)], f.x);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * NT;
      st4(&s_B[idx >> 5][4 * (idx & 31)], f.B[u]);
      st4(&s_C[idx >> 5][4 * (idx & 31)], f.C[u]);
    }
    if (tid < Q) s_dt[tid] = f.dt;
    __syncthreads();
    if (c + 1 < nch) pre.fetch(c + 1, f);   // the next chunk loads during this one
    const int n = pre.count(c);
    const bool out = c >= 0 && pre.outs;

    if (tid < Q) {   // decays; padded entries have dt = 0
      float cum = 0.f, tot = 0.f;
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const float d = s_dt[i];
        tot += d;
        if (i <= tid) cum += d;
      }
      s_cum[tid] = cum;
      s_gam[tid] = expf(Ah * cum);
      s_fw[tid] = expf(Ah * (tot - cum)) * s_dt[tid];
    }
    if (out) {   // this wave's part of E = C B^T: n = 32w .. 32w+31
      f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int nn = 32 * w + 4 * s + lq;
        e = mfma4(s_C[li][nn], s_B[li][nn], e);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s_E[w][4 * lq + r][li] = e[r];
    }
    __syncthreads();
    if (out) {
      {  // in-chunk weights W[j][i], causal
        const int j = tid >> 4, i = tid & 15;
        float wv = 0.f;
        if (i <= j)
          wv = (s_E[0][j][i] + s_E[1][j][i] + s_E[2][j][i] + s_E[3][j][i]) *
               expf(Ah * (s_cum[j] - s_cum[i])) * s_dt[i];
        s_W[j][i] = wv;
      }
#pragma unroll
      for (int u = 0; u < (Q * MN) / NT; ++u) {   // Gamma_j C_j in place
        const int idx = tid + u * NT, j = idx >> 7, nn = idx & 127;
        s_C[j][nn] *= s_gam[j];
      }
      __syncthreads();
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {   // Gamma_j h C_j, contracting over n
        const f32x4 cg = ld4(&s_C[li][16 * t + 4 * lq]);
        y = mfma4(cg.x, acc[t].x, y);
        y = mfma4(cg.y, acc[t].y, y);
        y = mfma4(cg.z, acc[t].z, y);
        y = mfma4(cg.w, acc[t].w, y);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)     // + sum_i W[j][i] x_i[p]
        y = mfma4(s_W[li][4 * s + lq], s_x[4 * s + lq][p], y);
#pragma unroll
      for (int r = 0; r < 4; ++r) {   // y[r] is token 4 lq + r, row p
        const int j = 4 * lq + r;
        if (j < n) a.y[(long)(c * Q + j) * sx + unit * MP + p] = y[r] + Dh * s_x[j][p];
      }
    }
    {  // fold: h <- Gamma_{Q-1} h + sum_i fw_i x_i B_i^T
      const float gq = expf(Ah * s_cum[Q - 1]);
      float bx[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bx[s] = s_fw[4 * s + lq] * s_x[4 * s + lq][p];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        acc[t] *= gq;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[t] = mfma4(s_B[4 * s + lq][16 * t + li], bx[s], acc[t]);
      }
    }
    __syncthreads();   // every read of this chunk's LDS is done
  }

  if constexpr (SCHEME != kSchemeShared) {
#pragma unroll
    for (int t = 0; t < 8; ++t) st_nt(a.ckpt + e0 + 16 * t, acc[t]);
  }
  if constexpr (SCHEME != kSchemeF32) {
    if constexpr (LP == kLpBf16) {
      uint16_t* lp = reinterpret_cast<uint16_t*>(a.ckpt_lp) + e0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        u32x2 v;
        v.x = bf16_rne(acc[t].x) | (bf16_rne(acc[t].y) << 16);
        v.y = bf16_rne(acc[t].z) | (bf16_rne(acc[t].w) << 16);
        *reinterpret_cast<u32x2*>(lp + 16 * t) = v;
      }
    } else {
      const float amax = tile_amax<NT, 8>(acc, s_red);
      const bool fin = amax <= 3.402823466e38f;
      const float sc = (amax > 0.f && fin) ? amax / 448.f : 1.f;
      if (!fin && tid == 0) raise_status(a.status, kStatusNonfinite);
      uint8_t* lp = reinterpret_cast<uint8_t*>(a.ckpt_lp) + e0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t v = fin ? e4m3_pack4(acc[t].x / sc, acc[t].y / sc, acc[t].z / sc, acc[t].w / sc)
                               : e4m3_pack4_nonfinite(acc[t].x, acc[t].y, acc[t].z, acc[t].w);
        *reinterpret_cast<uint32_t*>(lp + 16 * t) = v;
      }
      if (tid == 0) a.lp_scale[unit] = sc;
    }
  }

  IndexUpdate u;
  u.apply = true;
  u.pos_add = (int64_t)len + T;
  u.new_len = 0;
  finish_update(a.arrive, a.pos, a.len, b, a.H, arrived, u);
}

}  // namespace

hipError_t launch_m2_prefill(const M2Args& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  if (a.scheme == kSchemeF32)
    hipLaunchKernelGGL((m2_prefill_kernel<kSchemeF32, 0>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual && a.lp == kLpBf16)
    hipLaunchKernelGGL((m2_prefill_kernel<kSchemeDual, kLpBf16>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual)
    hipLaunchKernelGGL((m2_prefill_kernel<kSchemeDual, kLpE4m3>), grid, block, 0, s, a);
  else if (a.lp == kLpBf16)
    hipLaunchKernelGGL((m2_prefill_kernel<kSchemeShared, kLpBf16>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((m2_prefill_kernel<kSchemeShared, kLpE4m3>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace rssm
