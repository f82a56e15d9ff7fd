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

// Value of the lane M places higher in the same 16-lane row; the last M lanes
// of the row, which have no source, get 1 (DPP row_shl keeping the old value).
template <int M>
__device__ __forceinline__ float row_shl1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(v), 0x100 | M, 0xF, 0xF, false));
}

// Value of the lane M places lower in the same 16-lane row; the first M lanes
// of the row get 0 (DPP row_shr with zero fill).
template <int M>
__device__ __forceinline__ float row_shr(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 | M, 0xF, 0xF, true));
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

// Left alone the compiler gives this kernel ~220 registers (two waves per
// SIMD); asked for at least three waves it needs no spills and runs ~1.2x
// faster.  The fp32 and bf16 forms come out at 126-128 registers, which
// leaves room for four workgroups per CU (31 KB of LDS each).
template <int SCHEME, int LP>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3))) void m2_prefill_kernel(M2Args a) {
  const int tile = tile_index();
  const int b = tile / a.H, h = tile - b * a.H;
  if (a.mask && a.mask[b] == 0) return;   // the whole sequence skips: no arrival
  const int g = h / (a.H / a.G);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
  const int p = 16 * w + li;              // this lane's state row
  const int T = a.n_pos;
  const int len = a.len[b];
  const int64_t pos = a.pos[b];
  if (!indices_valid(len, pos, a.cap)) {   // refused: nothing read, written or counted
    if (h == 0 && tid == 0) raise_status(a.status, kStatusIndex);
    return;
  }
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
  const uint32_t arrived = arrive_early(a.arrive, b, len, pos, a.idx_ro);

  __shared__ __attribute__((aligned(16))) float s_x[Q][MP + PAD];
  __shared__ __attribute__((aligned(16))) float s_B[Q][MN + PAD];
  __shared__ __attribute__((aligned(16))) float s_C[Q][MN + PAD];
  __shared__ float s_dt[Q];
  __shared__ float s_E[4][Q][Q + 1];
  __shared__ float s_W[Q][Q + 1];
  __shared__ float s_red[NT / 64];
  // a chunk's outputs, staged so that each token's row of P outputs is
  // written as 16-byte stores after the chunk's last barrier
  __shared__ __attribute__((aligned(16))) float s_y[Q][MP];
  int yc = -1, yn = 0;   // chunk and token count staged in s_y, -1: none

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

    // decays, formed by every wave in registers: lane l holds token li's dt
    // and its inclusive prefix sum over the chunk (a 16-lane DPP scan; padded
    // entries have dt = 0), so no wave waits on another for them
    const float dtl = s_dt[li];
    float cum = dtl;
    cum += row_shr<1>(cum);
    cum += row_shr<2>(cum);
    cum += row_shr<4>(cum);
    cum += row_shr<8>(cum);
    const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), Q - 1));
    const float fwl = expf(Ah * (tot - cum)) * dtl;   // fold weight of token li

    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (out) {   // this wave's part of E = C B^T (n = 32w .. 32w+31), then h C_j
      f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int nn = 32 * w + 4 * s + lq;
        e = mfma4(s_C[li][nn], s_B[li][nn], e);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s_E[w][4 * lq + r][li] = e[r];
#pragma unroll
      for (int t = 0; t < 8; ++t) {   // h C_j, contracting over n
        const f32x4 cv = ld4(&s_C[li][16 * t + 4 * lq]);
        y = mfma4(cv.x, acc[t].x, y);
        y = mfma4(cv.y, acc[t].y, y);
        y = mfma4(cv.z, acc[t].z, y);
        y = mfma4(cv.w, acc[t].w, y);
      }
    }
    __syncthreads();
    if (out) {
      {  // in-chunk weights W[j][i], causal: j = 4w + lq, i = li
        const int j = 4 * w + lq;
        const float cj = __shfl(cum, j);
        float wv = 0.f;
        if (li <= j)
          wv = (s_E[0][j][li] + s_E[1][j][li] + s_E[2][j][li] + s_E[3][j][li]) *
               expf(Ah * (cj - cum)) * dtl;
        s_W[j][li] = wv;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r)     // Gamma_j h C_j
        y[r] *= expf(Ah * __shfl(cum, 4 * lq + r));
#pragma unroll
      for (int s = 0; s < 4; ++s)     // + sum_i W[j][i] x_i[p]
        y = mfma4(s_W[li][4 * s + lq], s_x[4 * s + lq][p], y);
#pragma unroll
      for (int r = 0; r < 4; ++r) {   // y[r] is token 4 lq + r, row p
        const int j = 4 * lq + r;
        s_y[j][p] = y[r] + Dh * s_x[j][p];
      }
      yc = c;
      yn = n;
    }
    {  // fold: h <- Gamma_{Q-1} h + sum_i fw_i x_i B_i^T
      const float gq = expf(Ah * tot);
      float bx[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bx[s] = __shfl(fwl, 4 * s + lq) * s_x[4 * s + lq][p];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        acc[t] *= gq;
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[t] = mfma4(s_B[4 * s + lq][16 * t + li], bx[s], acc[t]);
      }
    }
    __syncthreads();   // every read of this chunk's LDS is done
    if (yc == c) {   // token tid / 16, 16 bytes per thread
      const int j = tid >> 4, c4 = tid & 15;
      if (j < yn) st4(a.y + (long)(c * Q + j) * sx + unit * MP + 4 * c4, ld4(&s_y[j][4 * c4]));
    }
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
      const E4m3Scale sc = tile_e4m3_scale<NT, 8>(acc, reinterpret_cast<uint32_t*>(s_red));
      if (!sc.fin && tid == 0) raise_status(a.status, kStatusNonfinite);
      uint8_t* lp = reinterpret_cast<uint8_t*>(a.ckpt_lp) + e0;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<uint32_t*>(lp + 16 * t) = e4m3_encode4(acc[t], sc);
      if (tid == 0) a.lp_scale[unit] = sc.scale;
    }
  }

  IndexUpdate u;
  u.apply = true;
  u.pos_add = (int64_t)len + T;
  u.new_len = 0;
  finish_update(a.arrive, a.pos, a.len, b, a.H, arrived, u);
}

// ------------------------------------------------------------------ GDN ----
// Gated DeltaNet (one 512-thread workgroup per (sequence, head); wave w owns
// state rows (value index) 16w .. 16w+15, the state kept transposed in
// accumulators like the Mamba-2 one: tile t, register r of lane l holds
// S[16w + li][16t + 4lq + r]).  Per row, S <- alpha S + u k^T with
// u = beta (v - alpha S k).  Over a chunk of Q tokens from the chunk-start
// state S (prefix products Gp_t = alpha_0 .. alpha_t, G_{i+1..t} the product
// over i < m <= t, suffix g_i = G_{i+1..Q-1}):
//   W = S K^T,  z_t = beta_t (v_t - Gp_t W_t),  u = T z with
//   T = (I + Lm)^-1,  Lm[t][i] = beta_t G_{i+1..t} (k_i . k_t) for i < t,
//   o_t = Gp_t S q_t + sum_{i<=t} G_{i+1..t} (k_i . q_t) u_i,
//   S  <- Gp_{Q-1} S + sum_i g_i u_i k_i^T,
// the eager recurrence regrouped (the same closed form the commit kernels
// fold with).  W, S Q^T, K K^T, Q K^T, T z, the in-chunk output term and the
// fold are MFMA products; products over the token index take the token-major
// accumulator of the previous product as their B operand directly (k-slot lq
// of register r is token 4 lq + r on both operands).
constexpr int GD = 128;        // dk = dv
constexpr int GNT = 512;       // 8 waves x 16 state rows
constexpr int GPITCH = GD + PAD;

struct GdnChunk {
  f32x4 k, q, v;
  float al, be;
};

struct GdnPre {
  const float *ring_k, *ring_v, *ring_a, *ring_b, *k, *q, *v, *al, *be;
  long unit, sk, sd;
  int cap, slot0, nring, T;
  bool outs;
  __device__ int count(int c) const { return c < 0 ? nring : min(Q, T - c * Q); }
  // thread tid: float4 (tid & 31) of token tid >> 5 for k, q, v; alpha and
  // beta of token tid for tid < Q.  Padding tokens: k = v = q = 0, alpha = 1,
  // beta = 0, which leave the state unchanged.
  __device__ void fetch(int c, GdnChunk& f) const {
    const int tid = threadIdx.x, n = count(c), i = tid >> 5, c4 = tid & 31;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f.k = f.q = f.v = z;
    if (i < n) {
      if (c < 0) {
        const long e = (unit * cap + ring_slot(slot0, i, cap)) * GD + 4 * c4;
        f.k = ld4(ring_k + e);
        f.v = ld4(ring_v + e);
      } else {
        const long e = (long)(c * Q + i) * sk + unit * GD + 4 * c4;
        f.k = ld4(k + e);
        f.v = ld4(v + e);
        if (outs) f.q = ld4(q + e);
      }
    }
    f.al = 1.f;
    f.be = 0.f;
    if (tid < n) {
      if (c < 0) {
        const long e = unit * cap + ring_slot(slot0, tid, cap);
        f.al = ring_a[e];
        f.be = ring_b[e];
      } else {
        const long e = (long)(c * Q + tid) * sd + unit;
        f.al = al[e];
        f.be = be[e];
      }
    }
  }
};

// Capped at four waves per SIMD (two workgroups per CU): 128 registers, no
// spills, ~1.2x faster than the compiler's choice of 130 (one workgroup).
template <int SCHEME, int LP>
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(4))) void gdn_prefill_kernel(GdnArgs a) {
  const int tile = tile_index();
  const int b = tile / a.H, h = tile - b * a.H;
  if (a.mask && a.mask[b] == 0) return;   // the whole sequence skips: no arrival
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
  const int row = 16 * w + li;            // this lane's state row (value index)
  const int T = a.n_pos;
  const int len = a.len[b];
  const int64_t pos = a.pos[b];
  if (!indices_valid(len, pos, a.cap)) {   // refused: nothing read, written or counted
    if (h == 0 && tid == 0) raise_status(a.status, kStatusIndex);
    return;
  }
  const long unit = (long)b * a.H + h;

  GdnPre pre;
  pre.ring_k = a.ring_k;
  pre.ring_v = a.ring_v;
  pre.ring_a = a.ring_a;
  pre.ring_b = a.ring_b;
  pre.k = a.k;
  pre.q = a.q;
  pre.v = a.v;
  pre.al = a.alpha;
  pre.be = a.beta;
  pre.unit = unit;
  pre.sk = (long)a.batch * a.H * GD;
  pre.sd = (long)a.batch * a.H;
  pre.cap = a.cap;
  pre.slot0 = (int)(pos % a.cap);
  pre.nring = min(max(len, 0), min(a.cap, Q));
  pre.T = T;
  pre.outs = a.o != nullptr;

  const int c0 = pre.nring > 0 ? -1 : 0;
  const int nch = (T + Q - 1) / Q;
  GdnChunk f;
  pre.fetch(c0, f);

  f32x4 acc[8];
  const long e0 = unit * (GD * GD) + (long)row * GD + 4 * lq;
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
  const uint32_t arrived = arrive_early(a.arrive, b, len, pos, a.idx_ro);

  __shared__ __attribute__((aligned(16))) float s_k[Q][GPITCH];
  __shared__ __attribute__((aligned(16))) float s_q[Q][GPITCH];
  __shared__ __attribute__((aligned(16))) float s_v[Q][GPITCH];
  __shared__ float s_al[Q], s_be[Q], s_gp[Q], s_gs[Q];
  __shared__ float s_P[8][Q][Q + 1];   // partial K K^T (waves 0-3) and Q K^T (4-7)
  __shared__ __attribute__((aligned(16))) float s_L[Q][Q + 4];   // rows read as float4
  __shared__ float s_M[Q][Q + 1], s_T[Q][Q + 1];
  __shared__ float s_red[GNT / 64];
  // a chunk's outputs, staged so that each token's row of dv outputs is
  // written as 16-byte stores after the chunk's last barrier
  __shared__ __attribute__((aligned(16))) float s_o[Q][GD];
  int oc_ = -1, on_ = 0;   // chunk and token count staged in s_o, -1: none

  for (int c = c0; c < nch; ++c) {
    {
      const int i = tid >> 5, c4 = tid & 31;
      st4(&s_k[i][4 * c4], f.k);
      st4(&s_q[i][4 * c4], f.q);
      st4(&s_v[i][4 * c4], f.v);
      if (tid < Q) {
        s_al[tid] = f.al;
        s_be[tid] = f.be;
      }
    }
    __syncthreads();
    if (c + 1 < nch) pre.fetch(c + 1, f);
    const int n = pre.count(c);
    const bool out = c >= 0 && pre.outs;

    if (tid < Q) {   // prefix and suffix alpha products
      float gp = 1.f, gs = 1.f;
#pragma unroll
      for (int m = 0; m < Q; ++m) {
        const float am = s_al[m];
        if (m <= tid) gp *= am;
        else gs *= am;
      }
      s_gp[tid] = gp;
      s_gs[tid] = gs;
    }
    if (w < 4 || out) {   // K K^T (waves 0-3) / Q K^T (waves 4-7) over a quarter of dk
      const int quarter = w & 3;
      f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int nn = 32 * quarter + 4 * s + lq;
        const float av = w < 4 ? s_k[li][nn] : s_q[li][nn];
        e = mfma4(av, s_k[li][nn], e);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s_P[w][4 * lq + r][li] = e[r];
    }
    __syncthreads();
    {  // Lm and M, one element per thread of the first 256
      if (tid < Q * Q) {
        const int t = tid >> 4, i = tid & 15;
        // G_{i+1..t}: the row of 16 lanes (one t, i = lane) takes the product
        // of alpha_m over m > i of (alpha_m for m <= t, else 1) by a DPP
        // suffix scan
        float g = i <= t ? s_al[i] : 1.f;
        g *= row_shl1<1>(g);
        g *= row_shl1<2>(g);
        g *= row_shl1<4>(g);
        g *= row_shl1<8>(g);
        g = row_shl1<1>(g);
        const float kk = s_P[0][t][i] + s_P[1][t][i] + s_P[2][t][i] + s_P[3][t][i];
        s_L[t][i] = i < t ? s_be[t] * g * kk : 0.f;
        if (out) {
          const float qk = s_P[4][t][i] + s_P[5][t][i] + s_P[6][t][i] + s_P[7][t][i];
          s_M[t][i] = i <= t ? g * qk : 0.f;
        }
      }
    }
    __syncthreads();
    if (tid < Q) {   // T = (I + Lm)^-1, column tid, by forward substitution
      const int j = tid;
      float col[Q];
#pragma unroll
      for (int t = 0; t < Q; ++t) {
        float lt[Q];   // row t of Lm, entries 0 .. t-1, in 16-byte reads
#pragma unroll
        for (int i = 0; i < t; i += 4) {
          const f32x4 r4 = ld4(&s_L[t][i]);
          lt[i] = r4.x;
          if (i + 1 < Q) lt[i + 1] = r4.y;
          if (i + 2 < Q) lt[i + 2] = r4.z;
          if (i + 3 < Q) lt[i + 3] = r4.w;
        }
        float acc2 = 0.f;
#pragma unroll
        for (int i = 0; i < t; ++i) acc2 += lt[i] * col[i];   // col[i] = 0 for i < j
        col[t] = t == j ? 1.f : (t > j ? -acc2 : 0.f);
      }
#pragma unroll
      for (int t = 0; t < Q; ++t) s_T[t][j] = col[t];
    }
    // W^T = K S^T and (outputs) S Q^T, contracting over the state's column index
    f32x4 wt = {0.f, 0.f, 0.f, 0.f}, oc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const f32x4 kv = ld4(&s_k[li][16 * t + 4 * lq]);
      wt = mfma4(kv.x, acc[t].x, wt);
      wt = mfma4(kv.y, acc[t].y, wt);
      wt = mfma4(kv.z, acc[t].z, wt);
      wt = mfma4(kv.w, acc[t].w, wt);
    }
    if (out) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const f32x4 qv = ld4(&s_q[li][16 * t + 4 * lq]);
        oc = mfma4(qv.x, acc[t].x, oc);
        oc = mfma4(qv.y, acc[t].y, oc);
        oc = mfma4(qv.z, acc[t].z, oc);
        oc = mfma4(qv.w, acc[t].w, oc);
      }
    }
    __syncthreads();   // s_T complete
    // z (token 4 lq + r, row `row`), then u = T z
    f32x4 z;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * lq + r;
      z[r] = s_be[t] * (s_v[t][row] - s_gp[t] * wt[r]);
    }
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) u = mfma4(s_T[li][4 * lq + r], z[r], u);
    if (out) {   // o_t = Gp_t S q_t + sum_i M[t][i] u_i
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = s_gp[4 * lq + r] * oc[r];
#pragma unroll
      for (int r = 0; r < 4; ++r) o = mfma4(s_M[li][4 * lq + r], u[r], o);
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[4 * lq + r][row] = o[r];
      oc_ = c;
      on_ = n;
    }
    {  // fold: S <- Gp_{Q-1} S + sum_i g_i u_i k_i^T
      const float gall = s_gp[Q - 1];
      float gu[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) gu[r] = s_gs[4 * lq + r] * u[r];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        acc[t] *= gall;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t] = mfma4(s_k[4 * lq + r][16 * t + li], gu[r], acc[t]);
      }
    }
    __syncthreads();
    if (oc_ == c) {   // token tid / 32, 16 bytes per thread
      const int t = tid >> 5, c4 = tid & 31;
      if (t < on_)
        st4(a.o + (long)(c * Q + t) * ((long)a.batch * a.H * GD) + unit * GD + 4 * c4, ld4(&s_o[t][4 * c4]));
    }
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
      const E4m3Scale sc = tile_e4m3_scale<GNT, 8>(acc, reinterpret_cast<uint32_t*>(s_red));
      if (!sc.fin && tid == 0) raise_status(a.status, kStatusNonfinite);
      uint8_t* lp = reinterpret_cast<uint8_t*>(a.ckpt_lp) + e0;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<uint32_t*>(lp + 16 * t) = e4m3_encode4(acc[t], sc);
      if (tid == 0) a.lp_scale[unit] = sc.scale;
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

hipError_t launch_gdn_prefill(const GdnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(GNT);
  if (a.scheme == kSchemeF32)
    hipLaunchKernelGGL((gdn_prefill_kernel<kSchemeF32, 0>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual && a.lp == kLpBf16)
    hipLaunchKernelGGL((gdn_prefill_kernel<kSchemeDual, kLpBf16>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual)
    hipLaunchKernelGGL((gdn_prefill_kernel<kSchemeDual, kLpE4m3>), grid, block, 0, s, a);
  else if (a.lp == kLpBf16)
    hipLaunchKernelGGL((gdn_prefill_kernel<kSchemeShared, kLpBf16>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gdn_prefill_kernel<kSchemeShared, kLpE4m3>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace rssm
