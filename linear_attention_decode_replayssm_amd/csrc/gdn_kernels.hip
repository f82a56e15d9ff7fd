// gdn_kernels.hip -- Gated DeltaNet decode kernels for gfx950.
//
// State of one (sequence, head): S[dv=128][dk=128], 64 KiB in fp32, 32 KiB in
// bf16, 16 KiB in E4M3 (+ one fp32 scale).  One 512-thread workgroup (8
// wave64) per head; 8,192 workgroups at batch 256 x 32 heads.  The state is
// read with 16-byte lane loads: a row of dk elements is spread over
// LPR = dk / (16 / element bytes) consecutive lanes.
//
// Recurrence: S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T, o_t = S_t q_t.
// Unrolled over the buffered entries i = c+1..t (ReplaySSM: checkpoint +
// buffer of inputs), the output needs one matrix-vector product with the
// checkpoint: carry the query backwards,
//   s_i = beta_i (k_i . q),  q <- alpha_i (q - s_i k_i)   (i = t .. c+1)
//   o_t = S_c q + sum_i s_i v_i
// and the commit folds the buffer with u_i = beta_i (v_i - alpha_i S_{i-1} k_i):
//   S_{i-1} k_i = G_{c+1..i-1} S_c k_i + sum_{m<i} G_{m+1..i-1} (k_m . k_i) u_m
//   S_new = G_{c+1..t} S_c + sum_i G_{i+1..t} u_i k_i^T      (G: products of alpha)
#include "common.hpp"
#include "launch.hpp"

namespace rssm {
namespace {

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NT = 512;
constexpr int kSchemeF32 = 0, kSchemeDual = 1, kSchemeShared = 2;
constexpr int kLpBf16 = 1, kLpE4m3 = 2;

// Lane geometry of a state read with 16-byte lane loads of EB-byte elements.
template <int EB>
struct LpGeo {
  static constexpr int EPL = 16 / EB;   // elements per lane load
  static constexpr int LPR = DK / EPL;  // lanes per state row
  static constexpr int RPL = NT / LPR;  // rows per workgroup-wide load
  static constexpr int NLD = DV / RPL;  // loads per thread
  static_assert(LPR <= 64 && 64 % LPR == 0, "row must sit in one wave");
};
using F32Geo = LpGeo<4>;

struct Geo {
  int b, h, tid, lane, cl, r0;
  long unit;
};

template <int LPR>
__device__ __forceinline__ Geo geometry(const GdnArgs& a) {
  Geo q;
  const int tile = tile_index();
  q.b = tile / a.H;
  q.h = tile - q.b * a.H;
  q.tid = threadIdx.x;
  q.lane = q.tid & 63;
  q.cl = q.tid % LPR;
  q.r0 = q.tid / LPR;
  q.unit = (long)q.b * a.H + q.h;
  return q;
}

// ---- element codecs --------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// bf16 round-to-nearest-even of an fp32 value (NaN -> quiet NaN, sign kept).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP E4M3 code pair -> fp32 via the gfx950 conversion (bytes 0,1 or 2,3).
__device__ __forceinline__ f32x2 e4m3_pair(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
            : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// Four fp32 values (already divided by the scale) -> four E4M3 codes.
// Values are clamped to the largest finite magnitude first, so the
// conversion never overflows: saturating, round to nearest even.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int EB>
__device__ __forceinline__ void expand(u32x4 w, float (&f)[16 / EB]) {
  if constexpr (EB == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
  } else if constexpr (EB == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(w[e]);
      f[2 * e + 1] = bf16_hi(w[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 lo = e4m3_pair(w[e], false), hi = e4m3_pair(w[e], true);
      f[4 * e] = lo.x;
      f[4 * e + 1] = lo.y;
      f[4 * e + 2] = hi.x;
      f[4 * e + 3] = hi.y;
    }
  }
}

template <int EB>
__device__ __forceinline__ const char* state_base(const GdnArgs& a, long unit) {
  if constexpr (EB == 4)
    return reinterpret_cast<const char*>(a.ckpt + unit * (DV * DK));
  else
    return reinterpret_cast<const char*>(a.ckpt_lp) + unit * (DV * DK * EB);
}

// Entry sources: buffered entries i < len come from the ring, later ones from
// the per-position input arrays (position i - len).
struct Src {
  const GdnArgs* a;
  long unit;
  int len, slot0, cap;
  long sk, sd;  // per-position strides of k/v and alpha/beta inputs
  __device__ __forceinline__ const float* k(int i) const {
    return i < len ? a->ring_k + (unit * cap + ring_slot(slot0, i, cap)) * DK
                   : a->k + (i - len) * sk + unit * DK;
  }
  __device__ __forceinline__ const float* v(int i) const {
    return i < len ? a->ring_v + (unit * cap + ring_slot(slot0, i, cap)) * DV
                   : a->v + (i - len) * sk / DK * DV + unit * DV;
  }
  __device__ __forceinline__ float alpha(int i) const {
    return i < len ? a->ring_a[unit * cap + ring_slot(slot0, i, cap)]
                   : a->alpha[(i - len) * sd + unit];
  }
  __device__ __forceinline__ float beta(int i) const {
    return i < len ? a->ring_b[unit * cap + ring_slot(slot0, i, cap)]
                   : a->beta[(i - len) * sd + unit];
  }
};

// Append input position j (0-based) to the ring at entry len + j.
__device__ __forceinline__ void append_entry(const GdnArgs& a, const Src& src, int j, int tid) {
  const int s = ring_slot(src.slot0, src.len + j, src.cap);
  const long u = src.unit;
  if (tid < DK) a.ring_k[(u * src.cap + s) * DK + tid] = a.k[j * src.sk + u * DK + tid];
  else if (tid < DK + DV)
    a.ring_v[(u * src.cap + s) * DV + (tid - DK)] = a.v[j * src.sk + u * DV + (tid - DK)];
  else if (tid == DK + DV) a.ring_a[u * src.cap + s] = a.alpha[j * src.sd + u];
  else if (tid == DK + DV + 1) a.ring_b[u * src.cap + s] = a.beta[j * src.sd + u];
}

template <int EPL>
__device__ __forceinline__ void load_vec(const float* p, float (&v)[EPL]) {
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const f32x4 t = ld4(p + e);
      v[e] = t.x; v[e + 1] = t.y; v[e + 2] = t.z; v[e + 3] = t.w;
    }
  } else if constexpr (EPL == 2) {
    const f32x2 t = *reinterpret_cast<const f32x2*>(p);
    v[0] = t.x; v[1] = t.y;
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = p[e];
  }
}

// Backward carry of a query through entries hi..0 (newest first), held as EPL
// consecutive elements per lane on LPR lanes (lanes repeat every LPR).
template <int EPL, int LPR>
__device__ __forceinline__ void carry(const Src& src, int hi, int cl, float (&q)[EPL],
                                      float (&s)[kMaxCap]) {
#pragma unroll
  for (int i = kMaxCap - 1; i >= 0; --i) {
    if (i <= hi) {
      float kv[EPL];
      load_vec<EPL>(src.k(i) + cl * EPL, kv);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part += kv[e] * q[e];
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m);
      const float si = src.beta(i) * part;
      const float al = src.alpha(i);
      s[i] = si;
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[e] = al * (q[e] - si * kv[e]);
    } else {
      s[i] = 0.f;
    }
  }
}

// ---------------------------------------------------------------- fold ----
// Shared-memory workspace of the fold (fp32 geometry, whole head per WG).
struct FoldSmem {
  float k[kMaxCap][DK];
  float v[kMaxCap][DV];
  float al[kMaxCap], be[kMaxCap];
  float G[kMaxCap + 1][kMaxCap + 1];   // G[a][e] = prod_{j=a}^{e-1} alpha_j
  float gram[kMaxCap][kMaxCap];        // k_m . k_i
  float W[DV][kMaxCap + 1];            // S_c k_i
  float U[DV][kMaxCap + 1];            // G_{i+1..L-1} u_i
  float red[NT / 64];
};

// Fold entries 0..L-1 into the fp32 tile hv (fp32 geometry), in place.
__device__ void fold_tile(f32x4 (&hv)[F32Geo::NLD], const Src& src, int L, const Geo& q,
                          FoldSmem& sm) {
  constexpr int RPL = F32Geo::RPL, NLD = F32Geo::NLD, LPR = F32Geo::LPR;
  for (int idx = q.tid; idx < L * DK; idx += NT) {
    const int i = idx / DK, c = idx % DK;
    sm.k[i][c] = src.k(i)[c];
    sm.v[i][c] = src.v(i)[c];
  }
  if (q.tid < L) {
    sm.al[q.tid] = src.alpha(q.tid);
    sm.be[q.tid] = src.beta(q.tid);
  }
  __syncthreads();
  if (q.tid < (L + 1) * (L + 1)) {
    const int a0 = q.tid / (L + 1), e0 = q.tid % (L + 1);
    float p = 1.f;
    for (int j = a0; j < e0; ++j) p *= sm.al[j];
    sm.G[a0][e0] = p;
  }
  {  // Gram matrix, 16 lanes per pair
    const int sgm = q.tid & 15;
    for (int pass = 0; pass < (kMaxCap * kMaxCap) / (NT / 16); ++pass) {
      const int pi = pass * (NT / 16) + (q.tid >> 4);
      const int m = pi / kMaxCap, i = pi % kMaxCap;
      float part = 0.f;
      if (m < L && i < L) {
#pragma unroll
        for (int e = 0; e < DK / 16; ++e) part += sm.k[m][sgm * (DK / 16) + e] * sm.k[i][sgm * (DK / 16) + e];
      }
      part += __shfl_xor(part, 8);
      part += __shfl_xor(part, 4);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 1);
      if (sgm == 0 && m < L && i < L) sm.gram[m][i] = part;
    }
  }
  // W = S_c k_i, four entries at a time
  for (int i0 = 0; i0 < L; i0 += 4) {
    float d[NLD * 4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 kv = {0.f, 0.f, 0.f, 0.f};
      if (i0 + jj < L) kv = ld4(&sm.k[i0 + jj][q.cl * 4]);
#pragma unroll
      for (int k = 0; k < NLD; ++k) d[k * 4 + jj] = dot4(hv[k], kv);
    }
    xreduce<NLD * 4, LPR>(d, q.lane);
    using M = XMap<NLD * 4, LPR>;
    static_assert(M::VOUT == 1 && M::BFLY == 0, "one sum per lane");
    const int idx = M::index(q.lane, 0);
    const int k = idx / 4, jj = idx % 4;
    if (i0 + jj < L) sm.W[k * RPL + q.r0][i0 + jj] = d[0];
  }
  __syncthreads();
  if (q.tid < DV) {  // forward substitution for row r
    const int r = q.tid;
    float u[kMaxCap];
#pragma unroll
    for (int i = 0; i < kMaxCap; ++i) {
      u[i] = 0.f;
      if (i < L) {
        float acc = sm.G[0][i] * sm.W[r][i];
#pragma unroll
        for (int m = 0; m < kMaxCap; ++m)
          if (m < i) acc += sm.G[m + 1][i] * sm.gram[m][i] * u[m];
        u[i] = sm.be[i] * (sm.v[i][r] - sm.al[i] * acc);
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxCap; ++i)
      if (i < L) sm.U[r][i] = sm.G[i + 1][L] * u[i];
  }
  __syncthreads();
  const float gall = sm.G[0][L];
#pragma unroll
  for (int k = 0; k < NLD; ++k) hv[k] *= gall;
  for (int i = 0; i < L; ++i) {
    const f32x4 kv = ld4(&sm.k[i][q.cl * 4]);
#pragma unroll
    for (int k = 0; k < NLD; ++k) hv[k] += sm.U[k * RPL + q.r0][i] * kv;
  }
}

// Workgroup max of |hv|.
__device__ float tile_amax(const f32x4 (&hv)[F32Geo::NLD], const Geo& q, float* red) {
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < F32Geo::NLD; ++k)
    m = fmaxf(m, fmaxf(fmaxf(fabsf(hv[k].x), fabsf(hv[k].y)), fmaxf(fabsf(hv[k].z), fabsf(hv[k].w))));
  // NaN must survive the reduction: fmaxf would drop it
#pragma unroll
  for (int k = 0; k < F32Geo::NLD; ++k)
    if (!(hv[k].x == hv[k].x && hv[k].y == hv[k].y && hv[k].z == hv[k].z && hv[k].w == hv[k].w))
      m = __builtin_inff();
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  __syncthreads();
  if (q.lane == 0) red[q.tid >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

// Write the low-precision copy of the fp32 tile (fp32 geometry).
template <int LP>
__device__ void store_lp(const f32x4 (&hv)[F32Geo::NLD], const GdnArgs& a, const Geo& q,
                         float* red) {
  constexpr int RPL = F32Geo::RPL, NLD = F32Geo::NLD;
  if constexpr (LP == kLpBf16) {
    uint16_t* base = reinterpret_cast<uint16_t*>(a.ckpt_lp) + q.unit * (DV * DK);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      u32x2 w;
      w.x = bf16_rne(hv[k].x) | (bf16_rne(hv[k].y) << 16);
      w.y = bf16_rne(hv[k].z) | (bf16_rne(hv[k].w) << 16);
      *reinterpret_cast<u32x2*>(base + (k * RPL + q.r0) * DK + q.cl * 4) = w;
    }
  } else {
    const float amax = tile_amax(hv, q, red);
    const bool fin = amax <= 3.402823466e38f;
    const float scale = (amax > 0.f && fin) ? amax / 448.f : 1.f;
    if (!fin && q.tid == 0) raise_status(a.status, kStatusNonfinite);
    uint8_t* base = reinterpret_cast<uint8_t*>(a.ckpt_lp) + q.unit * (DV * DK);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const uint32_t w = e4m3_pack4(hv[k].x / scale, hv[k].y / scale, hv[k].z / scale,
                                    hv[k].w / scale);
      *reinterpret_cast<uint32_t*>(base + (k * RPL + q.r0) * DK + q.cl * 4) = w;
    }
    if (q.tid == 0) a.lp_scale[q.unit] = scale;
  }
}

// Read the low-precision copy into the fp32 geometry (exact value for bf16;
// code * scale rounded to fp32 for E4M3).
template <int LP>
__device__ void load_lp_as_f32(f32x4 (&hv)[F32Geo::NLD], const GdnArgs& a, const Geo& q) {
  constexpr int RPL = F32Geo::RPL, NLD = F32Geo::NLD;
  if constexpr (LP == kLpBf16) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(a.ckpt_lp) + q.unit * (DV * DK);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(base + (k * RPL + q.r0) * DK + q.cl * 4);
      hv[k] = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    }
  } else {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.ckpt_lp) + q.unit * (DV * DK);
    const float scale = a.lp_scale[q.unit];
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(base + (k * RPL + q.r0) * DK + q.cl * 4);
      const f32x2 lo = e4m3_pair(w, false), hi = e4m3_pair(w, true);
      hv[k] = f32x4{lo.x * scale, lo.y * scale, hi.x * scale, hi.y * scale};
    }
  }
}

__device__ __forceinline__ void load_f32_tile(f32x4 (&hv)[F32Geo::NLD], const float* base,
                                              const Geo& q) {
#pragma unroll
  for (int k = 0; k < F32Geo::NLD; ++k)
    hv[k] = ld_nt(base + (k * F32Geo::RPL + q.r0) * DK + q.cl * 4);
}

__device__ __forceinline__ void store_f32_tile(const f32x4 (&hv)[F32Geo::NLD], float* base,
                                               const Geo& q) {
#pragma unroll
  for (int k = 0; k < F32Geo::NLD; ++k)
    st_nt(base + (k * F32Geo::RPL + q.r0) * DK + q.cl * 4, hv[k]);
}

// ---------------------------------------------------------------- step ----
// EB: bytes per checkpoint element read for the output (4: ckpt fp32; 2: bf16
// ckpt_lp; 1: E4M3 ckpt_lp).  FUSED (fp32 only): fold and store after output.
template <int EB, bool FUSED>
__global__ __launch_bounds__(NT) void gdn_step_kernel(GdnArgs a) {
  using Gm = LpGeo<EB>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPL = Gm::RPL, NLD = Gm::NLD;
  const Geo q = geometry<LPR>(a);
  const int cap = a.cap;

  const char* base = state_base<EB>(a, q.unit);
  u32x4 raw[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) raw[k] = ld_nt_u(base + ((k * RPL + q.r0) * DK + q.cl * EPL) * EB);

  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  const bool ok = len < cap;
  const int L = len + 1;
  Src src{&a, q.unit, len, (int)(pos % cap), cap, 0, 0};
  const float scale = (EB == 1) ? a.lp_scale[q.unit] : 1.f;

  if (ok && !FUSED) append_entry(a, src, 0, q.tid);

  float qv[EPL];
  load_vec<EPL>(a.q + q.unit * DK + q.cl * EPL, qv);
  float s[kMaxCap];
  if (ok) {
    carry<EPL, LPR>(src, L - 1, q.cl, qv, s);
  } else {
#pragma unroll
    for (int i = 0; i < kMaxCap; ++i) s[i] = 0.f;
  }

  float d[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    float f[EPL];
    expand<EB>(raw[k], f);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc += f[e] * qv[e];
    d[k] = acc;
  }
  xreduce<NLD, LPR>(d, q.lane);
  using M = XMap<NLD, LPR>;
  if (M::writer(q.lane)) {
    const int r = M::index(q.lane, 0) * RPL + q.r0;
    float ov;
    if (ok) {
      ov = scale * d[0];
#pragma unroll
      for (int i = 0; i < kMaxCap; ++i)
        if (i < L) ov += s[i] * src.v(i)[r];
    } else {
      ov = __builtin_nanf("");
    }
    a.o[q.unit * DV + r] = ov;
  }

  if constexpr (FUSED) {
    static_assert(EB == 4, "fused commit folds the fp32 checkpoint");
    if (ok) {
      __shared__ FoldSmem sm;
      f32x4 hv[NLD];
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        hv[k] = f32x4{__uint_as_float(raw[k].x), __uint_as_float(raw[k].y),
                      __uint_as_float(raw[k].z), __uint_as_float(raw[k].w)};
      fold_tile(hv, src, L, q, sm);
      store_f32_tile(hv, a.ckpt + q.unit * (DV * DK), q);
    }
  }

  IndexUpdate u;
  u.apply = ok;
  u.pos_add = FUSED ? L : 0;
  u.new_len = FUSED ? 0 : L;
  arrive_and_update(a.arrive, a.pos, a.len, q.b, a.H, u);
  if (!ok && q.tid == 0) raise_status(a.status, kStatusOverflow);
}

// -------------------------------------------------------------- commit ----
// SCHEME/LP select: F32 (fold fp32), DUAL (fold fp32, then re-quantise the
// copy), SHARED (fold the dequantised copy, re-quantise).
template <int SCHEME, int LP>
__global__ __launch_bounds__(NT) void gdn_commit_kernel(GdnArgs a) {
  const Geo q = geometry<F32Geo::LPR>(a);
  const int len = a.len[q.b];
  const bool sel = (a.mask == nullptr || a.mask[q.b] != 0) && len >= a.min_len;
  if (!sel) return;                         // uniform for the whole sequence
  if (len == 0 && SCHEME != kSchemeDual) {  // nothing to fold, nothing to refresh
    return;
  }
  __shared__ FoldSmem sm;
  f32x4 hv[F32Geo::NLD];
  if constexpr (SCHEME == kSchemeShared)
    load_lp_as_f32<LP>(hv, a, q);
  else
    load_f32_tile(hv, a.ckpt + q.unit * (DV * DK), q);
  Src src{&a, q.unit, len, (int)(a.pos[q.b] % a.cap), a.cap, 0, 0};
  if (len > 0) {
    fold_tile(hv, src, len, q, sm);
    if constexpr (SCHEME != kSchemeShared) store_f32_tile(hv, a.ckpt + q.unit * (DV * DK), q);
  }
  if constexpr (SCHEME != kSchemeF32) store_lp<LP>(hv, a, q, sm.red);

  IndexUpdate u;
  u.apply = len > 0;
  u.pos_add = len;
  u.new_len = 0;
  arrive_and_update(a.arrive, a.pos, a.len, q.b, a.H, u);
}

// -------------------------------------------------------------- verify ----
// n_pos drafts appended at entries len..len+n-1.  Wave j carries draft j's
// query backwards through entries len+j..0; then one pass over the checkpoint
// dots every row with all carried queries.
template <int EB, int NPAD>
__global__ __launch_bounds__(NT) void gdn_verify_kernel(GdnArgs a) {
  using Gm = LpGeo<EB>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPL = Gm::RPL, NLD = Gm::NLD;
  static_assert(NPAD <= NT / 64, "one wave per draft position");
  const Geo q = geometry<LPR>(a);
  const int cap = a.cap, n = a.n_pos;

  const char* base = state_base<EB>(a, q.unit);
  u32x4 raw[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) raw[k] = ld_nt_u(base + ((k * RPL + q.r0) * DK + q.cl * EPL) * EB);

  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  const bool ok = len + n <= cap;
  const long sk = (long)a.batch * a.H * DK;
  const long sd = (long)a.batch * a.H;
  Src src{&a, q.unit, len, (int)(pos % cap), cap, sk, sd};
  const float scale = (EB == 1) ? a.lp_scale[q.unit] : 1.f;

  __shared__ __attribute__((aligned(16))) float s_q[NPAD][DK];
  __shared__ float s_s[NPAD][kMaxCap];

  if (ok) {
    for (int j = 0; j < n; ++j) append_entry(a, src, j, q.tid);
    const int w = q.tid >> 6;
    if (w < n) {  // wave w carries draft w (2 elements per lane)
      float qv[2];
      load_vec<2>(a.q + w * sk + q.unit * DK + 2 * q.lane, qv);
      float s[kMaxCap];
      carry<2, 64>(src, len + w, q.lane, qv, s);
      s_q[w][2 * q.lane] = qv[0];
      s_q[w][2 * q.lane + 1] = qv[1];
      if (q.lane < kMaxCap) {
        float sv = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxCap; ++i)
          if (i == q.lane) sv = s[i];
        s_s[w][q.lane] = sv;
      }
    }
  }
  __syncthreads();

  constexpr int V = NLD * NPAD;
  float d[V];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    float f[EPL];
    expand<EB>(raw[k], f);
#pragma unroll
    for (int j = 0; j < NPAD; ++j) {
      float acc = 0.f;
      if (j < n && ok) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc += f[e] * s_q[j][q.cl * EPL + e];
      }
      d[k * NPAD + j] = acc;
    }
  }
  xreduce<V, LPR>(d, q.lane);
  using M = XMap<V, LPR>;
  if (M::writer(q.lane)) {
#pragma unroll
    for (int jj = 0; jj < M::VOUT; ++jj) {
      const int idx = M::index(q.lane, jj);
      const int k = idx / NPAD, j = idx % NPAD;
      if (j < n) {
        const int r = k * RPL + q.r0;
        float ov;
        if (ok) {
          ov = scale * d[jj];
          for (int i = 0; i <= len + j; ++i) ov += s_s[j][i] * src.v(i)[r];
        } else {
          ov = __builtin_nanf("");
        }
        a.o[j * (long)a.batch * a.H * DV + q.unit * DV + r] = ov;
      }
    }
  }

  IndexUpdate u;
  u.apply = ok;
  u.pos_add = 0;
  u.new_len = len + n;
  arrive_and_update(a.arrive, a.pos, a.len, q.b, a.H, u);
  if (!ok && q.tid == 0) raise_status(a.status, kStatusOverflow);
}

// --------------------------------------------------------------- eager ----
// Per row r: (S k)_r, then S_r <- alpha S_r + beta (v_r - alpha (S k)_r) k^T,
// then o_r = S_r . q with the updated row; the state is written back.
__global__ __launch_bounds__(NT) void gdn_eager_kernel(GdnArgs a) {
  constexpr int RPL = F32Geo::RPL, NLD = F32Geo::NLD, LPR = F32Geo::LPR;
  const Geo q = geometry<LPR>(a);
  float* st = a.ckpt + q.unit * (DV * DK);
  f32x4 hv[NLD];
  load_f32_tile(hv, st, q);
  const f32x4 kv = ld4(a.k + q.unit * DK + q.cl * 4);
  const f32x4 qv = ld4(a.q + q.unit * DK + q.cl * 4);
  const float al = a.alpha[q.unit], be = a.beta[q.unit];
  const float* vv = a.v + q.unit * DV;
  float sk[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) sk[k] = dot4(hv[k], kv);
  allreduce<NLD, LPR>(sk);
  float d[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const float coef = be * (vv[k * RPL + q.r0] - al * sk[k]);
    hv[k] = al * hv[k] + coef * kv;
    d[k] = dot4(hv[k], qv);
  }
  store_f32_tile(hv, st, q);
  xreduce<NLD, LPR>(d, q.lane);
  using M = XMap<NLD, LPR>;
  if (M::writer(q.lane)) {
    const int r = M::index(q.lane, 0) * RPL + q.r0;
    a.o[q.unit * DV + r] = d[0];
  }
}

}  // namespace

hipError_t launch_gdn_step(const GdnArgs& a, bool fused, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  if (a.scheme == kSchemeF32) {
    if (fused)
      hipLaunchKernelGGL((gdn_step_kernel<4, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((gdn_step_kernel<4, false>), grid, block, 0, s, a);
  } else if (a.lp == kLpBf16) {
    hipLaunchKernelGGL((gdn_step_kernel<2, false>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((gdn_step_kernel<1, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gdn_commit(const GdnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  if (a.scheme == kSchemeF32)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeF32, 0>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual && a.lp == kLpBf16)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeDual, kLpBf16>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeDual, kLpE4m3>), grid, block, 0, s, a);
  else if (a.lp == kLpBf16)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeShared, kLpBf16>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeShared, kLpE4m3>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int EB>
static void launch_gdn_verify_eb(const GdnArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.n_pos <= 1)
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 1>), grid, block, 0, s, a);
  else if (a.n_pos <= 2)
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 2>), grid, block, 0, s, a);
  else if (a.n_pos <= 4)
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 4>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 8>), grid, block, 0, s, a);
}

hipError_t launch_gdn_verify(const GdnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  if (a.scheme == kSchemeF32)
    launch_gdn_verify_eb<4>(a, grid, block, s);
  else if (a.lp == kLpBf16)
    launch_gdn_verify_eb<2>(a, grid, block, s);
  else
    launch_gdn_verify_eb<1>(a, grid, block, s);
  return hipGetLastError();
}

hipError_t launch_gdn_eager(const GdnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(gdn_eager_kernel, dim3((unsigned)(a.batch * a.H)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace rssm
