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

// ---- buffered entries staged in LDS ---------------------------------------
// Every kernel that replays the buffer first fetches all of its entries
// (k, v, alpha, beta of up to kMaxCap positions, one float4 of k and v per
// thread) into registers, issues the state stream after them, and then parks
// the entries in LDS.  The sequential backward carry and the fold then run
// from LDS instead of waiting on a dependent global load per entry.
struct EntrySmem {
  float k[kMaxCap][DK];
  float v[kMaxCap][DV];
  float al[kMaxCap], be[kMaxCap];
};
static_assert(kMaxCap * DK / 4 <= NT && kMaxCap * DV / 4 <= NT, "one float4 per thread");

struct EntryRegs {
  f32x4 k, v;
  float al, be;
};

__device__ __forceinline__ EntryRegs fetch_entries(const Src& src, int L, int tid) {
  EntryRegs e;
  e.k = e.v = f32x4{0.f, 0.f, 0.f, 0.f};
  e.al = e.be = 0.f;
  const int i = tid / (DK / 4), c = (tid % (DK / 4)) * 4;
  if (i < L) {
    e.k = ld4(src.k(i) + c);
    e.v = ld4(src.v(i) + c);
  }
  if (tid < L) {
    e.al = src.alpha(tid);
    e.be = src.beta(tid);
  }
  return e;
}

__device__ __forceinline__ void stash_entries(const EntryRegs& e, int L, int tid, EntrySmem& s) {
  const int i = tid / (DK / 4), c = (tid % (DK / 4)) * 4;
  if (i < L) {
    st4(&s.k[i][c], e.k);
    st4(&s.v[i][c], e.v);
  }
  if (tid < L) {
    s.al[tid] = e.al;
    s.be[tid] = e.be;
  }
}

// Write entry i (held in registers by fetch_entries) to its ring slot.
__device__ __forceinline__ void append_from_regs(const GdnArgs& a, const Src& src,
                                                 const EntryRegs& e, int i, int tid) {
  const int s = ring_slot(src.slot0, i, src.cap);
  const long u = src.unit;
  const int ei = tid / (DK / 4), c = (tid % (DK / 4)) * 4;
  if (ei == i) {
    st4(a.ring_k + (u * src.cap + s) * DK + c, e.k);
    st4(a.ring_v + (u * src.cap + s) * DV + c, e.v);
  }
  if (tid == i) {
    a.ring_a[u * src.cap + s] = e.al;
    a.ring_b[u * src.cap + s] = e.be;
  }
}

// Backward carry of a query through entries hi..0 (newest first), held as EPL
// consecutive elements per lane on LPR lanes (lanes repeat every LPR).
template <int EPL, int LPR>
__device__ __forceinline__ void carry(const EntrySmem& s, int hi, int cl, float (&q)[EPL],
                                      float (&sv)[kMaxCap]) {
#pragma unroll
  for (int i = kMaxCap - 1; i >= 0; --i) {
    if (i <= hi) {
      float kv[EPL];
      load_vec<EPL>(&s.k[i][cl * EPL], kv);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part += kv[e] * q[e];
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m);
      const float si = s.be[i] * part;
      const float al = s.al[i];
      sv[i] = si;
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[e] = al * (q[e] - si * kv[e]);
    } else {
      sv[i] = 0.f;
    }
  }
}

// ---------------------------------------------------------------- fold ----
// With u_i = beta_i (v_i - alpha_i a_i) and a_i = G_{c+1..i-1} (S_c k_i)
// + sum_{m<i} G_{m+1..i-1} (k_m . k_i) u_m, every row r satisfies the same
// unit lower-triangular system (I + diag(beta alpha) Lc) u = z,
// z_j = beta_j v_j - beta_j alpha_j G_{c+1..j-1} (S_c k_j),
// Lc[i][m] = G_{m+1..i-1} (k_m . k_i).  Its inverse T is the same for all
// rows, so it is formed once (L x L) and each row's fold weights
// U'_i = G_{i+1..t} u_i = sum_j T'[i][j] z_j are independent dot products.
struct FoldSmem {
  float G[kMaxCap + 1][kMaxCap + 1];   // G[a][e] = prod_{j=a}^{e-1} alpha_j
  float gram[kMaxCap][kMaxCap];        // k_m . k_i
  float P1[kMaxCap][kMaxCap];          // G_{i+1..} T[i][j] beta_j
  float P2[kMaxCap][kMaxCap];          // G_{i+1..} T[i][j] beta_j alpha_j G_{..j-1}
  float W[DV][kMaxCap + 1];            // S_c k_i
  float U[DV][kMaxCap + 1];            // U'_i of row r
  float red[NT / 64];
};

// Fold entries 0..L-1 (staged in es) into the fp32 tile hv (fp32 geometry).
__device__ void fold_tile(f32x4 (&hv)[F32Geo::NLD], const EntrySmem& es, int L, const Geo& q,
                          FoldSmem& sm) {
  constexpr int RPL = F32Geo::RPL, NLD = F32Geo::NLD, LPR = F32Geo::LPR;
  if (q.tid < (L + 1) * (L + 1)) {
    const int a0 = q.tid / (L + 1), e0 = q.tid % (L + 1);
    float p = 1.f;
    for (int j = a0; j < e0; ++j) p *= es.al[j];
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
        for (int e = 0; e < DK / 16; ++e)
          part += es.k[m][sgm * (DK / 16) + e] * es.k[i][sgm * (DK / 16) + e];
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
      if (i0 + jj < L) kv = ld4(&es.k[i0 + jj][q.cl * 4]);
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
  if (q.tid < L) {  // column j of T = (I + diag(beta alpha) Lc)^-1
    const int j = q.tid;
    float t[kMaxCap];
#pragma unroll
    for (int i = 0; i < kMaxCap; ++i) {
      float v = 0.f;
      if (i == j) {
        v = 1.f;
      } else if (i > j && i < L) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < kMaxCap; ++m)
          if (m >= j && m < i) acc += sm.G[m + 1][i] * sm.gram[m][i] * t[m];
        v = -es.be[i] * es.al[i] * acc;
      }
      t[i] = v;
    }
    const float bj = es.be[j], bag = es.be[j] * es.al[j] * sm.G[0][j];
#pragma unroll
    for (int i = 0; i < kMaxCap; ++i) {
      if (i < L) {
        const float w = sm.G[i + 1][L] * t[i];
        sm.P1[i][j] = w * bj;
        sm.P2[i][j] = w * bag;
      }
    }
  }
  __syncthreads();
  {  // U'[r][i] = sum_{j<=i} P1[i][j] v_j[r] - P2[i][j] W[r][j]
    const int r = q.tid % DV, ig = q.tid / DV;
    for (int i = ig; i < L; i += NT / DV) {
      float acc = 0.f;
      for (int j = 0; j <= i; ++j) acc += sm.P1[i][j] * es.v[j][r] - sm.P2[i][j] * sm.W[r][j];
      sm.U[r][i] = acc;
    }
  }
  __syncthreads();
  const float gall = sm.G[0][L];
#pragma unroll
  for (int k = 0; k < NLD; ++k) hv[k] *= gall;
  for (int i = 0; i < L; ++i) {
    const f32x4 kv = ld4(&es.k[i][q.cl * 4]);
#pragma unroll
    for (int k = 0; k < NLD; ++k) hv[k] += sm.U[k * RPL + q.r0][i] * kv;
  }
}

// Workgroup max of |hv|; a NaN anywhere makes the result +inf.
__device__ float tile_amax(const f32x4 (&hv)[F32Geo::NLD], const Geo& q, float* red) {
  float m = 0.f;
  bool nan = false;
#pragma unroll
  for (int k = 0; k < F32Geo::NLD; ++k) {
    m = fmaxf(m, fmaxf(fmaxf(fabsf(hv[k].x), fabsf(hv[k].y)), fmaxf(fabsf(hv[k].z), fabsf(hv[k].w))));
    nan |= !(hv[k].x == hv[k].x && hv[k].y == hv[k].y && hv[k].z == hv[k].z && hv[k].w == hv[k].w);
  }
  if (nan) m = __builtin_inff();
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
// Order: buffered entries and the query are fetched, then the state stream is
// issued, then the entries are parked in LDS while the stream is in flight.
template <int EB, bool FUSED>
__global__ __launch_bounds__(NT) void gdn_step_kernel(GdnArgs a) {
  using Gm = LpGeo<EB>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPL = Gm::RPL, NLD = Gm::NLD;
  const Geo q = geometry<LPR>(a);
  const int cap = a.cap;

  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  const bool ok = len < cap;
  const int L = len + 1;
  Src src{&a, q.unit, len, (int)(pos % cap), cap, 0, 0};
  const float scale = (EB == 1) ? a.lp_scale[q.unit] : 1.f;

  EntryRegs er = fetch_entries(src, ok ? L : 0, q.tid);
  float qv[EPL];
  load_vec<EPL>(a.q + q.unit * DK + q.cl * EPL, qv);

  const char* base = state_base<EB>(a, q.unit);
  u32x4 raw[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) raw[k] = ld_nt_u(base + ((k * RPL + q.r0) * DK + q.cl * EPL) * EB);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos);

  __shared__ __attribute__((aligned(16))) EntrySmem es;
  stash_entries(er, ok ? L : 0, q.tid, es);
  __syncthreads();

  float s[kMaxCap];
  if (ok) {
    carry<EPL, LPR>(es, L - 1, q.cl, qv, s);
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
        if (i < L) ov += s[i] * es.v[i][r];
    } else {
      ov = __builtin_nanf("");
    }
    a.o[q.unit * DV + r] = ov;
  }

  if constexpr (FUSED) {
    static_assert(EB == 4, "fused commit folds the fp32 checkpoint");
    if (ok) {
      __shared__ __attribute__((aligned(16))) FoldSmem sm;
      f32x4 hv[NLD];
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        hv[k] = f32x4{__uint_as_float(raw[k].x), __uint_as_float(raw[k].y),
                      __uint_as_float(raw[k].z), __uint_as_float(raw[k].w)};
      fold_tile(hv, es, L, q, sm);
      store_f32_tile(hv, a.ckpt + q.unit * (DV * DK), q);
    }
  } else {
    if (ok) append_from_regs(a, src, er, len, q.tid);
  }

  IndexUpdate u;
  u.apply = ok;
  u.pos_add = FUSED ? L : 0;
  u.new_len = FUSED ? 0 : L;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H, arrived, u);
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
  const int64_t pos = a.pos[q.b];
  Src src{&a, q.unit, len, (int)(pos % a.cap), a.cap, 0, 0};
  EntryRegs er = fetch_entries(src, len, q.tid);
  f32x4 hv[F32Geo::NLD];
  if constexpr (SCHEME == kSchemeShared)
    load_lp_as_f32<LP>(hv, a, q);
  else
    load_f32_tile(hv, a.ckpt + q.unit * (DV * DK), q);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos);
  __shared__ __attribute__((aligned(16))) EntrySmem es;
  __shared__ __attribute__((aligned(16))) FoldSmem sm;
  stash_entries(er, len, q.tid, es);
  __syncthreads();
  if (len > 0) {
    fold_tile(hv, es, len, q, sm);
    if constexpr (SCHEME != kSchemeShared) store_f32_tile(hv, a.ckpt + q.unit * (DV * DK), q);
  }
  if constexpr (SCHEME != kSchemeF32) store_lp<LP>(hv, a, q, sm.red);

  IndexUpdate u;
  u.apply = len > 0;
  u.pos_add = len;
  u.new_len = 0;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H, arrived, u);
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

  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  const bool ok = len + n <= cap;
  const long sk = (long)a.batch * a.H * DK;
  const long sd = (long)a.batch * a.H;
  Src src{&a, q.unit, len, (int)(pos % cap), cap, sk, sd};
  const float scale = (EB == 1) ? a.lp_scale[q.unit] : 1.f;

  EntryRegs er = fetch_entries(src, ok ? len + n : 0, q.tid);
  const int w = q.tid >> 6;
  float qv[2] = {0.f, 0.f};
  if (ok && w < n) load_vec<2>(a.q + w * sk + q.unit * DK + 2 * q.lane, qv);

  const char* base = state_base<EB>(a, q.unit);
  u32x4 raw[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) raw[k] = ld_nt_u(base + ((k * RPL + q.r0) * DK + q.cl * EPL) * EB);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos);

  __shared__ __attribute__((aligned(16))) EntrySmem es;
  __shared__ __attribute__((aligned(16))) float s_q[NPAD][DK];
  __shared__ float s_s[NPAD][kMaxCap];
  stash_entries(er, ok ? len + n : 0, q.tid, es);
  __syncthreads();

  if (ok && w < n) {  // wave w carries draft w (2 elements per lane)
    float s[kMaxCap];
    carry<2, 64>(es, len + w, q.lane, qv, s);
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
          for (int i = 0; i <= len + j; ++i) ov += s_s[j][i] * es.v[i][r];
        } else {
          ov = __builtin_nanf("");
        }
        a.o[j * (long)a.batch * a.H * DV + q.unit * DV + r] = ov;
      }
    }
  }
  if (ok)
    for (int j = 0; j < n; ++j) append_from_regs(a, src, er, len + j, q.tid);

  IndexUpdate u;
  u.apply = ok;
  u.pos_add = 0;
  u.new_len = len + n;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H, arrived, u);
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
