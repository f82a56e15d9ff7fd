// m2_kernels.hip -- Mamba-2 (SSD) decode kernels for gfx950.
//
// State tile of one (sequence, head): h_c[P=64][N=128] fp32, 32 KiB.
// One 256-thread workgroup (4 wave64) per tile; 20,480 tiles at batch 256 x
// 80 heads.  Thread t owns float4 column c4 = t % 32 of rows r0 + 8k,
// r0 = t / 32, k = 0..7: every load instruction of the workgroup reads 4 KiB
// of consecutive bytes (1 KiB per wavefront).
//
// Replay step (ReplaySSM abstract; explainer "Compute outputs without eagerly
// updating the checkpoint"), with Gamma_{m..n} = exp(A * sum_{j=m..n} dt_j):
//   y_t = Gamma_{c+1..t} h_c C_t + sum_i Gamma_{i+1..t} dt_i (B_i . C_t) x_i + D x_t
// The replay prologue's operands (B_i and C_t segments, dt_i, x_i) are loaded
// first, the checkpoint stream right after; the prologue (B_i . C_t dots, dt
// suffix sums, decay weights, the sum over buffered x_i) runs while the stream
// is in flight; then each row is dotted with C_t and reduced across the 32
// lanes that hold it.  The checkpoint is not written.
//
// Commit (explainer, "Periodically commit a new checkpoint"), a rank-L update:
//   h <- Gamma_{c+1..t} h_c + sum_i Gamma_{i+1..t} dt_i x_i B_i^T
#include "common.hpp"
#include "launch.hpp"
#include "lp_codec.hpp"

namespace rssm {
namespace {

constexpr int P = 64;
constexpr int N = 128;
constexpr int NT = 256;
constexpr int LPR = N / 4;     // lanes sharing one state row (one float4 each)
constexpr int RPL = NT / LPR;  // state rows covered by one workgroup-wide load
constexpr int NLD = P / RPL;   // float4 loads per thread for the whole tile
constexpr int QD = NT / P;     // thread groups splitting the buffered-entry sum
static_assert(LPR <= 64 && 64 % LPR == 0, "a state row must sit in one wave");
static_assert(P % RPL == 0 && NT % P == 0, "tile geometry");
constexpr int kSchemeF32 = 0, kSchemeDual = 1, kSchemeShared = 2;

// Read geometry of a checkpoint of EB-byte elements (4: fp32, 2: bf16, 1:
// E4M3): 16-byte lane loads, LPR lanes per row of N elements.
// ROWS: rows read by one workgroup (P, or HPW * P for HPW consecutive heads,
// which are contiguous in memory).
template <int EB, int ROWS = P>
struct RdGeo {
  static constexpr int EPL = 16 / EB;    // elements per lane load
  static constexpr int LPR = N / EPL;    // lanes per state row
  static constexpr int RPL = NT / LPR;   // rows per workgroup-wide load
  static constexpr int NLD = ROWS / RPL; // loads per thread
  static_assert(LPR <= 64 && 64 % LPR == 0 && ROWS % RPL == 0, "read geometry");
};

// First byte of head `unit`'s checkpoint that the output reads.
template <int EB>
__device__ __forceinline__ const char* read_base(const M2Args& a, long unit) {
  if constexpr (EB == 4)
    return reinterpret_cast<const char*>(a.ckpt + unit * (P * N));
  else
    return reinterpret_cast<const char*>(a.ckpt_lp) + unit * (P * N) * EB;
}

template <int EB, int ROWS = P>
__device__ __forceinline__ void load_raw(const M2Args& a, long unit, int tid,
                                         u32x4 (&raw)[RdGeo<EB, ROWS>::NLD]) {
  using Gm = RdGeo<EB, ROWS>;
  const char* base = read_base<EB>(a, unit);
  const int cl = tid % Gm::LPR, r0 = tid / Gm::LPR;
#pragma unroll
  for (int k = 0; k < Gm::NLD; ++k)
    raw[k] = ld_nt_u(base + ((k * Gm::RPL + r0) * N + cl * Gm::EPL) * EB);
}

// Row dots of the raw tile with a vector held as EPL elements per lane
// (column block cl): d[k] for row k * RPL + r0.
template <int EB, int ROWS = P>
__device__ __forceinline__ void row_dots(const u32x4 (&raw)[RdGeo<EB, ROWS>::NLD],
                                         const float (&cv)[RdGeo<EB, ROWS>::EPL],
                                         float (&d)[RdGeo<EB, ROWS>::NLD]) {
  using Gm = RdGeo<EB, ROWS>;
#pragma unroll
  for (int k = 0; k < Gm::NLD; ++k) {
    float f[Gm::EPL];
    expand<EB>(raw[k], f);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < Gm::EPL; ++e) acc += f[e] * cv[e];
    d[k] = acc;
  }
}

template <int EPL>
__device__ __forceinline__ void load_seg(const float* p, float (&v)[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; e += 4) {
    const f32x4 t = ld4(p + e);
    v[e] = t.x; v[e + 1] = t.y; v[e + 2] = t.z; v[e + 3] = t.w;
  }
}

struct Geo {
  int b, h, g, tid, lane, c4, r0;
  long unit, gunit;
};

// Workgroup -> (sequence b, first head h of HPW consecutive heads of one
// group).  SPLIT: every XCD takes an eighth of each sequence's heads (one
// group of 10 at 80 heads and 8 groups; tile_index_split), else whole
// sequences (tile_index); each kernel takes the order that measured faster
// for it.
template <int HPW = 1, bool SPLIT = false>
__device__ __forceinline__ Geo geometry(const M2Args& a) {
  Geo q;
  const int hb = a.H / HPW;
  const int tile = SPLIT ? tile_index_split(hb) : tile_index();
  q.b = tile / hb;
  q.h = (tile - q.b * hb) * HPW;
  q.g = q.h / (a.H / a.G);
  q.tid = threadIdx.x;
  q.lane = q.tid & 63;
  q.c4 = q.tid % LPR;
  q.r0 = q.tid / LPR;
  q.unit = (long)q.b * a.H + q.h;
  q.gunit = (long)q.b * a.G + q.g;
  return q;
}

__device__ __forceinline__ void load_tile(const float* ck, const Geo& q, f32x4 (&hv)[NLD]) {
#pragma unroll
  for (int k = 0; k < NLD; ++k) hv[k] = ld_nt(ck + (k * RPL + q.r0) * N + q.c4 * 4);
}

__device__ __forceinline__ void store_tile(float* ck, const Geo& q, const f32x4 (&hv)[NLD]) {
#pragma unroll
  for (int k = 0; k < NLD; ++k) st_nt(ck + (k * RPL + q.r0) * N + q.c4 * 4, hv[k]);
}

// ---------------------------------------------------------------- step ----
// Load order matters: vector loads complete in issue order, so every small
// load the replay prologue needs (B_i and C_t segments, dt_i, x_i) is issued
// before the checkpoint stream.  Waiting for them then leaves the stream in
// flight while the prologue runs.  The ring append is done last, after the
// stream has been consumed.
//
// HPW: heads per workgroup, consecutive heads of one group (their checkpoints
// are contiguous).  The fp32 and bf16 steps take one head (32 and 16 KiB of
// stream); the E4M3 step takes two, so that a workgroup streams 16 KiB rather
// than 8 behind the same fixed chain of index read, operand loads and
// prologue (53 -> 42 us per step at batch 256 x 80 heads; two bf16 heads per
// workgroup measured no faster than one).  B_i . C_t is shared by the heads
// of a group and formed once.
//
// LP (fused commit of a DUAL layer): the boundary step reads, folds and stores
// the fp32 checkpoint as for F32, takes its output from the fp32 checkpoint it
// reads, and then writes the low-precision image of the folded state.
//
// MAXL: the most buffered entries (ring capacity) the kernel serves, 16 or 32;
// each 16-lane group of the prologue handles MAXL / 16 entries.
template <int EB, bool FUSED, int HPW = 1, int LP = 0, int MAXL = kMaxCap>
__global__ __launch_bounds__(NT) void m2_step_kernel(M2Args a) {
  constexpr int ROWS = HPW * P;
  using Gm = RdGeo<EB, ROWS>;
  static_assert(!FUSED || (EB == 4 && HPW == 1), "the fused commit folds one fp32 head");
  static_assert(LP == 0 || FUSED, "a low-precision image is written only by the fused commit");
  static_assert(HPW <= 16, "dt of head hl is loaded by lane hl of an entry's 16 lanes");
  static_assert(MAXL % 16 == 0 && MAXL * HPW <= NT, "entries per 16-lane group");
  const Geo q = geometry<HPW, FUSED || EB != 4>(a);
  const int cap = a.cap;
  float* ck = a.ckpt + q.unit * (P * N);

  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  const bool valid = indices_valid(len, pos, cap);
  const bool ok = valid && len < cap;
  const int L = len + 1;
  const int slot0 = valid ? (int)(pos % cap) : 0;
  float Ah[HPW], Dh[HPW];
#pragma unroll
  for (int hl = 0; hl < HPW; ++hl) {
    Ah[hl] = a.A[q.h + hl];
    Dh[hl] = a.D[q.h + hl];
  }

  const float* xt = a.x + q.unit * P;   // HPW heads' x_t, contiguous
  const float* Bt = a.B + q.gunit * N;
  const float* Ct = a.C + q.gunit * N;
  auto xsrc = [&](int hl, int i) -> const float* {
    return i < len ? a.ring_x + ((q.unit + hl) * cap + ring_slot(slot0, i, cap)) * P
                   : xt + hl * P;
  };
  auto Bsrc = [&](int i) -> const float* {
    return i < len ? a.ring_B + (q.gunit * cap + ring_slot(slot0, i, cap)) * N : Bt;
  };

  // prologue operands: entries ei + 16 u (u < EPG) of the 16-lane group
  // ei = tid/16 dot segment sg of B with C_t (lane sg < HPW also loads head
  // sg's dt); thread (p, qd) sums entries qd, qd+QD, ... of every head's x_i[p]
  constexpr int SEG = N / 16;
  constexpr int EPG = MAXL / 16;     // entries per 16-lane group
  constexpr int XPT = MAXL / QD;     // buffered x values per thread and head
  const int ei = q.tid >> 4, sg = q.tid & 15;
  const int p = q.tid % P, qd = q.tid / P;
  f32x4 bseg[EPG][SEG / 4], cseg[SEG / 4];
  float dti[EPG];
  float xv[HPW][XPT];
  if (ok) {
#pragma unroll
    for (int e = 0; e < SEG / 4; ++e) cseg[e] = ld4(Ct + sg * SEG + 4 * e);
#pragma unroll
    for (int u = 0; u < EPG; ++u) {
      const int en = ei + 16 * u;
      dti[u] = 0.f;
#pragma unroll
      for (int e = 0; e < SEG / 4; ++e) bseg[u][e] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (en < L) {
#pragma unroll
        for (int e = 0; e < SEG / 4; ++e) bseg[u][e] = ld4(Bsrc(en) + sg * SEG + 4 * e);
        if (sg < HPW)
          dti[u] = en < len ? a.ring_dt[(q.unit + sg) * cap + ring_slot(slot0, en, cap)]
                            : a.dt[q.unit + sg];
      }
    }
#pragma unroll
    for (int hl = 0; hl < HPW; ++hl) {
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const int i = qd + m * QD;
        xv[hl][m] = i < L ? xsrc(hl, i)[p] : 0.f;
      }
    }
  }
  const int cl = q.tid % Gm::LPR, rr0 = q.tid / Gm::LPR;   // read geometry
  float cv[Gm::EPL];
  load_seg<Gm::EPL>(Ct + cl * Gm::EPL, cv);
  float scale[HPW];
#pragma unroll
  for (int hl = 0; hl < HPW; ++hl) scale[hl] = (EB == 1) ? a.lp_scale[q.unit + hl] : 1.f;

  u32x4 raw[Gm::NLD];
  load_raw<EB, ROWS>(a, q.unit, q.tid, raw);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos, a.idx_ro);

  __shared__ float s_e[MAXL], s_dt[HPW][MAXL], s_w[HPW][MAXL], s_fw[MAXL];
  __shared__ float s_gamma[HPW];
  __shared__ float s_yb[QD][HPW][P];
  // fused commit: the entries' x_i and B_i, parked from the prologue registers
  __shared__ __attribute__((aligned(16))) float s_x[FUSED ? MAXL : 1][P];
  __shared__ __attribute__((aligned(16))) float s_B[FUSED ? MAXL : 1][N];

  if (ok) {
#pragma unroll
    for (int u = 0; u < EPG; ++u) {  // e_i = B_i . C_t
      const int en = ei + 16 * u;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < SEG / 4; ++e) part += dot4(bseg[u][e], cseg[e]);
      part = group_sum<16>(part);
      if (sg == 0 && en < L) s_e[en] = part;
      if (sg < HPW && en < L) s_dt[sg][en] = dti[u];
      if constexpr (FUSED) {   // no second fetch of the entries at the fold
        if (en < L) {
#pragma unroll
          for (int e = 0; e < SEG / 4; ++e) st4(&s_B[en][sg * SEG + 4 * e], bseg[u][e]);
        }
      }
    }
    if constexpr (FUSED) {
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const int i = qd + m * QD;
        if (i < L) s_x[i][p] = xv[0][m];
      }
    }
    __syncthreads();
    if (q.tid < HPW * MAXL) {  // decay weights from dt suffix sums, per head
      const int hl = q.tid / MAXL, i = q.tid % MAXL;
      if (i < L) {
        float suf = 0.f;
        for (int j = i + 1; j < L; ++j) suf += s_dt[hl][j];
        const float dec = expf(Ah[hl] * suf);
        s_w[hl][i] = dec * s_dt[hl][i] * s_e[i];
        if (FUSED) s_fw[i] = dec * s_dt[hl][i];
        if (i == 0) s_gamma[hl] = expf(Ah[hl] * (suf + s_dt[hl][0]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int hl = 0; hl < HPW; ++hl) {  // sum_i w_i x_i[p]
      float yb = 0.f;
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const int i = qd + m * QD;
        if (i < L) yb += s_w[hl][i] * xv[hl][m];
      }
      s_yb[qd][hl][p] = yb;
    }
  }

  {  // Gamma * (h_c C_t) + buffered part + D x_t
    float d[Gm::NLD];
    row_dots<EB, ROWS>(raw, cv, d);
    xreduce<Gm::NLD, Gm::LPR>(d, q.lane);
    __syncthreads();
    using M = XMap<Gm::NLD, Gm::LPR>;
    if (M::writer(q.lane)) {
      const int pr = M::index(q.lane, 0) * Gm::RPL + rr0;   // row of the HPW heads
      const int hl = pr / P, pp = pr - hl * P;
      float yv;
      if (ok) {
        float yb = 0.f;
#pragma unroll
        for (int j = 0; j < QD; ++j) yb += s_yb[j][hl][pp];
        float sc = scale[0], dh = Dh[0];
#pragma unroll
        for (int k = 1; k < HPW; ++k)
          if (hl == k) {
            sc = scale[k];
            dh = Dh[k];
          }
        yv = s_gamma[hl] * (sc * d[0]) + yb + dh * xt[pr];
      } else {
        yv = __builtin_nanf("");
      }
      a.y[q.unit * P + pr] = yv;
    }
  }

  if constexpr (FUSED) {
    if (ok) {  // fold the whole buffer, this entry included, and store
      f32x4 hv[NLD];   // the fp32 read geometry is the tile geometry
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        hv[k] = f32x4{__uint_as_float(raw[k].x), __uint_as_float(raw[k].y),
                      __uint_as_float(raw[k].z), __uint_as_float(raw[k].w)};
      const float gam = s_gamma[0];
#pragma unroll
      for (int k = 0; k < NLD; ++k) hv[k] *= gam;
      for (int i = 0; i < L; ++i) {
        const f32x4 bi = ld4(&s_B[i][q.c4 * 4]);
        const float w = s_fw[i];
#pragma unroll
        for (int k = 0; k < NLD; ++k) hv[k] += (w * s_x[i][k * RPL + q.r0]) * bi;
      }
      store_tile(ck, q, hv);
      if constexpr (LP != 0) {   // DUAL: the serving copy re-quantised from fp32
        __shared__ float s_red[NT / 64];
        char* lp = reinterpret_cast<char*>(a.ckpt_lp) + q.unit * (P * N) * (LP == kLpBf16 ? 2 : 1);
        store_lp_tile<LP, NT, NLD, RPL, N>(hv, lp, a.lp_scale ? a.lp_scale + q.unit : nullptr,
                                           a.status, q.r0, q.c4, s_red);
      }
    }
  } else {
    if (ok) {  // append this step's entry from the registers that loaded it
      const int s = ring_slot(slot0, len, cap);
#pragma unroll
      for (int hl = 0; hl < HPW; ++hl) {
#pragma unroll
        for (int m = 0; m < XPT; ++m)
          if (qd + m * QD == len) a.ring_x[((q.unit + hl) * cap + s) * P + p] = xv[hl][m];
      }
#pragma unroll
      for (int u = 0; u < EPG; ++u) {
        if (ei + 16 * u == len) {
          if ((q.h % (a.H / a.G)) == 0) {
#pragma unroll
            for (int e = 0; e < SEG / 4; ++e)
              st4(a.ring_B + (q.gunit * cap + s) * N + sg * SEG + 4 * e, bseg[u][e]);
          }
          if (sg < HPW) a.ring_dt[(q.unit + sg) * cap + s] = dti[u];
        }
      }
    }
  }

  IndexUpdate u;
  u.apply = ok;
  u.pos_add = FUSED ? L : 0;
  u.new_len = FUSED ? 0 : L;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H / HPW, arrived, u);
  if (!ok && last_arrival(arrived, a.H / HPW))
    raise_status(a.status, valid ? kStatusOverflow : kStatusIndex);
}

// -------------------------------------------------------------- commit ----
// SCHEME/LP: F32 folds the fp32 checkpoint; DUAL folds fp32 and then writes
// the low-precision image of the result (with len 0 it only refreshes the
// image); SHARED folds the dequantised low-precision copy and re-encodes it.
// One workgroup holds a whole head, so the E4M3 scale's amax is local.
template <int SCHEME, int LP, int MAXL = kMaxCap>
__global__ __launch_bounds__(NT) void m2_commit_kernel(M2Args a) {
  const Geo q = geometry<1, SCHEME == kSchemeF32>(a);
  const int cap = a.cap;
  if (a.mask != nullptr && a.mask[q.b] == 0) return;   // uniform for the sequence
  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  if (!indices_valid(len, pos, cap)) {   // refused: nothing read, written or counted
    if (q.h == 0 && q.tid == 0) raise_status(a.status, kStatusIndex);
    return;
  }
  if (len < a.min_len || (len == 0 && SCHEME != kSchemeDual)) return;   // not due

  const int L = len;
  const int slot0 = (int)(pos % cap);
  // the buffered entries first, into registers (thread tid: x of entry
  // (tid + 256u) / 64, float4 (tid + 256u) % 32 of B_{(tid + 256u) / 32}, dt_tid):
  // waiting for them then leaves the state stream in flight
  constexpr int XR = MAXL * P / NT, BR = MAXL * N / 4 / NT;
  float xr[XR];
  f32x4 br[BR];
  float dtr = 0.f;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const int idx = q.tid + u * NT, i = idx / P;
    xr[u] = i < L ? a.ring_x[(q.unit * cap + ring_slot(slot0, i, cap)) * P + idx % P] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < BR; ++u) {
    const int idx = q.tid + u * NT, i = idx / (N / 4);
    br[u] = i < L ? ld4(a.ring_B + (q.gunit * cap + ring_slot(slot0, i, cap)) * N + 4 * (idx % (N / 4)))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (q.tid < L) dtr = a.ring_dt[q.unit * cap + ring_slot(slot0, q.tid, cap)];

  float* ck = a.ckpt + q.unit * (P * N);
  char* lp = reinterpret_cast<char*>(a.ckpt_lp) + q.unit * (P * N) * (LP == kLpBf16 ? 2 : 1);
  float* lps = a.lp_scale ? a.lp_scale + q.unit : nullptr;
  f32x4 hv[NLD];
  if constexpr (SCHEME == kSchemeShared)
    load_lp_tile<LP, NLD, RPL, N>(hv, lp, lps, q.r0, q.c4);
  else
    load_tile(ck, q, hv);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos, a.idx_ro);

  const float Ah = a.A[q.h];
  __shared__ float s_dt[MAXL], s_fw[MAXL];
  __shared__ float s_gamma;
  __shared__ float s_red[NT / 64];
  __shared__ __attribute__((aligned(16))) float s_x[MAXL][P];
  __shared__ __attribute__((aligned(16))) float s_B[MAXL][N];
  if (L > 0) {
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      const int idx = q.tid + u * NT;
      s_x[idx / P][idx % P] = xr[u];
    }
#pragma unroll
    for (int u = 0; u < BR; ++u) {
      const int idx = q.tid + u * NT;
      st4(&s_B[idx / (N / 4)][4 * (idx % (N / 4))], br[u]);
    }
    if (q.tid < L) s_dt[q.tid] = dtr;
    __syncthreads();
    if (q.tid < L) {
      float suf = 0.f;
      for (int j = q.tid + 1; j < L; ++j) suf += s_dt[j];
      s_fw[q.tid] = expf(Ah * suf) * s_dt[q.tid];
      if (q.tid == 0) s_gamma = expf(Ah * (suf + s_dt[0]));
    }
    __syncthreads();
    const float gam = s_gamma;
#pragma unroll
    for (int k = 0; k < NLD; ++k) hv[k] *= gam;
    for (int i = 0; i < L; ++i) {
      const f32x4 bi = ld4(&s_B[i][q.c4 * 4]);
      const float w = s_fw[i];
#pragma unroll
      for (int k = 0; k < NLD; ++k) hv[k] += (w * s_x[i][k * RPL + q.r0]) * bi;
    }
    if constexpr (SCHEME != kSchemeShared) store_tile(ck, q, hv);
  }
  if constexpr (SCHEME != kSchemeF32)
    store_lp_tile<LP, NT, NLD, RPL, N>(hv, lp, lps, a.status, q.r0, q.c4, s_red);

  IndexUpdate u;
  u.apply = L > 0;
  u.pos_add = L;
  u.new_len = 0;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H, arrived, u);
}

// -------------------------------------------------------------- verify ----
// n_pos drafts at entries len..len+n-1; draft j's output uses the buffered
// entries and the drafts on its path (a.anc[j]: for a chain, drafts 0..j).
// A chain (a.append) appends the drafts; a tree appends nothing.  One
// checkpoint read serves all positions: each row of h_c is dotted with every
// C_j before the cross-lane reduction.  As in the step kernel, every small
// operand (the drafts' C_j, B_i segments, dt_i, x_i) is loaded before the
// checkpoint stream, so the prologue runs while the stream is in flight.
//
// COMMIT (fp32 checkpoint only): a sequence whose buffer holds at least
// a.min_len entries also folds those entries into its checkpoint from the
// same read of the state -- the commit that would otherwise precede this
// verify as a separate pass over the state -- and its checkpoint moves to the
// end of the buffer; the drafts then sit at entries 0..n-1 of the new buffer
// (the same ring slots).  The outputs are those of commit-then-verify.
//
// MF (fp32 checkpoint, 4 or 8 drafts): the contraction Y^T = [C_j] h_c^T runs
// on v_mfma_f32_16x16x4f32 (drafts padded to 16 rows of the A operand).  The
// MFMA operand layout puts 16 rows x 64 B in one wave load, which streams ~10%
// slower than consecutive bytes, so each wave streams its own 16 state rows
// with consecutive 1 KiB loads (rows 16w + 2k + lane/32, k = 0..7), parks
// them in a wave-private LDS tile and reads the operands from there: no
// cross-lane reduction, and no barrier between the waves for the transpose.
//
// W16 (fp32, eight drafts, with or without the fold): 16 lanes per state row instead of 32,
// each holding columns 4c..4c+3 and 64+4c..64+4c+3 of rows r0 + 16k (every
// load instruction still reads 256 contiguous bytes per row).  The 4 rows x 8
// drafts of partial sums per lane are then reduced across 16 lanes, with DPP
// only, in one pass instead of two passes of 32 sums across 32 lanes.
template <int EB, int NPAD, bool COMMIT = false, bool MF = false>
__global__ __launch_bounds__(NT) void m2_verify_kernel(M2Args a) {
  static_assert(!COMMIT || EB == 4, "the fused commit folds the fp32 checkpoint");
  static_assert(!MF || (EB == 4 && NPAD >= 4), "matrix-core contraction: fp32, 4 or 8 drafts");
  constexpr bool W16 = EB == 4 && NPAD == 8 && !MF;
  using Gm = RdGeo<EB>;
  const Geo q = geometry<1, NPAD != 8 || COMMIT>(a);
  const int cap = a.cap, n = a.n_pos;
  const int64_t pos = a.pos[q.b];
  const RolledLen rl = rolled_len(a.len[q.b], pos, cap, a.n_reject, q.b);
  const int len = rl.len;
  const bool valid = rl.valid;
  const bool ok = valid && len + n <= cap;
  const bool fold = COMMIT && ok && len > 0 && len >= a.min_len;   // uniform per sequence
  const int LT = len + n;
  const int slot0 = valid ? (int)(pos % cap) : 0;
  const float Ah = a.A[q.h];
  const float Dh = a.D[q.h];
  const long sx = (long)a.batch * a.H * P;   // per-draft strides
  const long sg = (long)a.batch * a.G * N;
  const long sd = (long)a.batch * a.H;

  auto xsrc = [&](int i) -> const float* {
    return i < len ? a.ring_x + (q.unit * cap + ring_slot(slot0, i, cap)) * P
                   : a.x + (i - len) * sx + q.unit * P;
  };
  auto Bsrc = [&](int i) -> const float* {
    return i < len ? a.ring_B + (q.gunit * cap + ring_slot(slot0, i, cap)) * N
                   : a.B + (i - len) * sg + q.gunit * N;
  };

  // prologue operands: entry ei = tid/16 holds segment sgm of B_ei (and dt_ei);
  // thread (p, qd) holds x_i[p] of entries qd, qd+QD, ...; the drafts' C_j
  // go to LDS (CPT values per thread)
  constexpr int SEG = N / 16;
  constexpr int XPT = kMaxCap / QD;
  constexpr int CPT = (NPAD * N + NT - 1) / NT;
  const int ei = q.tid >> 4, sgm = q.tid & 15;
  const int p = q.tid % P, qd = q.tid / P;
  f32x4 bseg[SEG / 4];
  float dti = 0.f, xv[XPT], cst[CPT];
#pragma unroll
  for (int e = 0; e < SEG / 4; ++e) bseg[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < XPT; ++m) xv[m] = 0.f;
#pragma unroll
  for (int u = 0; u < CPT; ++u) cst[u] = 0.f;
  if (ok) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int idx = q.tid + u * NT, j = idx / N;
      if (idx < NPAD * N && j < n) cst[u] = a.C[j * sg + q.gunit * N + idx % N];
    }
    if (ei < LT) {
#pragma unroll
      for (int e = 0; e < SEG / 4; ++e) bseg[e] = ld4(Bsrc(ei) + sgm * SEG + 4 * e);
      if (sgm == 0)
        dti = ei < len ? a.ring_dt[q.unit * cap + ring_slot(slot0, ei, cap)]
                       : a.dt[(ei - len) * sd + q.unit];
    }
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int i = qd + m * QD;
      if (i < LT) xv[m] = xsrc(i)[p];
    }
  }
  u32x4 raw[Gm::NLD];
  // row of the thread's k-th state load: consecutive workgroup loads, or
  // (MF) each wave's own 16 rows
  auto rowk = [&](int k) -> int {
    return MF ? 16 * (q.tid >> 6) + 2 * k + (q.lane >> 5) : k * RPL + q.r0;
  };
  if constexpr (MF) {
    const float* ck0 = a.ckpt + q.unit * (P * N) + q.c4 * 4;
#pragma unroll
    for (int k = 0; k < NLD; ++k) raw[k] = ld_nt_u(ck0 + rowk(k) * N);
  } else if constexpr (W16) {   // raw[2 k + hf]: row tid/16 + 16 k, column half hf
    const float* ck0 = a.ckpt + q.unit * (P * N) + (q.tid >> 4) * N + 4 * (q.tid & 15);
#pragma unroll
    for (int k = 0; k < NLD / 2; ++k) {
      raw[2 * k] = ld_nt_u(ck0 + 16 * k * N);
      raw[2 * k + 1] = ld_nt_u(ck0 + 16 * k * N + 64);
    }
  } else {
    load_raw<EB>(a, q.unit, q.tid, raw);
  }
  const int cl = q.tid % Gm::LPR, rr0 = q.tid / Gm::LPR;
  const float scale = (EB == 1) ? a.lp_scale[q.unit] : 1.f;

  constexpr int CP = N + 4;   // padded LDS row pitch of C_j and the MF tile
  __shared__ __attribute__((aligned(16))) float s_C[NPAD][CP];
  // entries' B and x: the drafts' (the append, and the outputs' D x_j) and,
  // with COMMIT, the buffered entries' for the fold, in one array of entries
  // 0 .. len+n-1 (the buffer first); without COMMIT the drafts only
  constexpr int EA = COMMIT ? kMaxCap : NPAD;
  __shared__ __attribute__((aligned(16))) float s_Be[EA][N];
  __shared__ __attribute__((aligned(16))) float s_xe[EA][P];
  const int e0 = COMMIT ? len : 0;   // row of draft 0
  __shared__ float s_dta[NPAD];
  __shared__ float s_dt[kMaxCap];
  __shared__ float s_e[NPAD][kMaxCap];
  __shared__ float s_w[NPAD][kMaxCap];
  __shared__ float s_gam[NPAD];
  __shared__ float s_yb[QD][NPAD][P];
  __shared__ float s_fw[COMMIT ? kMaxCap : 1];
  __shared__ float s_gbuf;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int idx = q.tid + u * NT;
    if (idx < NPAD * N) s_C[idx / N][idx % N] = cst[u];
  }
  if (sgm == 0) s_dt[ei] = dti;
  if constexpr (COMMIT) {
    if (fold) {   // uniform
      if (ei < len) {
#pragma unroll
        for (int e = 0; e < SEG / 4; ++e) st4(&s_Be[ei][sgm * SEG + 4 * e], bseg[e]);
      }
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const int i = qd + m * QD;
        if (i < len) s_xe[i][p] = xv[m];
      }
    }
  }
  if (a.append) {   // uniform: the drafts' own rows, kept for the append below
    if (ei >= len && ei < LT) {
#pragma unroll
      for (int e = 0; e < SEG / 4; ++e) st4(&s_Be[ei - len + e0][sgm * SEG + 4 * e], bseg[e]);
      if (sgm == 0) s_dta[ei - len] = dti;
    }
  }
#pragma unroll
  for (int m = 0; m < XPT; ++m) {   // the drafts' x_j (append, and the outputs' D x_j)
    const int i = qd + m * QD;
    if (i >= len && i < LT) s_xe[i - len + e0][p] = xv[m];
  }
  indices_consumed(len, pos);   // its barrier also publishes the LDS above
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos, a.idx_ro);

  if (ok) {
    {  // e_{j,ei} = B_ei . C_j for every draft, 16 lanes per entry: the NPAD
       // partial dots of a lane reduced together across its 16 lanes
      float part[NPAD];
#pragma unroll
      for (int j = 0; j < NPAD; ++j) {   // C_j of an absent draft is zero in s_C
        part[j] = 0.f;
#pragma unroll
        for (int e = 0; e < SEG / 4; ++e) part[j] += dot4(bseg[e], ld4(&s_C[j][sgm * SEG + 4 * e]));
      }
      xreduce<NPAD, 16>(part, q.lane);
      using ME = XMap<NPAD, 16>;
      static_assert(ME::VOUT == 1, "one sum per lane");
      if (ME::writer(q.lane)) s_e[ME::index(q.lane, 0)][ei] = part[0];
    }
    __syncthreads();
    static_assert(kMaxCap == 16, "one 16-lane row per draft");
    if (q.tid < NPAD * kMaxCap) {   // decay weights; zero off the path
      const int j = q.tid / kMaxCap, i = q.tid % kMaxCap;
      const int Lj = len + j + 1;   // draft j is the last entry on its path
      // draft j's path as a mask over entries: the buffer, then its ancestors
      // and itself.  The masks are read with uniform indices (kernel-argument
      // loads), never indexed by a lane-varying j.
      uint32_t anc = 0u;
#pragma unroll
      for (int jj = 0; jj < NPAD; ++jj)
        if (j == jj) anc = a.anc[jj];
      const uint32_t path = ((1u << len) - 1u) | (anc << len);
      // lane i of draft j's 16-lane group: dt_i if entry i is on the path;
      // the suffix over the later path entries is the decay exponent
      const bool on = j < n && i < Lj && ((path >> i) & 1u);
      const float dv = on ? s_dt[i] : 0.f;
      const float suf = row_suffix_excl(dv);
      s_w[j][i] = on ? expf(Ah * suf) * dv * s_e[j][i] : 0.f;
      if (j < n && i == 0) s_gam[j] = expf(Ah * (dv + suf));   // Gamma over the whole path
    }
    if constexpr (COMMIT) {   // the commit's weights over the buffered entries
      const int i = q.tid - NPAD * kMaxCap;
      if (fold && i >= 0 && i < len) {
        float suf = 0.f;
        for (int m = i + 1; m < len; ++m) suf += s_dt[m];
        s_fw[i] = expf(Ah * suf) * s_dt[i];
        if (i == 0) s_gbuf = expf(Ah * (suf + s_dt[0]));
      }
    }
    __syncthreads();
    {  // sum_i w_{j,i} x_i[p] (the outputs add D x_j[p] from s_xe)
      float acc[NPAD];
#pragma unroll
      for (int j = 0; j < NPAD; ++j) acc[j] = 0.f;
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const int i = qd + m * QD;
#pragma unroll
        for (int j = 0; j < NPAD; ++j) acc[j] += s_w[j][i] * xv[m];
      }
#pragma unroll
      for (int j = 0; j < NPAD; ++j) s_yb[qd][j][p] = acc[j];
    }
  }

  float f[Gm::NLD][Gm::EPL];   // the tile, expanded once
#pragma unroll
  for (int k = 0; k < Gm::NLD; ++k) expand<EB>(raw[k], f[k]);
  if constexpr (MF) {
    // wave-private transpose of this wave's 16 rows, NPASS column slices at a
    // time (lane ch = lane % 32 holds columns 4ch .. 4ch + 3 of its rows), then
    // per 16-column block the A operand C_j[n] (lane: draft lane % 16,
    // n = 16cb + 4 (lane / 16) + s) and the B operand h[p][n] (lane: row
    // lane % 16, same n)
    constexpr int NPASS = 4, SW = N / NPASS, HP = SW + 4;
    __shared__ __attribute__((aligned(16))) float s_t[NT / 64][16][HP];
    float (*tw)[HP] = s_t[q.tid >> 6];
    const int li = q.lane & 15, lq = q.lane >> 4, ch = q.lane & 31;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      if (ps > 0) __builtin_amdgcn_sched_barrier(0);   // the last slice's operands are consumed
      if (ch / (SW / 4) == ps) {
#pragma unroll
        for (int k = 0; k < NLD; ++k)
          st4(&tw[2 * k + (q.lane >> 5)][4 * (ch % (SW / 4))],
              f32x4{f[k][0], f[k][1], f[k][2], f[k][3]});
      }
#pragma unroll
      for (int cb = 0; cb < SW / 16; ++cb) {
        const f32x4 bv = ld4(&tw[li][16 * cb + 4 * lq]);
        const int n0 = ps * SW + 16 * cb + 4 * lq;
        const f32x4 av = li < NPAD ? ld4(&s_C[li < NPAD ? li : 0][n0]) : f32x4{0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc, 0, 0, 0);
      }
    }
    __syncthreads();   // s_yb, s_gam complete
    // register r of lane (li, lq): draft 4 lq + r, row 16 w + li
    const int pr = 16 * (q.tid >> 6) + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * lq + r;
      if (j < NPAD && j < n) {
        float yv;
        if (ok) {
          float yb = 0.f;
#pragma unroll
          for (int g = 0; g < QD; ++g) yb += s_yb[g][j][pr];
          yv = s_gam[j] * acc[r] + yb + Dh * s_xe[e0 + j][pr];
        } else {
          yv = __builtin_nanf("");
        }
        a.y[j * sx + q.unit * P + pr] = yv;
      }
    }
  } else if constexpr (W16) {
    constexpr int RS = NLD / 2;        // rows per lane
    constexpr int V = RS * NPAD;       // partial sums per lane: row k, draft j at k * NPAD + j
    using M = XMap<V, 16>;
    static_assert(M::BFLY == 0, "every lane writes");
    const int c16 = q.tid & 15, r0 = q.tid >> 4;
    float d[V];
#pragma unroll
    for (int j = 0; j < NPAD; ++j) {
      const f32x4 c0 = ld4(&s_C[j][4 * c16]), c1 = ld4(&s_C[j][64 + 4 * c16]);
#pragma unroll
      for (int k = 0; k < RS; ++k)   // C_j of an absent draft is zero in s_C
        d[k * NPAD + j] = f[2 * k][0] * c0.x + f[2 * k][1] * c0.y + f[2 * k][2] * c0.z +
                          f[2 * k][3] * c0.w + f[2 * k + 1][0] * c1.x + f[2 * k + 1][1] * c1.y +
                          f[2 * k + 1][2] * c1.z + f[2 * k + 1][3] * c1.w;
    }
    xreduce<V, 16>(d, q.lane);
    __syncthreads();   // s_yb, s_gam complete; every wave is past its reads of s_C
    float (*s_out)[CP] = s_C;   // the drafts' rows of outputs, staged in s_C
#pragma unroll
    for (int jj = 0; jj < M::VOUT; ++jj) {
      const int idx = M::index(q.lane, jj);
      const int k = idx / NPAD, j = idx % NPAD;
      const int pr = r0 + 16 * k;
      float yv;
      if (ok) {
        float yb = 0.f;
#pragma unroll
        for (int g = 0; g < QD; ++g) yb += s_yb[g][j][pr];
        yv = s_gam[j] * d[jj] + yb + Dh * s_xe[e0 + j][pr];
      } else {
        yv = __builtin_nanf("");
      }
      s_out[j][pr] = yv;
    }
    __syncthreads();
    {  // each draft's row of P outputs as 16 float4 stores
      static_assert(NPAD * P / 4 <= NT, "one float4 per thread");
      const int j = q.tid / (P / 4), c = q.tid % (P / 4);
      if (j < n) st4(a.y + j * sx + q.unit * P + 4 * c, ld4(&s_out[j][4 * c]));
    }
  } else {
    // Row dots with every C_j, reduced across the LPR lanes of a row.  At most
    // 32 partial sums per lane at a time: drafts go in chunks of JC.
    constexpr int JC = (Gm::NLD * NPAD <= 32) ? NPAD : 32 / Gm::NLD;
    constexpr int NCH = NPAD / JC;
    constexpr int V = Gm::NLD * JC;
    using M = XMap<V, Gm::LPR>;
    float res[NCH][M::VOUT];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      // keep the scheduler from hoisting this chunk's LDS reads into the last
      if (c > 0) __builtin_amdgcn_sched_barrier(0);
      float d[V];
#pragma unroll
      for (int jl = 0; jl < JC; ++jl) {   // C_j's segment once per draft, then every row
        const int j = c * JC + jl;
        float cj[Gm::EPL];
#pragma unroll
        for (int e = 0; e < Gm::EPL; e += 4) {
          const f32x4 cv = ld4(&s_C[j][cl * Gm::EPL + e]);
          cj[e] = cv.x; cj[e + 1] = cv.y; cj[e + 2] = cv.z; cj[e + 3] = cv.w;
        }
#pragma unroll
        for (int k = 0; k < Gm::NLD; ++k) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < Gm::EPL; ++e) acc += f[k][e] * cj[e];
          d[k * JC + jl] = acc;
        }
      }
      xreduce<V, Gm::LPR>(d, q.lane);
#pragma unroll
      for (int jj = 0; jj < M::VOUT; ++jj) res[c][jj] = d[jj];
    }
    __syncthreads();
    if (M::writer(q.lane)) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int jj = 0; jj < M::VOUT; ++jj) {
          const int idx = M::index(q.lane, jj);
          const int k = idx / JC, j = c * JC + idx % JC;
          if (j < n) {
            const int pr = k * Gm::RPL + rr0;
            float yv;
            if (ok) {
              float yb = 0.f;
#pragma unroll
              for (int g = 0; g < QD; ++g) yb += s_yb[g][j][pr];
              yv = s_gam[j] * (scale * res[c][jj]) + yb + Dh * s_xe[e0 + j][pr];
            } else {
              yv = __builtin_nanf("");
            }
            if constexpr (COMMIT)
              a.y[j * sx + q.unit * P + pr] = yv;
            else
              s_C[j][pr] = yv;   // staged: every wave is past its reads of s_C
          }
        }
      }
    }
    if constexpr (!COMMIT) {   // each draft's row of P outputs as float4 stores
      static_assert(NPAD * P / 4 <= NT, "one float4 per thread");
      __syncthreads();
      const int j = q.tid / (P / 4), c = q.tid % (P / 4);
      if (j < n) st4(a.y + j * sx + q.unit * P + 4 * c, ld4(&s_C[j][4 * c]));
    }
  }

  if constexpr (COMMIT) {
    if (fold) {   // h <- Gamma_buf h_c + sum_{i<len} fw_i x_i B_i^T, from the expanded tile
      f32x4 hv[NLD];   // the tile's own geometry
      const float gb = s_gbuf;
#pragma unroll
      for (int k = 0; k < NLD; ++k) hv[k] = gb * f32x4{f[k][0], f[k][1], f[k][2], f[k][3]};
      if constexpr (W16) {   // hv[2 k + hf]: row tid/16 + 16 k, column half hf
        const int c16 = q.tid & 15, rw = q.tid >> 4;
        for (int i = 0; i < len; ++i) {
          const f32x4 b0 = ld4(&s_Be[i][4 * c16]), b1 = ld4(&s_Be[i][64 + 4 * c16]);
          const float w = s_fw[i];
#pragma unroll
          for (int k = 0; k < NLD / 2; ++k) {
            const float xw = w * s_xe[i][rw + 16 * k];
            hv[2 * k] += xw * b0;
            hv[2 * k + 1] += xw * b1;
          }
        }
        float* ck = a.ckpt + q.unit * (P * N) + rw * N + 4 * c16;
#pragma unroll
        for (int k = 0; k < NLD / 2; ++k) {
          st_nt(ck + 16 * k * N, hv[2 * k]);
          st_nt(ck + 16 * k * N + 64, hv[2 * k + 1]);
        }
      } else {   // the fp32 read geometry is the tile geometry
        for (int i = 0; i < len; ++i) {
          const f32x4 bi = ld4(&s_Be[i][q.c4 * 4]);
          const float w = s_fw[i];
#pragma unroll
          for (int k = 0; k < NLD; ++k) hv[k] += (w * s_xe[i][rowk(k)]) * bi;
        }
        float* ck = a.ckpt + q.unit * (P * N) + q.c4 * 4;
#pragma unroll
        for (int k = 0; k < NLD; ++k) st_nt(ck + rowk(k) * N, hv[k]);
      }
    }
  }

  if (ok && a.append) {   // append the drafts (a chain) from LDS
    for (int j = 0; j < n; ++j) {
      const int s = ring_slot(slot0, len + j, cap);
      if (q.tid < P) a.ring_x[(q.unit * cap + s) * P + q.tid] = s_xe[e0 + j][q.tid];
      if (q.tid == 0) a.ring_dt[q.unit * cap + s] = s_dta[j];
      if ((q.h % (a.H / a.G)) == 0 && q.tid < N)
        a.ring_B[(q.gunit * cap + s) * N + q.tid] = s_Be[e0 + j][q.tid];
    }
  }

  IndexUpdate u;   // a rollback passed with the drafts stands even if they overflow
  u.apply = (ok && (a.append || fold)) || rl.rolled;
  u.pos_add = fold ? len : 0;
  u.new_len = ok ? (fold ? 0 : len) + (a.append ? n : 0) : len;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H, arrived, u);
  if (last_arrival(arrived, a.H)) {
    if (!ok) raise_status(a.status, valid ? kStatusOverflow : kStatusIndex);
    if (rl.bad) raise_status(a.status, kStatusRollback);
  }
}

// ----------------------------------------------------------- append path ----
// Append, for every sequence b, the drafts path[b][0..path_len[b]) (indices
// into the verify inputs) at entries len.., then len += path_len.  One
// workgroup per (sequence, group) copies the group's B and its heads' x and dt
// with 16-byte accesses; the workgroups of a sequence count themselves in its
// arrival counter and the last one moves len.  A path that would overflow the
// ring, or names a draft outside 0..n_pos-1, leaves the sequence unchanged and
// raises RSSM_STATUS_OVERFLOW (every workgroup of the sequence sees the same
// path and takes the same decision).
__global__ __launch_bounds__(NT) void m2_append_path_kernel(M2Args a) {
  const int tile = tile_index();
  const int b = tile / a.G, g = tile - b * a.G;
  const int cap = a.cap, n = a.n_pos;
  const int len = a.len[b];
  const int64_t pos = a.pos[b];
  const int pl = a.path_len[b];
  const bool valid = indices_valid(len, pos, cap);
  bool ok = valid && pl >= 0 && pl <= a.depth && len + pl <= cap;
  for (int k = 0; ok && k < pl; ++k) {
    const int j = a.path[(long)b * a.depth + k];
    ok = j >= 0 && j < n;
  }
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, b, len, pos, a.idx_ro);
  if (ok) {
    const int slot0 = (int)(pos % cap);
    const int hpg = a.H / a.G;
    const long sx = (long)a.batch * a.H * P, sg = (long)a.batch * a.G * N, sd = (long)a.batch * a.H;
    const long gunit = (long)b * a.G + g;
    const long unit0 = (long)b * a.H + (long)g * hpg;   // first head of the group
    const int XV = hpg * (P / 4), BV = N / 4;           // float4 chunks per entry
    for (int e = threadIdx.x; e < pl * (XV + BV); e += NT) {
      const int k = e / (XV + BV), c = e - k * (XV + BV);
      const int j = a.path[(long)b * a.depth + k];
      const int sl = ring_slot(slot0, len + k, cap);
      if (c < XV) {
        const long unit = unit0 + c / (P / 4);
        const int o = 4 * (c % (P / 4));
        st4(a.ring_x + (unit * cap + sl) * P + o, ld4(a.x + j * sx + unit * P + o));
      } else {
        const int o = 4 * (c - XV);
        st4(a.ring_B + (gunit * cap + sl) * N + o, ld4(a.B + j * sg + gunit * N + o));
      }
    }
    for (int e = threadIdx.x; e < pl * hpg; e += NT) {
      const int k = e / hpg, hh = e - k * hpg;
      const int j = a.path[(long)b * a.depth + k];
      const long unit = unit0 + hh;
      a.ring_dt[unit * cap + ring_slot(slot0, len + k, cap)] = a.dt[j * sd + unit];
    }
  }
  IndexUpdate u;
  u.apply = ok;
  u.pos_add = 0;
  u.new_len = len + pl;
  finish_update(a.arrive, a.pos, a.len, b, a.G, arrived, u);
  if (!ok && last_arrival(arrived, a.G))
    raise_status(a.status, valid ? kStatusOverflow : kStatusIndex);
}

// --------------------------------------------------------------- eager ----
// Read the whole state, update it, write it back, every step.  LP = 0: the
// fp32 checkpoint.  LP = bf16 / E4M3: the comparator that keeps the state in
// low precision only (the shared scheme's copy): decode, update in fp32,
// output from the updated values, re-encode, so that the rounding of every
// step feeds the next one.
template <int LP>
__global__ __launch_bounds__(NT) void m2_eager_kernel(M2Args a) {
  const Geo q = geometry<1, LP == 0>(a);
  float* ck = a.ckpt + q.unit * (P * N);
  char* lp = reinterpret_cast<char*>(a.ckpt_lp) + q.unit * (P * N) * (LP == kLpBf16 ? 2 : 1);
  float* lps = a.lp_scale ? a.lp_scale + q.unit : nullptr;
  f32x4 hv[NLD];
  if constexpr (LP == 0)
    load_tile(ck, q, hv);
  else
    load_lp_tile<LP, NLD, RPL, N>(hv, lp, lps, q.r0, q.c4);
  const float dtv = a.dt[q.unit];
  const float dec = expf(dtv * a.A[q.h]);
  const float* xt = a.x + q.unit * P;
  const f32x4 bb = ld4(a.B + q.gunit * N + q.c4 * 4);
  const f32x4 cc = ld4(a.C + q.gunit * N + q.c4 * 4);
  float d[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const float xv = dtv * xt[k * RPL + q.r0];
    hv[k] = dec * hv[k] + xv * bb;
    d[k] = dot4(hv[k], cc);
  }
  if constexpr (LP == 0) {
    store_tile(ck, q, hv);
  } else {
    __shared__ float s_red[NT / 64];
    store_lp_tile<LP, NT, NLD, RPL, N>(hv, lp, lps, a.status, q.r0, q.c4, s_red);
  }
  xreduce<NLD, LPR>(d, q.lane);
  using M = XMap<NLD, LPR>;
  if (M::writer(q.lane)) {
    const int p = M::index(q.lane, 0) * RPL + q.r0;
    a.y[q.unit * P + p] = d[0] + a.D[q.h] * xt[p];
  }
}

}  // namespace

hipError_t launch_m2_step(const M2Args& a, bool fused, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  // E4M3: two heads per workgroup when a group's head count allows it
  const bool pair = (a.H / a.G) % 2 == 0;
  const dim3 grid2((unsigned)(a.batch * (a.H / 2)));
  if (a.scheme == kSchemeF32 && a.cap > kMaxCap) {   // rings of up to 32 entries
    if (fused)
      hipLaunchKernelGGL((m2_step_kernel<4, true, 1, 0, kMaxCapM2>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((m2_step_kernel<4, false, 1, 0, kMaxCapM2>), grid, block, 0, s, a);
  } else if (a.scheme == kSchemeF32) {
    if (fused)
      hipLaunchKernelGGL((m2_step_kernel<4, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((m2_step_kernel<4, false>), grid, block, 0, s, a);
  } else if (fused) {   // DUAL (checked by the caller): fold fp32, re-quantise the copy
    if (a.lp == kLpBf16)
      hipLaunchKernelGGL((m2_step_kernel<4, true, 1, kLpBf16>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((m2_step_kernel<4, true, 1, kLpE4m3>), grid, block, 0, s, a);
  } else if (a.lp == kLpBf16) {
    hipLaunchKernelGGL((m2_step_kernel<2, false>), grid, block, 0, s, a);
  } else {
    if (pair)
      hipLaunchKernelGGL((m2_step_kernel<1, false, 2>), grid2, block, 0, s, a);
    else
      hipLaunchKernelGGL((m2_step_kernel<1, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_m2_commit(const M2Args& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  if (a.scheme == kSchemeF32 && a.cap > kMaxCap)
    hipLaunchKernelGGL((m2_commit_kernel<kSchemeF32, 0, kMaxCapM2>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeF32)
    hipLaunchKernelGGL((m2_commit_kernel<kSchemeF32, 0>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual && a.lp == kLpBf16)
    hipLaunchKernelGGL((m2_commit_kernel<kSchemeDual, kLpBf16>), grid, block, 0, s, a);
  else if (a.scheme == kSchemeDual)
    hipLaunchKernelGGL((m2_commit_kernel<kSchemeDual, kLpE4m3>), grid, block, 0, s, a);
  else if (a.lp == kLpBf16)
    hipLaunchKernelGGL((m2_commit_kernel<kSchemeShared, kLpBf16>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((m2_commit_kernel<kSchemeShared, kLpE4m3>), grid, block, 0, s, a);
  return hipGetLastError();
}

// The matrix-core contraction of verify (MF above) is correct but slower at
// the serving shape than the FMA dots with DPP reductions (4 drafts 167 vs
// 137 us, 8 drafts 202 vs 164 us, with the folded commit 207 vs 165 us per
// launch at batch 256 x 80 heads), so the FMA path is the default; building
// with -DRSSM_M2_VERIFY_MFMA selects MF for fp32 verification of 3-8 drafts.
#ifdef RSSM_M2_VERIFY_MFMA
constexpr bool kVerifyMfma = true;
#else
constexpr bool kVerifyMfma = false;
#endif

template <int EB, bool COMMIT = false>
static void launch_m2_verify_eb(const M2Args& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  constexpr bool MF = EB == 4 && kVerifyMfma;   // fp32, 3-8 drafts on the matrix cores
  if (a.n_pos <= 1)
    hipLaunchKernelGGL((m2_verify_kernel<EB, 1, COMMIT>), grid, block, 0, s, a);
  else if (a.n_pos <= 2)
    hipLaunchKernelGGL((m2_verify_kernel<EB, 2, COMMIT>), grid, block, 0, s, a);
  else if (a.n_pos <= 4)
    hipLaunchKernelGGL((m2_verify_kernel<EB, 4, COMMIT, MF>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((m2_verify_kernel<EB, 8, COMMIT, MF>), grid, block, 0, s, a);
}

hipError_t launch_m2_verify(const M2Args& a, hipStream_t s) {
  if (a.min_len > 0)   // fused commit (fp32 checkpoint; checked by the caller)
    launch_m2_verify_eb<4, true>(a, s);
  else if (a.scheme == kSchemeF32)
    launch_m2_verify_eb<4>(a, s);
  else if (a.lp == kLpBf16)
    launch_m2_verify_eb<2>(a, s);
  else
    launch_m2_verify_eb<1>(a, s);
  return hipGetLastError();
}

hipError_t launch_m2_append_path(const M2Args& a, hipStream_t s) {
  hipLaunchKernelGGL(m2_append_path_kernel, dim3((unsigned)(a.batch * a.G)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_m2_eager(const M2Args& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.H)), block(NT);
  if (a.scheme != kSchemeShared)
    hipLaunchKernelGGL((m2_eager_kernel<0>), grid, block, 0, s, a);
  else if (a.lp == kLpBf16)
    hipLaunchKernelGGL((m2_eager_kernel<kLpBf16>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((m2_eager_kernel<kLpE4m3>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace rssm
