// gdn_kernels.hip -- Gated DeltaNet decode kernels for gfx950.
//
// State of one (sequence, head): S[dv=128][dk=128], 64 KiB in fp32, 32 KiB in
// bf16, 16 KiB in E4M3 (+ one fp32 scale).  The state is read with 16-byte
// lane loads: a row of dk elements is spread over LPR = dk / (16 / element
// bytes) consecutive lanes.  Kernels whose work is row-independent (replay
// step, fused and fp32 commit, eager) run one 256-thread workgroup per half
// head (64 rows): 16,384 workgroups at batch 256 x 32 heads, each with a
// small register and LDS footprint so that several fit on a CU.  Kernels
// that need a whole head at once (the per-head E4M3 scale of a
// low-precision commit, the per-draft waves of verify) run one 512-thread
// workgroup per head.
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
#include "lp_codec.hpp"

namespace rssm {
namespace {

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int kSchemeF32 = 0, kSchemeDual = 1, kSchemeShared = 2;

// Lane geometry: NTH threads cover ROWS rows of a head's state with 16-byte
// lane loads of EB-byte elements.
template <int EB, int NTH, int ROWS>
struct LpGeo {
  static constexpr int EPL = 16 / EB;   // elements per lane load
  static constexpr int LPR = DK / EPL;  // lanes per state row
  static constexpr int RPL = NTH / LPR; // rows per workgroup-wide load
  static constexpr int NLD = ROWS / RPL;// loads per thread
  static_assert(LPR <= 64 && 64 % LPR == 0, "row must sit in one wave");
  static_assert(ROWS % RPL == 0, "tile geometry");
};

struct Geo {
  int b, h, tid, lane, cl, r0, row0;
  long unit;
};

// Workgroup -> (sequence b, head h, row block): row blocks of a head are
// adjacent, heads of a sequence are adjacent.  SPLIT: every XCD takes an
// eighth of each sequence's tiles (tile_index_split), else whole sequences
// (tile_index); each kernel takes the order that measured faster for it.
template <int LPR, int ROWS, bool SPLIT = false>
__device__ __forceinline__ Geo geometry(const GdnArgs& a) {
  constexpr int PARTS = DV / ROWS;
  Geo q;
  const int tile = SPLIT ? tile_index_split(a.H * PARTS) : tile_index();
  const int hp = tile / PARTS;
  q.row0 = (tile - hp * PARTS) * ROWS;
  q.b = hp / a.H;
  q.h = hp - q.b * a.H;
  q.tid = threadIdx.x;
  q.lane = q.tid & 63;
  q.cl = q.tid % LPR;
  q.r0 = q.tid / LPR;
  q.unit = (long)q.b * a.H + q.h;
  return q;
}

// First byte of row `row0` of head `unit`'s state (fp32 checkpoint for EB 4,
// the low-precision copy otherwise).
template <int EB>
__device__ __forceinline__ const char* state_base(const GdnArgs& a, long unit, int row0) {
  if constexpr (EB == 4)
    return reinterpret_cast<const char*>(a.ckpt + unit * (DV * DK) + row0 * DK);
  else
    return reinterpret_cast<const char*>(a.ckpt_lp) + (unit * (DV * DK) + row0 * DK) * EB;
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
// k rows are padded by 4 floats so that the 16 rows read by one MFMA operand
// load (16 lanes, one row each) start in different LDS banks.
constexpr int kKPitch = DK + 4;
struct EntrySmem {
  float k[kMaxCap][kKPitch];
  float v[kMaxCap][kKPitch];
  float al[kMaxCap], be[kMaxCap];
};

template <int NTH>
struct EntryRegs {
  static constexpr int EPT = kMaxCap * (DK / 4) / NTH;   // float4 chunks per thread
  static_assert(EPT * NTH == kMaxCap * (DK / 4) && DK == DV, "entry chunking");
  f32x4 k[EPT], v[EPT];
  float al, be;
};

template <int NTH>
__device__ __forceinline__ EntryRegs<NTH> fetch_entries(const Src& src, int L, int tid) {
  EntryRegs<NTH> e;
#pragma unroll
  for (int x = 0; x < EntryRegs<NTH>::EPT; ++x) {
    const int ch = tid + x * NTH, i = ch / (DK / 4), c = (ch % (DK / 4)) * 4;
    e.k[x] = e.v[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < L) {
      e.k[x] = ld4(src.k(i) + c);
      e.v[x] = ld4(src.v(i) + c);
    }
  }
  e.al = e.be = 0.f;
  if (tid < L) {
    e.al = src.alpha(tid);
    e.be = src.beta(tid);
  }
  return e;
}

// Park the fetched entries in LDS.  Rows L..kMaxCap-1 are written as zeros
// (fetch_entries zero-fills them), which pads the MFMA operands of the fold.
template <int NTH>
__device__ __forceinline__ void stash_entries(const EntryRegs<NTH>& e, int L, int tid,
                                              EntrySmem& s) {
  (void)L;
#pragma unroll
  for (int x = 0; x < EntryRegs<NTH>::EPT; ++x) {
    const int ch = tid + x * NTH, i = ch / (DK / 4), c = (ch % (DK / 4)) * 4;
    st4(&s.k[i][c], e.k[x]);
    st4(&s.v[i][c], e.v[x]);
  }
  if (tid < kMaxCap) {
    s.al[tid] = e.al;
    s.be[tid] = e.be;
  }
}

// Write entry i (held in registers by fetch_entries) to its ring slot.
template <int NTH>
__device__ __forceinline__ void append_from_regs(const GdnArgs& a, const Src& src,
                                                 const EntryRegs<NTH>& e, int i, int tid) {
  const int s = ring_slot(src.slot0, i, src.cap);
  const long u = src.unit;
#pragma unroll
  for (int x = 0; x < EntryRegs<NTH>::EPT; ++x) {
    const int ch = tid + x * NTH, ei = ch / (DK / 4), c = (ch % (DK / 4)) * 4;
    if (ei == i) {
      st4(a.ring_k + (u * src.cap + s) * DK + c, e.k[x]);
      st4(a.ring_v + (u * src.cap + s) * DV + c, e.v[x]);
    }
  }
  if (tid == i) {
    a.ring_a[u * src.cap + s] = e.al;
    a.ring_b[u * src.cap + s] = e.be;
  }
}

// The drafts i0..i0+n-1 appended from the entries parked in LDS, 32 threads
// per draft (the fetch registers are then free for the rest of the kernel).
template <int NTH>
__device__ __forceinline__ void append_drafts_from_smem(const GdnArgs& a, const Src& src,
                                                        const EntrySmem& es, int i0, int n,
                                                        int tid) {
  static_assert(DK == DV, "k and v rows of one length");
  const int j = tid / (DK / 4), ch = tid % (DK / 4);
  if (j < n) {
    const int i = i0 + j;
    const long row = src.unit * src.cap + ring_slot(src.slot0, i, src.cap);
    st4(a.ring_k + row * DK + 4 * ch, ld4(&es.k[i][4 * ch]));
    st4(a.ring_v + row * DV + 4 * ch, ld4(&es.v[i][4 * ch]));
    if (ch == 0) {
      a.ring_a[row] = es.al[i];
      a.ring_b[row] = es.be[i];
    }
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
      part = group_sum<LPR>(part);
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

// As carry(), through the entries on one draft's path only: buffered entries
// lo..len-1 and the drafts whose bit is set in `anc` (entry len + m <-> bit
// m), up to entry hi.  A whole wave carries one query (LPR = 64 lanes of EPL
// elements, which are also rows cl*EPL.. of the value vectors): on the way it
// accumulates the replay term sum_i s_i v_i of those rows into rep, in the
// shadow of each entry's reduction.
template <int EPL, int LPR>
__device__ __forceinline__ void carry_path(const EntrySmem& s, int lo, int len, uint32_t anc,
                                           int hi, int cl, float (&q)[EPL], float (&rep)[EPL]) {
  static_assert(LPR * EPL == DV, "one wave carries a whole query");
#pragma unroll
  for (int e = 0; e < EPL; ++e) rep[e] = 0.f;
#pragma unroll
  for (int i = kMaxCap - 1; i >= 0; --i) {
    const bool on = i >= lo && i <= hi && (i < len || ((anc >> (i - len)) & 1u));
    if (on) {
      float kv[EPL], vv[EPL];
      load_vec<EPL>(&s.k[i][cl * EPL], kv);
      load_vec<EPL>(&s.v[i][cl * EPL], vv);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part += kv[e] * q[e];
      part = group_sum<LPR>(part);
      const float si = s.be[i] * part;
      const float al = s.al[i];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        rep[e] += si * vv[e];
        q[e] = al * (q[e] - si * kv[e]);
      }
    }
  }
}

// As carry(), for the replay step: instead of keeping every s_i, accumulate
// sum_i s_i v_i[r] for the lane's own output row r on the way.
template <int EPL, int LPR>
__device__ __forceinline__ float carry_acc(const EntrySmem& s, int hi, int cl, int r,
                                           float (&q)[EPL]) {
  float acc = 0.f;
#pragma unroll
  for (int i = kMaxCap - 1; i >= 0; --i) {
    if (i <= hi) {
      float kv[EPL];
      load_vec<EPL>(&s.k[i][cl * EPL], kv);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part += kv[e] * q[e];
      part = group_sum<LPR>(part);
      const float si = s.be[i] * part;
      const float al = s.al[i];
      acc += si * s.v[i][r];
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[e] = al * (q[e] - si * kv[e]);
    }
  }
  return acc;
}

// ---------------------------------------------------------------- fold ----
// With u_i = beta_i (v_i - alpha_i a_i) and a_i = G_{c+1..i-1} (S_c k_i)
// + sum_{m<i} G_{m+1..i-1} (k_m . k_i) u_m, every row satisfies the same unit
// lower-triangular system (I + diag(beta alpha) Lc) u = z with
// z_j = beta_j v_j - beta_j alpha_j G_{c+1..j-1} (S_c k_j) and
// Lc[i][m] = G_{m+1..i-1} (k_m . k_i).  Its inverse T is formed once per
// workgroup (L x L); each row's fold weights U'_i = G_{i+1..t} u_i are then
// independent short dot products, and the new state is
// S_new = G_{c+1..t} S_c + U' K (rank L).  The state stays in the
// consecutive-load geometry of the stream and the products run on fp32 FMA:
// a matrix-core version (v_mfma_f32_16x16x4f32) measured slower, because its
// operand layout (16 rows x 64 B per wave load) streams the state more slowly
// than consecutive bytes, half of each 16-wide block is padding at L = 8, and
// the ~4 L flop per element are hidden under the stream anyway.
template <int ROWS>
struct FoldSmem {
  float G[kMaxCap + 1][kMaxCap + 1];   // G[a][e] = prod_{j=a}^{e-1} alpha_j, a <= e <= L
  union {                              // gram is dead once Lc is formed
    float gram[kMaxCap][kMaxCap + 1];  // k_m . k_i
    float P1[kMaxCap][kMaxCap + 1];    //  G_{i+1..} T[i][j] beta_j
  };
  float Lc[kMaxCap][kMaxCap + 1];      // G_{m+1..i-1} (k_m . k_i), m < i
  float P2[kMaxCap][kMaxCap + 1];      // -G_{i+1..} T[i][j] beta_j alpha_j G_{..j-1}
  float WU[ROWS][kMaxCap + 1];         // S_c k_i of the workgroup's rows, then U'_i
  float red[16];
};

// Gram matrix (16 lanes per pair) and the alpha product table.
template <int NTH, int ROWS>
__device__ __forceinline__ void coef_gram_g(const EntrySmem& es, int L, int tid,
                                            FoldSmem<ROWS>& sm) {
  const int sgm = tid & 15;
  for (int pi = tid >> 4; pi < L * L; pi += NTH / 16) {   // uniform per 16 lanes
    const int m = pi / L, i = pi % L;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < DK / 16; ++e)
      part += es.k[m][sgm * (DK / 16) + e] * es.k[i][sgm * (DK / 16) + e];
    part = group_sum<16>(part);
    if (sgm == 0) sm.gram[m][i] = part;
  }
  for (int idx = tid; idx < (kMaxCap + 1) * (kMaxCap + 1); idx += NTH) {
    const int a0 = idx / (kMaxCap + 1), e0 = idx % (kMaxCap + 1);
    if (a0 <= e0 && e0 <= L) {
      float p = 1.f;
      for (int j = a0; j < e0; ++j) p *= es.al[j];
      sm.G[a0][e0] = p;
    }
  }
}

template <int NTH, int ROWS>
__device__ __forceinline__ void coef_lc(int L, int tid, FoldSmem<ROWS>& sm) {
  for (int idx = tid; idx < kMaxCap * kMaxCap; idx += NTH) {
    const int i = idx / kMaxCap, m = idx % kMaxCap;
    sm.Lc[i][m] = (m < i && i < L) ? sm.G[m + 1][i] * sm.gram[m][i] : 0.f;
  }
}

// T = (I + diag(beta alpha) Lc)^-1 column by column (one thread per column,
// in registers), folded into the fold-weight matrices P1 and P2.
template <int ROWS>
__device__ __forceinline__ void coef_t(const EntrySmem& es, int L, int tid, FoldSmem<ROWS>& sm) {
  if (tid < kMaxCap) {
    const int j = tid;
    float t[kMaxCap];
#pragma unroll
    for (int i = 0; i < kMaxCap; ++i) {
      float v = (i == j && j < L) ? 1.f : 0.f;
      if (i > j && i < L) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc += sm.Lc[i][m] * t[m];   // t[m] = 0 for m < j
        v = -es.be[i] * es.al[i] * acc;
      }
      t[i] = v;
    }
    const float bj = (j < L) ? es.be[j] : 0.f;
    const float bag = (j < L) ? es.be[j] * es.al[j] * sm.G[0][j] : 0.f;
#pragma unroll
    for (int i = 0; i < kMaxCap; ++i) {
      const float w = (i < L) ? sm.G[i + 1][L] * t[i] : 0.f;
      sm.P1[i][j] = w * bj;
      sm.P2[i][j] = -w * bag;
    }
  }
}

// W = S_c K^T for the workgroup's rows, CH entries at a time (FMA dots,
// transposed cross-lane reduction), stored to sm.WU.  CH = 2 keeps the
// partial dots to 2 NLD registers beside the 4 NLD of the tile, which gives
// the whole-head fold kernels a third workgroup per CU and the half-head fp32
// fused step and commit a sixth (with gram and P1 sharing LDS); the DUAL bf16
// step and commit measured faster with CH = 4.
template <int NTH, int ROWS, int NLD, int CH>
__device__ __forceinline__ void fold_w(const f32x4 (&hv)[NLD], const EntrySmem& es, int L,
                                       const Geo& q, FoldSmem<ROWS>& sm) {
  using Gm = LpGeo<4, NTH, ROWS>;
  constexpr int RPL = Gm::RPL, LPR = Gm::LPR;
  static_assert(NLD == Gm::NLD, "tile registers");
  using M = XMap<NLD * CH, LPR>;
  static_assert(M::VOUT == 1, "one sum per lane");
  for (int i0 = 0; i0 < L; i0 += CH) {
    float d[NLD * CH];
#pragma unroll
    for (int jj = 0; jj < CH; ++jj) {
      const f32x4 kv = ld4(&es.k[i0 + jj][q.cl * 4]);   // rows >= L are zero
#pragma unroll
      for (int k = 0; k < NLD; ++k) d[k * CH + jj] = dot4(hv[k], kv);
    }
    xreduce<NLD * CH, LPR>(d, q.lane);
    if (M::writer(q.lane)) {
      const int idx = M::index(q.lane, 0);
      sm.WU[(idx / CH) * RPL + q.r0][i0 + idx % CH] = d[0];
    }
  }
}

// U'[r][i] = sum_{j<=i} P1[i][j] v_j[row0 + r] + P2[i][j] W[r][j], written
// over W once every thread has read it (barrier inside).
template <int NTH, int ROWS>
__device__ __forceinline__ void fold_u(const EntrySmem& es, int L, int row0, int tid,
                                       FoldSmem<ROWS>& sm) {
  static_assert(NTH % ROWS == 0, "whole row groups");
  constexpr int IG = NTH / ROWS, NI = (kMaxCap + IG - 1) / IG;
  const int r = tid % ROWS, ig = tid / ROWS;
  float acc[NI];
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int i = ig + t * IG;
    acc[t] = 0.f;
    if (i < L) {
      // a bounded unroll: unrolled further, the LDS loads of every term are
      // hoisted next to the live state tile and the kernels that fold into a
      // tile they still read need ten more registers
#pragma unroll 4
      for (int j = 0; j <= i; ++j)
        acc[t] += sm.P1[i][j] * es.v[j][row0 + r] + sm.P2[i][j] * sm.WU[r][j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int i = ig + t * IG;
    if (i < L) sm.WU[r][i] = acc[t];
  }
}

template <int NTH, int ROWS, int NLD>
__device__ __forceinline__ void fold_update(f32x4 (&hv)[NLD], const EntrySmem& es, int L,
                                            const Geo& q, const FoldSmem<ROWS>& sm) {
  constexpr int RPL = LpGeo<4, NTH, ROWS>::RPL;
  const float gall = sm.G[0][L];
#pragma unroll
  for (int k = 0; k < NLD; ++k) hv[k] *= gall;
  for (int i = 0; i < L; ++i) {
    const f32x4 kv = ld4(&es.k[i][q.cl * 4]);
#pragma unroll
    for (int k = 0; k < NLD; ++k) hv[k] += sm.WU[k * RPL + q.r0][i] * kv;
  }
}

// The fold in two halves (all threads; barriers inside; L >= 1).  The first
// needs only the entries (Gram matrix, alpha products, the triangular
// inverse and the fold weights), so the kernels run it while the state
// stream is still in flight; the second needs the state tile.
template <int NTH, int ROWS>
__device__ __forceinline__ void fold_coef(const EntrySmem& es, int L, int tid, FoldSmem<ROWS>& sm) {
  coef_gram_g<NTH, ROWS>(es, L, tid, sm);
  __syncthreads();
  coef_lc<NTH, ROWS>(L, tid, sm);
  __syncthreads();
  coef_t<ROWS>(es, L, tid, sm);
  __syncthreads();
}

template <int NTH, int ROWS, int NLD, int WCH = 2>
__device__ __forceinline__ void fold_apply(f32x4 (&hv)[NLD], const EntrySmem& es, int L, int row0, const Geo& q,
                           FoldSmem<ROWS>& sm) {
  fold_w<NTH, ROWS, NLD, WCH>(hv, es, L, q, sm);
  __syncthreads();
  fold_u<NTH, ROWS>(es, L, row0, q.tid, sm);
  __syncthreads();
  fold_update<NTH, ROWS, NLD>(hv, es, L, q, sm);
}

using WholeGeo = LpGeo<4, 512, DV>;
constexpr int kWholeNLD = WholeGeo::NLD;

template <int LP>
__device__ __forceinline__ void store_lp(const f32x4 (&hv)[kWholeNLD], const GdnArgs& a,
                                         const Geo& q, float* red) {
  char* lp = reinterpret_cast<char*>(a.ckpt_lp) + q.unit * (DV * DK) * (LP == kLpBf16 ? 2 : 1);
  store_lp_tile<LP, 512, kWholeNLD, WholeGeo::RPL, DK>(
      hv, lp, a.lp_scale ? a.lp_scale + q.unit : nullptr, a.status, q.r0, q.cl, red);
}

template <int LP>
__device__ __forceinline__ void load_lp_as_f32(f32x4 (&hv)[kWholeNLD], const GdnArgs& a,
                                               const Geo& q) {
  const char* lp = reinterpret_cast<const char*>(a.ckpt_lp) + q.unit * (DV * DK) * (LP == kLpBf16 ? 2 : 1);
  load_lp_tile<LP, kWholeNLD, WholeGeo::RPL, DK>(hv, lp, a.lp_scale ? a.lp_scale + q.unit : nullptr,
                                                 q.r0, q.cl);
}

// fp32 rows of a workgroup in the consecutive-load geometry (eager kernel).
template <int RPL, int NLD>
__device__ __forceinline__ void load_f32_tile(f32x4 (&hv)[NLD], const float* rows, const Geo& q) {
#pragma unroll
  for (int k = 0; k < NLD; ++k) hv[k] = ld_nt(rows + (k * RPL + q.r0) * DK + q.cl * 4);
}

template <int RPL, int NLD>
__device__ __forceinline__ void store_f32_tile(const f32x4 (&hv)[NLD], float* rows, const Geo& q) {
#pragma unroll
  for (int k = 0; k < NLD; ++k) st_nt(rows + (k * RPL + q.r0) * DK + q.cl * 4, hv[k]);
}

// ---------------------------------------------------------------- step ----
// EB: bytes per checkpoint element read for the output (4: ckpt fp32; 2: bf16
// ckpt_lp; 1: E4M3 ckpt_lp).  One 256-thread workgroup per half head, state
// read with consecutive 16-byte lane loads.  Order: buffered entries and the
// query are fetched, then the state stream is issued, then the entries are
// parked in LDS while the stream is in flight.
constexpr int kStepThreads = 256;
constexpr int kStepRows = 64;
// Rows per step workgroup.  A low-precision head is 32 KiB (bf16) or 16 KiB
// (E4M3): half of it is too little stream to cover the workgroup's fixed
// chain (index read, entry fetch, backward carry), so those take whole heads.
template <int EB>
constexpr int step_rows() { return EB == 4 ? kStepRows : DV; }
// Threads per step workgroup: an E4M3 head (16 KiB) is read by 128 threads,
// so that every thread keeps eight 16-byte loads in flight as in the fp32 and
// bf16 steps.
template <int EB>
constexpr int step_threads() { return EB == 1 ? kStepThreads / 2 : kStepThreads; }

// LP (fused commit of a DUAL layer): the boundary step folds and stores the
// fp32 checkpoint as for F32, takes its output from the fp32 checkpoint, and
// writes the low-precision image of the folded state; the per-head E4M3 scale
// needs the whole head, so these take one 512-thread workgroup per head.
template <int EB, bool FUSED, int LP = 0>
__global__ __launch_bounds__((LP != 0 ? 512 : step_threads<EB>())) void gdn_step_kernel(GdnArgs a) {
  static_assert(LP == 0 || (FUSED && EB == 4), "a low-precision image is written only by the fused commit");
  constexpr int NTH = LP != 0 ? 512 : step_threads<EB>();
  constexpr int ROWS = LP != 0 ? DV : step_rows<EB>(), PARTS = DV / ROWS;
  using Gm = LpGeo<EB, NTH, ROWS>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPL = Gm::RPL, NLD = Gm::NLD;
  const Geo q = geometry<LPR, ROWS, !(FUSED && LP == 0)>(a);
  const int cap = a.cap;

  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  const bool valid = indices_valid(len, pos, cap);
  const bool ok = valid && len < cap;
  const int L = len + 1;
  Src src{&a, q.unit, len, valid ? (int)(pos % cap) : 0, cap, 0, 0};
  const float scale = (EB == 1) ? a.lp_scale[q.unit] : 1.f;

  EntryRegs<NTH> er = fetch_entries<NTH>(src, ok ? L : 0, q.tid);
  float qv[EPL];
  load_vec<EPL>(a.q + q.unit * DK + q.cl * EPL, qv);

  const char* base = state_base<EB>(a, q.unit, q.row0);
  u32x4 raw[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) raw[k] = ld_nt_u(base + ((k * RPL + q.r0) * DK + q.cl * EPL) * EB);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos, a.idx_ro);

  __shared__ __attribute__((aligned(16))) EntrySmem es;
  stash_entries<NTH>(er, ok ? L : 0, q.tid, es);
  __syncthreads();
  // fused commit: the fold's coefficients while the stream is in flight
  __shared__ __attribute__((aligned(16))) FoldSmem<FUSED ? ROWS : 1> sm;
  if constexpr (FUSED) {
    if (ok) fold_coef<NTH, ROWS>(es, L, q.tid, sm);
  }

  using M = XMap<NLD, LPR>;
  const int r_out = q.row0 + M::index(q.lane, 0) * RPL + q.r0;   // this lane's output row
  float d[NLD];

  if constexpr (FUSED) {
    // fold the whole buffer, this entry included, and store.  The folded
    // state is the state after this token, so the output is o_t = S_t q_t
    // read from it: no backward carry of the query.
    static_assert(EB == 4, "fused commit folds the fp32 checkpoint");
    if (ok) {
      f32x4 hv[NLD];
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        hv[k] = f32x4{__uint_as_float(raw[k].x), __uint_as_float(raw[k].y),
                      __uint_as_float(raw[k].z), __uint_as_float(raw[k].w)};
      fold_apply<NTH, ROWS, NLD, LP == kLpBf16 ? 4 : 2>(hv, es, L, q.row0, q, sm);
      const f32x4 q4 = {qv[0], qv[1], qv[2], qv[3]};
#pragma unroll
      for (int k = 0; k < NLD; ++k) d[k] = dot4(hv[k], q4);
      xreduce<NLD, LPR>(d, q.lane);
      if (M::writer(q.lane)) a.o[q.unit * DV + r_out] = d[0];
      store_f32_tile<RPL, NLD>(hv, a.ckpt + q.unit * (DV * DK) + q.row0 * DK, q);
      if constexpr (LP != 0) store_lp<LP>(hv, a, q, sm.red);   // DUAL: re-quantise the copy
    } else if (M::writer(q.lane)) {
      a.o[q.unit * DV + r_out] = __builtin_nanf("");
    }
  } else {
    float obuf = 0.f;
    if (ok) obuf = carry_acc<EPL, LPR>(es, L - 1, q.cl, r_out, qv);
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
    if (M::writer(q.lane)) a.o[q.unit * DV + r_out] = ok ? scale * d[0] + obuf : __builtin_nanf("");
    if (ok && q.row0 == 0) append_from_regs<NTH>(a, src, er, len, q.tid);
  }

  IndexUpdate u;
  u.apply = ok;
  u.pos_add = FUSED ? L : 0;
  u.new_len = FUSED ? 0 : L;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H * PARTS, arrived, u);
  if (!ok && last_arrival(arrived, a.H * PARTS))
    raise_status(a.status, valid ? kStatusOverflow : kStatusIndex);
}

// -------------------------------------------------------------- commit ----
// SCHEME/LP select: F32 (fold fp32; half-head workgroups), DUAL (fold fp32,
// then re-quantise the copy; whole-head workgroups for the per-head scale),
// SHARED (fold the dequantised copy, re-quantise; whole head).
template <int SCHEME, int LP, int NTH>
__global__ __launch_bounds__(NTH) void gdn_commit_kernel(GdnArgs a) {
  constexpr int ROWS = NTH / 4, PARTS = DV / ROWS;   // 32 lanes per row, 4 fp32 each
  using Gm = LpGeo<4, NTH, ROWS>;
  constexpr int RPL = Gm::RPL, NLD = Gm::NLD;
  static_assert(SCHEME == kSchemeF32 || ROWS == DV, "low-precision copies need whole heads");
  const Geo q = geometry<Gm::LPR, ROWS, SCHEME == kSchemeF32>(a);
  if (a.mask != nullptr && a.mask[q.b] == 0) return;   // uniform for the sequence
  const int len = a.len[q.b];
  const int64_t pos = a.pos[q.b];
  if (!indices_valid(len, pos, a.cap)) {    // refused: nothing read, written or counted
    if (q.h == 0 && q.row0 == 0 && q.tid == 0) raise_status(a.status, kStatusIndex);
    return;
  }
  // not due, or nothing to fold and nothing to refresh
  if (len < a.min_len || (len == 0 && SCHEME != kSchemeDual)) return;
  Src src{&a, q.unit, len, (int)(pos % a.cap), a.cap, 0, 0};
  EntryRegs<NTH> er = fetch_entries<NTH>(src, len, q.tid);
  float* rows = a.ckpt + q.unit * (DV * DK) + q.row0 * DK;
  f32x4 hv[NLD];
  if constexpr (SCHEME == kSchemeShared)
    load_lp_as_f32<LP>(hv, a, q);
  else
    load_f32_tile<RPL, NLD>(hv, rows, q);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos, a.idx_ro);
  __shared__ __attribute__((aligned(16))) EntrySmem es;
  __shared__ __attribute__((aligned(16))) FoldSmem<ROWS> sm;
  stash_entries<NTH>(er, len, q.tid, es);
  __syncthreads();
  if (len > 0) {
    fold_coef<NTH, ROWS>(es, len, q.tid, sm);   // while the state stream is in flight
    fold_apply<NTH, ROWS, NLD, (SCHEME == kSchemeDual && LP == kLpBf16) ? 4 : 2>(
        hv, es, len, q.row0, q, sm);
    if constexpr (SCHEME != kSchemeShared) store_f32_tile<RPL, NLD>(hv, rows, q);
  }
  if constexpr (SCHEME != kSchemeF32) store_lp<LP>(hv, a, q, sm.red);

  IndexUpdate u;
  u.apply = len > 0;
  u.pos_add = len;
  u.new_len = 0;
  finish_update(a.arrive, a.pos, a.len, q.b, a.H * PARTS, arrived, u);
}

// -------------------------------------------------------------- verify ----
// n_pos drafts at entries len..len+n-1; draft j's output uses the buffered
// entries and the drafts on its path (a.anc[j]); a chain (a.append) appends
// the drafts, a tree appends nothing.  One 512-thread workgroup per
// head: wave j carries draft j's query backwards through entries len+j..0;
// then one pass over the checkpoint dots every row with all carried queries.
// The chain's drafts are appended from LDS at the end, so no fetched entry
// stays in registers: four fp32 drafts take 57 registers (four workgroups per
// CU), eight 80 (three), and with the commit folded in 74 and 80 (three).
//
// COMMIT (fp32 checkpoint only): a sequence whose buffer holds at least
// a.min_len entries also folds those entries into its checkpoint from the
// same state read (the fold's coefficients while the stream is in flight, the
// rank-len update once it has arrived); its checkpoint moves to the end of
// the buffer and the drafts become entries 0..n-1 (the same ring slots).  Its
// outputs are read from the folded state, with the queries carried back
// through the drafts only: those of commit-then-verify.
template <int EB, int NPAD, bool COMMIT = false>
__global__ __launch_bounds__(512) void gdn_verify_kernel(GdnArgs a) {
  static_assert(!COMMIT || EB == 4, "the fused commit folds the fp32 checkpoint");
  constexpr int NTH = 512, ROWS = DV;
  using Gm = LpGeo<EB, NTH, ROWS>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPL = Gm::RPL, NLD = Gm::NLD;
  static_assert(NPAD <= NTH / 64 && NPAD * (DK / 4) <= NTH, "one wave per draft position");
  const Geo q = geometry<LPR, ROWS, NPAD != 8 || COMMIT>(a);
  const int cap = a.cap, n = a.n_pos;

  const int64_t pos = a.pos[q.b];
  const RolledLen rl = rolled_len(a.len[q.b], pos, cap, a.n_reject, q.b);
  const int len = rl.len;
  const bool valid = rl.valid;
  const bool ok = valid && len + n <= cap;
  const bool fold = COMMIT && ok && len > 0 && len >= a.min_len;   // uniform per sequence
  const long sk = (long)a.batch * a.H * DK;
  const long sd = (long)a.batch * a.H;
  Src src{&a, q.unit, len, valid ? (int)(pos % cap) : 0, cap, sk, sd};
  const float scale = (EB == 1) ? a.lp_scale[q.unit] : 1.f;

  EntryRegs<NTH> er = fetch_entries<NTH>(src, ok ? len + n : 0, q.tid);
  const int w = q.tid >> 6;
  float qv[2] = {0.f, 0.f};
  if (ok && w < n) load_vec<2>(a.q + w * sk + q.unit * DK + 2 * q.lane, qv);

  const char* base = state_base<EB>(a, q.unit, 0);
  u32x4 raw[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) raw[k] = ld_nt_u(base + ((k * RPL + q.r0) * DK + q.cl * EPL) * EB);
  indices_consumed(len, pos);
  const uint32_t arrived = arrive_early(a.arrive, q.b, len, pos, a.idx_ro);

  __shared__ __attribute__((aligned(16))) EntrySmem es;
  __shared__ __attribute__((aligned(16))) float s_q[NPAD][DK];
  __shared__ __attribute__((aligned(16))) float s_rep[NPAD][DV];   // sum_i s_i v_i per draft
  stash_entries<NTH>(er, ok ? len + n : 0, q.tid, es);
  __syncthreads();
  __shared__ __attribute__((aligned(16))) FoldSmem<COMMIT ? ROWS : 1> sm;
  if constexpr (COMMIT) {
    if (fold) fold_coef<NTH, ROWS>(es, len, q.tid, sm);   // while the stream is in flight
  }

  if (ok && w < n) {  // wave w carries draft w (2 elements per lane)
    // its path mask, read with uniform indices (kernel-argument loads), never
    // indexed by the lane-derived w
    uint32_t anc = 0u;
#pragma unroll
    for (int j = 0; j < NPAD; ++j)
      if (w == j) anc = a.anc[j];
    // a folding sequence takes its outputs from the folded state: the carry
    // then runs through the drafts only
    float rep[2];
    carry_path<2, 64>(es, fold ? len : 0, len, anc, len + w, q.lane, qv, rep);
    s_q[w][2 * q.lane] = qv[0];
    s_q[w][2 * q.lane + 1] = qv[1];
    s_rep[w][2 * q.lane] = rep[0];
    s_rep[w][2 * q.lane + 1] = rep[1];
  }
  __syncthreads();
  f32x4 hv[COMMIT ? NLD : 1];
  if constexpr (COMMIT) {
    if (fold) {   // the buffered entries folded into the fp32 checkpoint first
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        hv[k] = f32x4{__uint_as_float(raw[k].x), __uint_as_float(raw[k].y),
                      __uint_as_float(raw[k].z), __uint_as_float(raw[k].w)};
      fold_apply<NTH, ROWS, NLD>(hv, es, len, 0, q, sm);
      store_f32_tile<RPL, NLD>(hv, a.ckpt + q.unit * (DV * DK), q);
#pragma unroll
      for (int k = 0; k < NLD; ++k)   // the rows the outputs read
        raw[k] = u32x4{__float_as_uint(hv[k].x), __float_as_uint(hv[k].y),
                       __float_as_uint(hv[k].z), __float_as_uint(hv[k].w)};
    }
  }

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
  // the outputs are staged in s_q and written a draft's row at a time where
  // that measured faster (no fold, or eight drafts)
  constexpr bool STAGE = !COMMIT || NPAD == 8;
  if constexpr (STAGE) __syncthreads();   // every wave is past its reads of s_q
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
          ov = scale * d[jj] + s_rep[j][r];
        } else {
          ov = __builtin_nanf("");
        }
        if constexpr (STAGE)
          s_q[j][r] = ov;
        else
          a.o[j * (long)a.batch * a.H * DV + q.unit * DV + r] = ov;
      }
    }
  }
  if constexpr (STAGE) {   // each draft's row of DV outputs as float4 stores
    static_assert(NPAD * DV / 4 <= NTH && DV == DK, "one float4 per thread");
    __syncthreads();
    const int j = q.tid / (DV / 4), c = q.tid % (DV / 4);
    if (j < n) st4(a.o + j * (long)a.batch * a.H * DV + q.unit * DV + 4 * c, ld4(&s_q[j][4 * c]));
  }
  if (ok)
    if (a.append)
      append_drafts_from_smem<NTH>(a, src, es, len, n, q.tid);

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

// --------------------------------------------------------------- eager ----
// Per row r: (S k)_r, then S_r <- alpha S_r + beta (v_r - alpha (S k)_r) k^T,
// then o_r = S_r . q with the updated row; the state is written back.
// LP = 0: the fp32 checkpoint, one 256-thread workgroup per half head.
// LP = bf16 / E4M3: the comparator that keeps the state in low precision only
// (decode, update in fp32, output from the updated rows, re-encode), one
// 512-thread workgroup per head for the per-head scale.
template <int LP>
__global__ __launch_bounds__(LP == 0 ? kStepThreads : 512) void gdn_eager_kernel(GdnArgs a) {
  constexpr int NTH = LP == 0 ? kStepThreads : 512, ROWS = LP == 0 ? kStepRows : DV;
  using Gm = LpGeo<4, NTH, ROWS>;
  constexpr int RPL = Gm::RPL, NLD = Gm::NLD, LPR = Gm::LPR;
  const Geo q = geometry<LPR, ROWS, LP == 0>(a);
  const f32x4 kv = ld4(a.k + q.unit * DK + q.cl * 4);
  const f32x4 qv = ld4(a.q + q.unit * DK + q.cl * 4);
  const float al = a.alpha[q.unit], be = a.beta[q.unit];
  const float* vv = a.v + q.unit * DV + q.row0;
  float vr[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) vr[k] = vv[k * RPL + q.r0];
  float* rows = a.ckpt + q.unit * (DV * DK) + q.row0 * DK;
  f32x4 hv[NLD];
  if constexpr (LP == 0)
    load_f32_tile<RPL, NLD>(hv, rows, q);
  else
    load_lp_as_f32<LP>(hv, a, q);
  float sk[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) sk[k] = dot4(hv[k], kv);
  allreduce<NLD, LPR>(sk);
  float d[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const float coef = be * (vr[k] - al * sk[k]);
    hv[k] = al * hv[k] + coef * kv;
    d[k] = dot4(hv[k], qv);
  }
  if constexpr (LP == 0) {
    store_f32_tile<RPL, NLD>(hv, rows, q);
  } else {
    __shared__ float s_red[NTH / 64];
    store_lp<LP>(hv, a, q, s_red);
  }
  xreduce<NLD, LPR>(d, q.lane);
  using M = XMap<NLD, LPR>;
  if (M::writer(q.lane)) {
    const int r = q.row0 + M::index(q.lane, 0) * RPL + q.r0;
    a.o[q.unit * DV + r] = d[0];
  }
}

// ----------------------------------------------------------- append path ----
// As m2_append_path_kernel, one workgroup per HPW heads of a sequence: the
// heads' k, v, alpha and beta of the drafts path[b][0..path_len[b]) are
// appended at entries len.. with 16-byte accesses, and the last workgroup of
// the sequence sets len += path_len; an overflowing or out-of-range path
// leaves the sequence unchanged and raises RSSM_STATUS_OVERFLOW.  Four heads
// per workgroup (2,048 workgroups at batch 256 x 32 heads instead of 8,192)
// took the launch from 14.4 to 9.5 us: the copy per head is only a few KiB
// behind the same chain of index and path reads.
template <int HPW>
__global__ __launch_bounds__(256) void gdn_append_path_kernel(GdnArgs a) {
  const int tile = tile_index();
  const int hb = a.H / HPW;   // workgroups per sequence
  const int b = tile / hb, h0 = (tile - b * hb) * HPW;
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
    const long unit0 = (long)b * a.H + h0;
    const long sk = (long)a.batch * a.H * DK, sv = (long)a.batch * a.H * DV, sd = (long)a.batch * a.H;
    constexpr int KV = DK / 4, VV = DV / 4;   // float4 chunks of k and v
    for (int e = threadIdx.x; e < pl * HPW * (KV + VV); e += 256) {
      const int k = e / (HPW * (KV + VV)), r = e - k * (HPW * (KV + VV));
      const int hh = r / (KV + VV), c = r - hh * (KV + VV);
      const long unit = unit0 + hh;
      const int j = a.path[(long)b * a.depth + k];
      const int sl = ring_slot(slot0, len + k, cap);
      if (c < KV)
        st4(a.ring_k + (unit * cap + sl) * DK + 4 * c, ld4(a.k + j * sk + unit * DK + 4 * c));
      else
        st4(a.ring_v + (unit * cap + sl) * DV + 4 * (c - KV),
            ld4(a.v + j * sv + unit * DV + 4 * (c - KV)));
    }
    if (threadIdx.x < pl * HPW) {
      const int k = threadIdx.x / HPW, hh = threadIdx.x - k * HPW;
      const long unit = unit0 + hh;
      const int j = a.path[(long)b * a.depth + k];
      const int sl = ring_slot(slot0, len + k, cap);
      a.ring_a[unit * cap + sl] = a.alpha[j * sd + unit];
      a.ring_b[unit * cap + sl] = a.beta[j * sd + unit];
    }
  }
  IndexUpdate u;
  u.apply = ok;
  u.pos_add = 0;
  u.new_len = len + pl;
  finish_update(a.arrive, a.pos, a.len, b, hb, arrived, u);
  if (!ok && last_arrival(arrived, hb))
    raise_status(a.status, valid ? kStatusOverflow : kStatusIndex);
}

}  // namespace

static dim3 half_grid(const GdnArgs& a) {
  return dim3((unsigned)(a.batch * a.H * (DV / kStepRows)));
}
static dim3 whole_grid(const GdnArgs& a) { return dim3((unsigned)(a.batch * a.H)); }

hipError_t launch_gdn_step(const GdnArgs& a, bool fused, hipStream_t s) {
  const dim3 block(kStepThreads);
  if (a.scheme == kSchemeF32) {
    if (fused)
      hipLaunchKernelGGL((gdn_step_kernel<4, true>), half_grid(a), block, 0, s, a);
    else
      hipLaunchKernelGGL((gdn_step_kernel<4, false>), half_grid(a), block, 0, s, a);
  } else if (fused) {   // DUAL (checked by the caller): fold fp32, re-quantise the copy
    if (a.lp == kLpBf16)
      hipLaunchKernelGGL((gdn_step_kernel<4, true, kLpBf16>), whole_grid(a), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((gdn_step_kernel<4, true, kLpE4m3>), whole_grid(a), dim3(512), 0, s, a);
  } else if (a.lp == kLpBf16) {
    hipLaunchKernelGGL((gdn_step_kernel<2, false>), whole_grid(a), block, 0, s, a);
  } else {
    hipLaunchKernelGGL((gdn_step_kernel<1, false>), whole_grid(a), dim3(step_threads<1>()), 0,
                       s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gdn_commit(const GdnArgs& a, hipStream_t s) {
  if (a.scheme == kSchemeF32)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeF32, 0, kStepThreads>), half_grid(a),
                       dim3(kStepThreads), 0, s, a);
  else if (a.scheme == kSchemeDual && a.lp == kLpBf16)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeDual, kLpBf16, 512>), whole_grid(a), dim3(512),
                       0, s, a);
  else if (a.scheme == kSchemeDual)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeDual, kLpE4m3, 512>), whole_grid(a), dim3(512),
                       0, s, a);
  else if (a.lp == kLpBf16)
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeShared, kLpBf16, 512>), whole_grid(a),
                       dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((gdn_commit_kernel<kSchemeShared, kLpE4m3, 512>), whole_grid(a),
                       dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int EB, bool COMMIT = false>
static void launch_gdn_verify_eb(const GdnArgs& a, hipStream_t s) {
  const dim3 grid = whole_grid(a), block(512);
  if (a.n_pos <= 1)
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 1, COMMIT>), grid, block, 0, s, a);
  else if (a.n_pos <= 2)
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 2, COMMIT>), grid, block, 0, s, a);
  else if (a.n_pos <= 4)
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 4, COMMIT>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gdn_verify_kernel<EB, 8, COMMIT>), grid, block, 0, s, a);
}

hipError_t launch_gdn_verify(const GdnArgs& a, hipStream_t s) {
  if (a.min_len > 0)   // fused commit (fp32 checkpoint; checked by the caller)
    launch_gdn_verify_eb<4, true>(a, s);
  else if (a.scheme == kSchemeF32)
    launch_gdn_verify_eb<4>(a, s);
  else if (a.lp == kLpBf16)
    launch_gdn_verify_eb<2>(a, s);
  else
    launch_gdn_verify_eb<1>(a, s);
  return hipGetLastError();
}

hipError_t launch_gdn_append_path(const GdnArgs& a, hipStream_t s) {
  if (a.H % 4 == 0)   // four heads per workgroup
    hipLaunchKernelGGL(gdn_append_path_kernel<4>, dim3((unsigned)(a.batch * (a.H / 4))), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gdn_append_path_kernel<1>, whole_grid(a), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gdn_eager(const GdnArgs& a, hipStream_t s) {
  if (a.scheme != kSchemeShared)
    hipLaunchKernelGGL((gdn_eager_kernel<0>), half_grid(a), dim3(kStepThreads), 0, s, a);
  else if (a.lp == kLpBf16)
    hipLaunchKernelGGL((gdn_eager_kernel<kLpBf16>), whole_grid(a), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((gdn_eager_kernel<kLpE4m3>), whole_grid(a), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace rssm
