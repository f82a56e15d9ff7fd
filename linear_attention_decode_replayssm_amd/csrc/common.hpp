// common.hpp -- device helpers shared by the gfx950 kernels of librssm.
//
// Wave64 cross-lane reductions, 16-byte streaming loads/stores, the
// workgroup -> tile mapping across the MI355X's 8 XCDs, and the per-sequence
// "last workgroup updates the indices" protocol.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxCap = 16;   // ring slots per sequence
constexpr int kMaxCapM2 = 32; // Mamba-2 fp32 step and commit: rings of up to 32 slots
constexpr int kMaxPos = 8;    // draft positions per verify call
// Arrival counters sit one 128-byte line apart: every workgroup of a launch
// performs one atomic on its sequence's counter, and atomics to one line are
// serialised, so packed counters (32 sequences per line) cost ~3% of a step.
constexpr int kArriveStride = 32;

constexpr uint32_t kStatusOverflow = 1u;
constexpr uint32_t kStatusRollback = 2u;
constexpr uint32_t kStatusNonfinite = 4u;
constexpr uint32_t kStatusIndex = 8u;

// A sequence's indices can be used when 0 <= len <= cap and ckpt_pos >= 0.
// Anything else (indices the library never wrote) is refused: the sequence is
// left as it is, its outputs are NaN and kStatusIndex is raised, so that no
// ring slot outside the sequence's own is ever addressed.
__device__ __forceinline__ bool indices_valid(int32_t len, int64_t pos, int cap) {
  return len >= 0 && len <= cap && pos >= 0;
}

// The buffer length a verify works from when the previous round's rollback
// is passed with it (n_reject, may be NULL): len - n_reject[b], as a rollback
// launch would leave it.  A count outside 0..len is refused as the rollback
// refuses it (bad: the length stays, the caller raises the rollback bit);
// indices that are not valid are left to the verify's own check.
struct RolledLen {
  int32_t len;
  bool valid, rolled, bad;
};

__device__ __forceinline__ RolledLen rolled_len(int32_t len, int64_t pos, int cap,
                                                const int32_t* n_reject, int b) {
  RolledLen r{len, indices_valid(len, pos, cap), false, false};
  if (n_reject != nullptr && r.valid) {
    const int32_t nr = n_reject[b];
    if (nr < 0 || nr > len) {
      r.bad = true;
    } else {
      r.len = len - nr;
      r.rolled = true;
    }
  }
  return r;
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// ---- memory ---------------------------------------------------------------
// The checkpoint is streamed once per step and not reused by this kernel:
// nontemporal loads keep it from evicting the ring entries and inputs that
// the other heads of the same sequence re-read from L2.
__device__ __forceinline__ f32x4 ld_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ u32x4 ld_nt_u(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_nt(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st_nt_u(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ f32x4 ld4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void st4(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// ---- workgroup -> tile ----------------------------------------------------
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  Remap so that every XCD receives one contiguous range of
// tiles: the heads of one sequence (and the heads of one Mamba-2 group, which
// share B and C) then land on the same XCD and share its L2.
__device__ __forceinline__ int tile_index() {
  const int id = blockIdx.x, n = gridDim.x;
  if ((n & 7) == 0) return (id & 7) * (n >> 3) + (id >> 3);
  return id;
}

// As tile_index, for a grid of whole sequences of tps tiles each: every XCD
// receives tps / 8 consecutive tiles of every sequence instead of whole
// sequences, so that work that differs from sequence to sequence (the fold
// of a due buffer) is spread evenly over the XCDs.  At batch 256 it made the
// standalone fp32 commits 9-13% faster, the chain verifies that fold due
// buffers 3-6%, the fused Mamba-2 step 3% and the fp32 eager
// read-modify-write kernels 4-8%; the plain replay step, the tree verifies
// of 8 drafts and the fused fp32 GDN step stayed with whole sequences, which
// measured as fast or faster for them.
// Built with -DRSSM_XCD_WHOLE every kernel takes whole sequences per XCD: the
// comparison build for the per-kernel choice.
#ifdef RSSM_XCD_WHOLE
constexpr bool kXcdSplit = false;
#else
constexpr bool kXcdSplit = true;
#endif

__device__ __forceinline__ int tile_index_split(int tps) {
  const int id = blockIdx.x, n = gridDim.x;
  if (!kXcdSplit || (n & 7) != 0 || (tps & 7) != 0) return tile_index();
  const int per = tps >> 3, li = id >> 3;
  const int b = li / per;
  return b * tps + (id & 7) * per + (li - b * per);
}

// ---- reduction partners ----------------------------------------------------
// Value of a partner lane for reductions over lane bit M.  The partner has the
// opposite bit M and the same higher bits; its lower bits may differ.  That is
// all a reduction needs that processes lane bits from high to low (each lane
// ends with the complete sum, and in the transposed reduction below with the
// same index assignment as an exact xor partner).  So DPP row permutations
// serve for M <= 8 (quad_perm for 1 and 2, row_half_mirror i <-> 7-i for 4,
// row_mirror i <-> 15-i for 8), ds_swizzle xor-16 for 16 and ds_bpermute only
// for 32.  The sums below take bits 4 and 5 with the lane swaps instead
// (swap_add); these two forms remain for the wave-wide max and xor folds.
// The DPP forms zero-fill (bound_ctrl) with an old value of 0: every lane of
// these permutations has a source, so the value is the same, and the compiler
// can then fold the move into the add that consumes it (v_add_f32_dpp).
template <int M>
__device__ __forceinline__ float rpartner(float v) {
  const int x = __float_as_int(v);
  int r;
  if constexpr (M == 1)
    r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true);
  else if constexpr (M == 2)
    r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true);
  else if constexpr (M == 4)
    r = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true);
  else if constexpr (M == 8)
    r = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, true);
  else if constexpr (M == 16)
    r = __builtin_amdgcn_ds_swizzle(x, 0x401F);
  else
    r = __shfl_xor(x, M);
  return __int_as_float(r);
}

// Exchange across lane bit M = 16 or 32 with the gfx950 lane swaps
// (v_permlane16_swap / v_permlane32_swap, checked on the GPU with an in-bounds
// probe): afterwards a lane with bit M clear holds (its own a, its partner's
// a) and a lane with bit M set holds (its partner's b, its own b).  So a + b is
// a + partner's a on the lower lanes and b + partner's b on the upper ones --
// one step of the transposed reduction below, in two VALU instructions and
// without the LDS round trip of ds_swizzle / ds_bpermute or the selects of
// the DPP form.  With a == b it is a butterfly step.  The whole wave must be
// active (every call site is wave-uniform).
template <int M>
__device__ __forceinline__ float swap_add(float a, float b) {
  static_assert(M == 16 || M == 32, "lane swaps exist for bits 4 and 5");
  uint32_t x, y;
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    x = r[0];
    y = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    x = r[0];
    y = r[1];
  }
  return __uint_as_float(x) + __uint_as_float(y);
}

// Exclusive suffix sum within each 16-lane row: lane i receives the sum of
// v over lanes i+1..15 of its row.  DPP row_shl:k hands lane i the value of
// lane i+k of the same row, and 0 past the row's end (bound_ctrl; both
// checked on the GPU with an in-bounds probe).  Every lane of a row must be
// active.
template <int K>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + K, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_suffix_excl(float v) {
  float s = row_shl<1>(v);
  s += row_shl<1>(s);
  s += row_shl<2>(s);
  s += row_shl<4>(s);
  s += row_shl<8>(s);
  return s;
}

// Sum over the LPR lanes of a lane group (every lane receives the sum).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 64) v = swap_add<32>(v, v);
  if constexpr (LPR >= 32) v = swap_add<16>(v, v);
  if constexpr (LPR >= 16) v += rpartner<8>(v);
  if constexpr (LPR >= 8) v += rpartner<4>(v);
  if constexpr (LPR >= 4) v += rpartner<2>(v);
  if constexpr (LPR >= 2) v += rpartner<1>(v);
  return v;
}

// ---- transposed cross-lane reduction --------------------------------------
// Each lane holds C partial sums; the LPR lanes that differ only in lane bits
// below log2(LPR) share a row.  Going from the highest of those bits down, a
// lane keeps the half of its values that its bit selects and adds the
// partner's copy of that half, so V values cost V-1 exchanges instead of
// V*log2(LPR).  Once one value is left, the remaining bits are plain
// butterflies.
template <int C, int M>
struct XRed {
  static __device__ __forceinline__ void run(float* v, int lane) {
    if constexpr (M == 0) {
      return;
    } else if constexpr (C > 1) {
      if constexpr (M >= 16) {
#pragma unroll
        for (int j = 0; j < C / 2; ++j) v[j] = swap_add<M>(v[j], v[j + C / 2]);
      } else {
        const bool up = (lane & M) != 0;
#pragma unroll
        for (int j = 0; j < C / 2; ++j) {
          const float send = up ? v[j] : v[j + C / 2];
          const float keep = up ? v[j + C / 2] : v[j];
          v[j] = keep + rpartner<M>(send);
        }
      }
      XRed<C / 2, M / 2>::run(v, lane);
    } else {
      if constexpr (M >= 16)
        v[0] = swap_add<M>(v[0], v[0]);
      else
        v[0] += rpartner<M>(v[0]);
      XRed<1, M / 2>::run(v, lane);
    }
  }
};

// Index bookkeeping for XRed<V, LPR/2>: after the reduction a lane holds
// VOUT complete sums; value j of lane `lane` is the sum of original index
// index(lane, j).  Lanes that differ only in the low BFLY bits hold equal
// results; writer() picks one of them.
template <int V, int LPR>
struct XMap {
  static_assert(V > 0 && (V & (V - 1)) == 0 && LPR > 0 && (LPR & (LPR - 1)) == 0,
                "the transposed reduction halves the values and the lanes: powers of two");
  static constexpr int kLogL = ilog2(LPR);
  static constexpr int kLogV = ilog2(V);
  static constexpr int VOUT = V > LPR ? V / LPR : 1;
  static constexpr int BFLY = kLogL > kLogV ? kLogL - kLogV : 0;
  static __device__ __forceinline__ int index(int lane, int j) {
    int idx = j, c = V;
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) {
      if (c > 1) {
        if (lane & m) idx += c / 2;
        c /= 2;
      }
    }
    return idx;
  }
  static __device__ __forceinline__ bool writer(int lane) {
    return (lane & ((1 << BFLY) - 1)) == 0;
  }
};

template <int V, int LPR>
__device__ __forceinline__ void xreduce(float (&v)[V], int lane) {
  static_assert(V > 0 && (V & (V - 1)) == 0 && LPR > 0 && (LPR & (LPR - 1)) == 0,
                "the transposed reduction halves the values and the lanes: powers of two");
  XRed<V, LPR / 2>::run(v, lane);
}

// Full butterfly: every lane of each LPR-lane group ends with all V sums.
template <int V, int LPR>
__device__ __forceinline__ void allreduce(float (&v)[V]) {
#pragma unroll
  for (int j = 0; j < V; ++j) v[j] = group_sum<LPR>(v[j]);
}

// ---- per-sequence index update --------------------------------------------
// Every workgroup of sequence b reads len[b] / ckpt_pos[b] at its start.  The
// workgroup that completes the per-sequence count in arrive[b] knows that all
// `nwg` workgroups of the sequence have read the indices; it resets the
// counter and applies the update.  Nothing in the launch reads the indices
// afterwards and the next launch sees them through the kernel boundary, so
// the counter needs no fence: a relaxed device-scope atomic.  (A device-scope
// fence would write back and invalidate the XCD's L2 once per workgroup.)
struct IndexUpdate {
  int64_t pos_add;
  int32_t new_len;
  bool apply;
};

// Each wave reads the indices with its own scalar load.  Once this returns,
// every wave of the workgroup has received them: each wave's leader stores a
// value computed from them to LDS before the barrier, which cannot happen
// before its loads have returned.  (The barrier does not wait for the
// workgroup's outstanding vector loads.)
__device__ __forceinline__ void indices_consumed(int32_t len, int64_t pos) {
  __shared__ int32_t seen[16];
  if ((threadIdx.x & 63) == 0) seen[threadIdx.x >> 6] = len ^ (int32_t)pos;
  __syncthreads();
}

// Early variant: count the workgroup right after its index reads, so that the
// atomic's round trip overlaps the state stream instead of ending the
// workgroup.  The increment is always 1, so the count of a sequence always
// reaches nwg and its counter returns to zero, whatever the indices hold.  It
// passes through an empty asm statement that takes the index values as
// inputs: the compiler must wait for their loads before it and cannot tell
// that the increment is unchanged, so the atomic is not issued before those
// reads have returned.  Once the count is complete every workgroup of the
// sequence holds its copy of the indices and the last one may update them at
// any time.  Returns the pre-increment count (thread 0).
// Pre-increment count returned for a layer whose indices are read-only: no
// counter is touched, no workgroup updates the indices, and per-sequence
// errors are reported by every workgroup of the sequence.
constexpr uint32_t kNoArrival = 0xffffffffu;

__device__ __forceinline__ uint32_t arrive_early(uint32_t* arrive, int b, int32_t len,
                                                 int64_t pos, bool ro = false) {
  if (ro) return kNoArrival;
  uint32_t old = 0u;
  if (threadIdx.x == 0) {
    uint32_t inc = 1u;
    asm volatile("" : "+v"(inc) : "v"(len), "v"((uint32_t)pos), "v"((uint32_t)(pos >> 32)));
    old = __hip_atomic_fetch_add(&arrive[(long)b * kArriveStride], inc, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  }
  return old;
}

// Completes arrive_early: the workgroup that completed the count resets it and
// applies the update.  Thread 0 only; no barrier needed.
__device__ __forceinline__ void finish_update(uint32_t* arrive, int64_t* pos, int32_t* len,
                                              int b, int nwg, uint32_t old, IndexUpdate u) {
  if (threadIdx.x == 0 && old == (uint32_t)(nwg - 1)) {
    __hip_atomic_store(&arrive[(long)b * kArriveStride], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (u.apply) {
      pos[b] += u.pos_add;
      len[b] = u.new_len;
    }
  }
}

// Thread 0 of the workgroup that completed its sequence's arrival count: the
// one workgroup per sequence that reports a per-sequence error, so that a
// failing batch costs one status atomic per sequence, not one per workgroup.
__device__ __forceinline__ bool last_arrival(uint32_t old, int nwg) {
  return threadIdx.x == 0 && (old == (uint32_t)(nwg - 1) || old == kNoArrival);
}

__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bits) {
  atomicOr(status, bits);
}

__device__ __forceinline__ int ring_slot(int slot0, int i, int cap) {
  int s = slot0 + i;
  return s >= cap ? s - cap : s;
}

}  // namespace rssm
