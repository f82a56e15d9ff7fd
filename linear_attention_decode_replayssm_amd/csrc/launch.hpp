// launch.hpp -- internal interface between the C ABI (api.cpp) and the
// kernel translation units.  Not installed; the public ABI is include/rssm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

// Mamba-2 replay/eager/commit/verify arguments.  Pointers as in rssm.h.
struct M2Args {
  float* ckpt;          // [b][H][P][N] fp32 (NULL under SHARED)
  void* ckpt_lp;        // [b][H][P][N] bf16 / E4M3 codes (NULL under F32)
  float* lp_scale;      // [b][H] (E4M3)
  const float* A;       // [H]
  const float* D;       // [H]
  float* ring_x;        // [b][H][cap][P]
  float* ring_B;        // [b][G][cap][N]
  float* ring_dt;       // [b][H][cap]
  int64_t* pos;
  int32_t* len;
  uint32_t* arrive;
  uint32_t* status;
  const float* x;       // [n][b][H][P]
  const float* B;       // [n][b][G][N]
  const float* C;       // [n][b][G][N]
  const float* dt;      // [n][b][H]
  float* y;             // [n][b][H][P]
  const uint8_t* mask;  // commit, prefill
  int batch, H, G, cap, n_pos, min_len;
  int scheme, lp;       // rssm_scheme / rssm_lp values
  // verify: anc[j] has bit m set when draft m lies on the path to draft j
  // (j included); append != 0 appends the drafts (linear chains only)
  uint32_t anc[8];
  int append;
  const int32_t* path;      // append_path: [b][depth] draft indices
  const int32_t* path_len;  // append_path: [b]
  int depth;
  int idx_ro;               // indices read, never written (RSSM_LAYER_INDEX_READONLY)
  const int32_t* n_reject;  // verify: [b] rejections rolled back first (NULL: none)
};

// Gated DeltaNet arguments.
struct GdnArgs {
  float* ckpt;          // fp32 [b][H][dv][dk] (NULL under SHARED)
  void* ckpt_lp;        // bf16 / e4m3 codes (NULL under F32)
  float* lp_scale;      // [b][H] (E4M3)
  float* ring_k;        // [b][H][cap][dk]
  float* ring_v;        // [b][H][cap][dv]
  float* ring_a;        // [b][H][cap]
  float* ring_b;        // [b][H][cap]
  int64_t* pos;
  int32_t* len;
  uint32_t* arrive;
  uint32_t* status;
  const float* q;       // [n][b][H][dk]
  const float* k;       // [n][b][H][dk]
  const float* v;       // [n][b][H][dv]
  const float* alpha;   // [n][b][H]
  const float* beta;    // [n][b][H]
  float* o;             // [n][b][H][dv]
  const uint8_t* mask;  // commit, prefill
  int batch, H, cap, n_pos, min_len;
  int scheme, lp;       // rssm_scheme / rssm_lp values
  uint32_t anc[8];      // as in M2Args
  int append;
  const int32_t* path;
  const int32_t* path_len;
  int depth;
  int idx_ro;           // as in M2Args
  const int32_t* n_reject;  // as in M2Args
};

hipError_t launch_m2_step(const M2Args& a, bool fused, hipStream_t s);
hipError_t launch_m2_commit(const M2Args& a, hipStream_t s);
hipError_t launch_m2_verify(const M2Args& a, hipStream_t s);
hipError_t launch_m2_eager(const M2Args& a, hipStream_t s);

hipError_t launch_gdn_step(const GdnArgs& a, bool fused, hipStream_t s);
hipError_t launch_gdn_commit(const GdnArgs& a, hipStream_t s);
hipError_t launch_gdn_verify(const GdnArgs& a, hipStream_t s);
hipError_t launch_gdn_eager(const GdnArgs& a, hipStream_t s);

hipError_t launch_m2_append_path(const M2Args& a, hipStream_t s);
hipError_t launch_m2_prefill(const M2Args& a, hipStream_t s);   // n_pos = prompt tokens
hipError_t launch_gdn_append_path(const GdnArgs& a, hipStream_t s);
hipError_t launch_gdn_prefill(const GdnArgs& a, hipStream_t s);  // n_pos = prompt tokens

// eager speculative comparator: n_pos drafts, state slots [n_pos + 1][...]
hipError_t launch_m2_eager_spec(const M2Args& a, float* slots, const int32_t* cur, hipStream_t s);
hipError_t launch_gdn_eager_spec(const GdnArgs& a, float* slots, const int32_t* cur,
                                 hipStream_t s);
hipError_t launch_eager_spec_accept(int32_t* cur, uint32_t* status, const int32_t* n_accept,
                                    int n, int batch, hipStream_t s);

// streaming probe: tiles x tile_bytes (32768 or 4096) read (dst == NULL: one
// float per wave to sink, every wave when check != 0) or copied to dst
hipError_t launch_probe(const void* src, void* dst, float* sink, long tiles, int tile_bytes,
                        int check, hipStream_t s);

hipError_t launch_rollback(int64_t* pos, int32_t* len, uint32_t* status,
                           const int32_t* n_reject, int batch, int cap, hipStream_t s);
hipError_t launch_clear_status(uint32_t* status, hipStream_t s);

}  // namespace rssm
