// Drives librssm's host-side validation (every call here is rejected, or has
// batch 0, before anything is launched) in a build whose host code carries
// address and undefined-behaviour sanitizers (tests/test_sanitize_host.py).
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "rssm.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAILED: %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  const uintptr_t fake = 0x10000;   // aligned stand-in address, never dereferenced
  auto P = [&](uintptr_t off = 0) { return reinterpret_cast<float*>(fake + off); };
  rssm_layer m2;
  std::memset(&m2, 0, sizeof m2);
  m2.kind = RSSM_MAMBA2;
  m2.scheme = RSSM_F32;
  m2.batch = 4;
  m2.nheads = 8;
  m2.ngroups = 2;
  m2.dim_v = 64;
  m2.dim_k = 128;
  m2.capacity = 8;
  m2.ckpt = P();
  m2.A = P();
  m2.D = P();
  for (int i = 0; i < 3; ++i) m2.ring[i] = P();
  m2.ckpt_pos = reinterpret_cast<int64_t*>(fake);
  m2.len = reinterpret_cast<int32_t*>(fake);
  m2.arrive = reinterpret_cast<uint32_t*>(fake);
  m2.status = reinterpret_cast<uint32_t*>(fake);

  expect(rssm_abi_version(), RSSM_ABI_VERSION, "abi version");
  for (int c = 0; c >= -6; --c) (void)std::strlen(rssm_strerror(c));
  expect(rssm_mamba2_step(nullptr, P(), P(), P(), P(), P(), 0, nullptr), RSSM_EINVAL, "null layer");
  expect(rssm_mamba2_step(&m2, nullptr, P(), P(), P(), P(), 0, nullptr), RSSM_EINVAL, "null x");
  expect(rssm_mamba2_step(&m2, P(), P(), P(8), P(), P(), 0, nullptr), RSSM_EALIGN, "misaligned C");
  rssm_layer bad = m2;
  bad.capacity = 33;
  expect(rssm_mamba2_step(&bad, P(), P(), P(), P(), P(), 0, nullptr), RSSM_EUNSUPPORTED, "capacity");
  bad = m2;
  bad.ngroups = 3;
  expect(rssm_commit(&bad, nullptr, 0, nullptr), RSSM_EINVAL, "groups");
  expect(rssm_commit(&m2, nullptr, -1, nullptr), RSSM_ERANGE, "min_len");
  rssm_inputs in;
  std::memset(&in, 0, sizeof in);
  in.x = P(); in.B = P(); in.C = P(); in.dt = P();
  expect(rssm_verify(&m2, 0, &in, P(), nullptr), RSSM_ERANGE, "verify 0");
  expect(rssm_verify(&m2, 9, &in, P(), nullptr), RSSM_ERANGE, "verify 9");
  const int32_t parent_bad[2] = {-1, 1};
  expect(rssm_verify_tree(&m2, 2, parent_bad, &in, P(), nullptr), RSSM_EINVAL, "tree parent");
  expect(rssm_append_path(&m2, 4, nullptr, nullptr, 5, &in, nullptr), RSSM_ERANGE, "path depth");
  expect(rssm_prefill(&m2, 0, &in, P(), nullptr, nullptr), RSSM_ERANGE, "prefill 0");
  in.C = nullptr;
  expect(rssm_prefill(&m2, 3, &in, P(), nullptr, nullptr), RSSM_EINVAL, "prefill C");
  expect(rssm_rollback(&m2, nullptr, nullptr), RSSM_EINVAL, "rollback null");
  in.C = P();
  expect(rssm_eager_spec_round(&m2, 0, &in, P(), P(), nullptr, nullptr), RSSM_ERANGE, "spec 0");
  expect(rssm_eager_spec_round(&m2, 4, &in, P(), nullptr, nullptr, nullptr), RSSM_EINVAL,
         "spec slots");
  bad = m2;
  bad.scheme = RSSM_DUAL;
  bad.lp_dtype = RSSM_BF16;
  expect(rssm_eager_spec_round(&bad, 4, &in, P(), P(), nullptr, nullptr), RSSM_EUNSUPPORTED,
         "spec scheme");
  expect(rssm_eager_spec_accept(&m2, 9, nullptr, nullptr, nullptr), RSSM_ERANGE, "accept 9");
  expect(rssm_eager_spec_accept(&m2, 4, nullptr, nullptr, nullptr), RSSM_EINVAL, "accept null");
  in.C = nullptr;
  expect(rssm_status(nullptr, nullptr, nullptr), RSSM_EINVAL, "status null");
  rssm_layer empty = m2;
  empty.batch = 0;
  empty.ckpt = nullptr;
  expect(rssm_commit(&empty, nullptr, 0, nullptr), RSSM_OK, "batch 0");
  expect(rssm_prefill(&empty, 3, &in, nullptr, nullptr, nullptr), RSSM_OK, "prefill batch 0");
  if (failures) return 1;
  std::printf("ABI host code under sanitizers: ok\n");
  return 0;
}
