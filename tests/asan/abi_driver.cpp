// Host-side driver for the AddressSanitizer build of the library: drives
// every entry point of include/attn.h through its argument validation,
// empty-problem, kernel-name and status-string paths.  Pointers are aligned
// fake addresses (validation only compares them, it never dereferences
// them).  Valid arguments end in ATTN_ERR_DEVICE because there is no GPU:
// the driver refuses to run when one is visible, since there those calls
// would launch kernels on the fake addresses.  Prints one "call" line per
// entry-point call and "done <calls>" at the end.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include <hip/hip_runtime_api.h>

#include "attn.h"

namespace {

// Distinct, 256-byte aligned, widely spaced fake device addresses.
void* fake(int i) { return reinterpret_cast<void*>(uintptr_t(1) << 40 | uintptr_t(i) << 32); }
float* fakef(int i) { return static_cast<float*>(fake(i)); }

int calls = 0;
void show(const char* what, attn_status s) {
  ++calls;
  std::printf("call %-36s %d %s\n", what, int(s), attn_status_string(s));
}

}  // namespace

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::printf("gpu present: not run\n");
    return 0;
  }
  const float nan = std::nanf("");
  const float scale = 0.125f;
  void *q = fake(1), *k = fake(2), *v = fake(3), *o = fake(4);
  float* lse = fakef(5);
  void *dq = fake(6), *dk = fake(7), *dv = fake(8), *dout = fake(9);
  float* ws = fakef(10);

  // forward: bad sizes, head dimension, flag, scale, pointers, alignment,
  // overlap, empty problems, valid arguments
  const int64_t shapes[][4] = {{-1, 1, 8, 64}, {1, -1, 8, 64}, {1, 1, -8, 64}, {1, 1, 8, 96},
                               {1, 1, 8, 0},   {0, 1, 8, 64},  {1, 0, 8, 64},  {1, 1, 0, 64},
                               {1, 1, 8, 64},  {1, 1, 8, 128}, {int64_t(1) << 40, 1, 8, 64},
                               {1, 1, int64_t(1) << 40, 128}};
  for (const auto& s : shapes) {
    for (int causal : {0, 1, 2}) {
      show("attn_fwd", attn_fwd(q, k, v, o, lse, s[0], s[1], s[2], s[3], causal, scale, nullptr));
      show("attn_fwd_f32", attn_fwd_f32(fakef(1), fakef(2), fakef(3), fakef(4), lse, s[0], s[1],
                                        s[2], s[3], causal, scale, nullptr));
      show("attn_fwd_gqa", attn_fwd_gqa(q, k, v, o, lse, s[0], s[1] * 2, s[1], s[2], s[3], causal,
                                        scale, nullptr));
      show("attn_bwd", attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, s[0], s[1], s[2], s[3],
                                causal, scale, nullptr));
      show("attn_bwd_gqa", attn_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, ws, s[0], s[1] * 2,
                                        s[1], s[2], s[3], causal, scale, nullptr));
      show("attn_fwd_materialized",
           attn_fwd_materialized(q, k, v, o, lse, fakef(11), fake(12), s[0], s[1], s[2], s[3],
                                 causal, scale, nullptr));
      show("attn_decode", attn_decode(q, k, v, o, lse, ws, int64_t(1) << 30, s[0], s[1] * 4,
                                      s[1], 1, s[2], s[2] + 16, s[3], causal, scale, nullptr));
    }
  }
  show("fwd nan scale", attn_fwd(q, k, v, o, lse, 1, 1, 8, 64, 1, nan, nullptr));
  show("fwd inf scale", attn_fwd(q, k, v, o, lse, 1, 1, 8, 64, 1, INFINITY, nullptr));
  show("fwd null q", attn_fwd(nullptr, k, v, o, lse, 1, 1, 8, 64, 1, scale, nullptr));
  show("fwd null lse", attn_fwd(q, k, v, o, nullptr, 1, 1, 8, 64, 1, scale, nullptr));
  show("fwd misaligned o", attn_fwd(q, k, v, static_cast<char*>(o) + 2, lse, 1, 1, 8, 64, 1,
                                    scale, nullptr));
  show("fwd o overlaps q", attn_fwd(q, k, v, q, lse, 1, 1, 8, 64, 1, scale, nullptr));
  show("gqa bad groups", attn_fwd_gqa(q, k, v, o, lse, 1, 6, 4, 8, 64, 1, scale, nullptr));
  show("bwd null ws", attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 1, 1, 8, 64, 1, scale,
                               nullptr));
  show("decode small ws", attn_decode(q, k, v, o, lse, ws, 16, 1, 32, 8, 1, 1 << 17, 1 << 17, 128,
                                      1, scale, nullptr));
  show("decode Tk < Tq causal", attn_decode(q, k, v, o, lse, ws, 1 << 20, 1, 8, 8, 16, 8, 8, 64,
                                            1, scale, nullptr));
  show("decode too many rows", attn_decode(q, k, v, o, lse, ws, 1 << 20, 1, 64, 1, 8, 64, 64, 64,
                                           1, scale, nullptr));

  // size queries and names
  for (int64_t tk : {int64_t(0), int64_t(1), int64_t(4096), int64_t(131072)}) {
    std::printf("decode_splits %lld ws %lld\n",
                (long long)attn_decode_splits(1, 32, 8, 1, tk),
                (long long)attn_decode_workspace_bytes(1, 32, 8, 1, tk, 128));
  }
  for (int is_f32 : {0, 1, 2})
    for (int64_t d : {int64_t(32), int64_t(64), int64_t(128)})
      for (int causal : {0, 1, 3}) {
        const char* a = attn_kernel_name(is_f32, d, causal);
        const char* b = attn_fwd_kernel_name_for(1, 8, 2048, d, causal);
        const char* c = attn_fwd_f32_kernel_name_for(1, 1, 256, d, causal);
        const char* e = attn_bwd_kernel_name(d, causal, is_f32);
        std::printf("names %s %s %s %s\n", a ? a : "-", b ? b : "-", c ? c : "-", e ? e : "-");
      }
  for (int s = -1; s <= 12; ++s) std::printf("status %d %s\n", s, attn_status_string(attn_status(s)));
  std::printf("done %d calls\n", calls);
  return 0;
}
