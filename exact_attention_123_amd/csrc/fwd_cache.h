// The bf16 forward kernel over a key/value cache, for the decode entry point
// when the new queries are many (a prefill in chunks): Tq new queries per
// query head are the last Tq positions of a cache of Tk keys (rows
// 0 .. Tk - 1 of each key/value head, stored with a stride of Tk_cap rows),
// under the causal mask query i sees keys j <= Tk - Tq + i.  Arguments as
// for attn_decode (already validated by it); enqueues one kernel, no
// workspace.
#ifndef ATTN_FWD_CACHE_H_
#define ATTN_FWD_CACHE_H_

#include <cstdint>

#include "attn.h"

namespace attn_internal {

// Whether the forward kernel's grid for B H query heads of Tq rows, in
// 128-row workgroups, has at least one workgroup per CU of the current
// device.
bool fwd_fills_device(int64_t B, int64_t H, int64_t Tq);

attn_status fwd_over_cache(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                           int64_t Tk_cap, int64_t d, int causal, float scale,
                           hipStream_t stream);

// Name of the forward instance fwd_over_cache launches for B H query heads
// of Tq new rows (NULL when the current device is not a gfx950).
const char* fwd_over_cache_kernel_name(int64_t B, int64_t H, int64_t Tq, int64_t d, int causal);

}  // namespace attn_internal

#endif  // ATTN_FWD_CACHE_H_
