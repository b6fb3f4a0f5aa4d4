// Host-side helpers shared by the library's source files (internal; not
// part of the C ABI, hidden from the library's exported symbols).
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>

namespace fa {

#define FA_INTERNAL __attribute__((visibility("hidden")))

// [a, a + na) and [b, b + nb) overlap (empty ranges never do).
FA_INTERNAL bool host_overlaps(const void* a, size_t na, const void* b, size_t nb);

// The argument checks of fa_fwd / fa_fwd_f32 (elem_bytes 2 or 4) and of
// fa_fwd_ex: the status those entry points return before any launch.
FA_INTERNAL int host_check(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                           int H, int N, int d, float scale, int elem_bytes);
FA_INTERNAL int host_check_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                              int Hq, int Hkv, int T, int S, int d, float scale, int causal, int offset,
                              int window);

// The fa_fwd_ex kernels in split-KV form: a work unit per (256-row query
// tile, key chunk of `chunk` keys), fp32 partials (O_g, L_g) into
// ws_o [G, B, Hq, T, d] and ws_lse [G, B, Hq, T]; arguments already checked,
// G = nsplit >= 2.  c = |scale| * log2(e), qsign the sign flip of Q.
FA_INTERNAL void host_launch_ex_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                      int Hq, int Hkv, int T, int S, int d, int causal, int offset, int window,
                                      float c, unsigned qsign, int nsplit, int chunk, float* ws_o, float* ws_lse,
                                      hipStream_t stream);

}  // namespace fa
