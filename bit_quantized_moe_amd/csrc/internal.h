// Declarations shared between the library's translation units (not part of the ABI).
#pragma once

#include "common.h"

namespace bqm {

// Stable counting sort of R routed pairs by expert (route.hip).  counts_ws needs
// permute_ws_bytes(R, E).  If tile_off != NULL it also receives the prefix sum of
// ceil(count_e / bm) over experts ([E+1] entries).
size_t permute_ws_bytes(int64_t R, int E);
bqm_status permute_launch(const int32_t *topk_idx, int64_t R, int E, int32_t *perm, int32_t *inv,
                          int32_t *offsets, int32_t *counts_ws, int bm, int32_t *tile_off,
                          hipStream_t s);

}  // namespace bqm
