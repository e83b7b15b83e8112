// Declarations shared between the library's translation units (not part of the ABI).
#pragma once

#include "common.h"

namespace bqm {

// Stable counting sort of R routed pairs by expert (route.hip).  counts_ws needs
// permute_ws_bytes(R, E).  If tile_off != NULL it also receives the prefix sum of
// ceil(count_e / bm) over experts ([E+1] entries); tile_off2 likewise for bm2.  With
// w_in, the R routing weights are also copied to w_out (by the permutation's own
// kernels: no separate copy).
size_t permute_ws_bytes(int64_t R, int E);
bqm_status permute_launch(const int32_t *topk_idx, int64_t R, int E, int32_t *perm, int32_t *inv,
                          int32_t *offsets, int32_t *counts_ws, int bm, int32_t *tile_off, int bm2,
                          int32_t *tile_off2, hipStream_t s, const float *w_in = nullptr, float *w_out = nullptr);

// Per-token NVFP4 (Four-Over-Six) of n_rows bf16 rows of cols elements (cols % 16 == 0,
// 16-byte aligned pointers), and in the same pass the rows of val * sb in bf16, exact
// (quant.hip): the activation rows of the W4A4 GEMMs, whose per-row s_dec is applied to
// the accumulator.
bqm_status nvfp4_quantize_rows_expand(const uint16_t *x, int64_t n_rows, int64_t cols, uint8_t *codes,
                                      uint8_t *scales, float *s_dec, uint16_t *expanded, hipStream_t s);

}  // namespace bqm
