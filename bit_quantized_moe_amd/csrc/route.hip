// Softmax top-k routing and the stable counting-sort permutation of routed rows.
//
// The expert module of the nf4moe page receives top_k_index / top_k_weights
// [T, k] and visits, for every expert that was hit, its tokens in token order
// (a one-hot mask per expert, then torch.where).  Here the R = T*k pairs
// f = t*k + j are sorted by expert with a deterministic three-pass counting sort
// (chunk histograms -> per-expert prefix over chunks and experts -> in-order
// scatter), so the GEMMs find every expert's rows as one contiguous segment of
// the permutation and no count ever travels to the host.
#include "common.h"
#include "internal.h"
#include "perm_dev.h"

namespace bqm {
namespace {

constexpr int kChunk = 2048;  // routed pairs per histogram/scatter chunk

// Wave-wide reductions with DPP moves inside each row of 16 lanes (xor 1, xor 2, the
// half-row mirror, the row mirror), then the four rows' results read from lanes 0, 16,
// 32 and 48: a few cycles each, where a butterfly of cross-lane shuffles waits for the
// LDS crossbar at every step.
template <class F>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, F op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const uint32_t a = op((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = op((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return op(a, b);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
  }));
}
// float -> uint32 with the same order (-inf lowest; NaN above +inf or below -inf by sign)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One wave per token: the E logits are spread over the 64 lanes (NJ <= 16 per lane,
// E <= 64 NJ).
template <int NJ>
__global__ void __launch_bounds__(256) route_kernel(const float *__restrict__ logits, int64_t T,
                                                   int E, int k, int renorm,
                                                   int32_t *__restrict__ topk_idx,
                                                   float *__restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *lg = logits + t * E;
  float v[NJ];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int e = lane + 64 * j;
    v[j] = e < E ? lg[e] : -INFINITY;
    mx = fmaxf(mx, v[j]);
  }
  // the maximum over the wave (fmaxf ignores NaN, as the lane-local maximum does)
  {
    const uint32_t km = wave_max_u32(mx != mx ? 0u : order_key(mx));
    mx = __uint_as_float((km & 0x80000000u) ? (km & 0x7FFFFFFFu) : ~km);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int e = lane + 64 * j;
    if (e < E) sum += expf(v[j] - mx);
  }
  sum = wave_sum_f32(sum);
  uint32_t taken = 0u;  // bit j: this lane's slot j already chosen
  float vsel = -INFINITY;  // lane r: the value and index chosen in round r
  int isel = 0;
  for (int r = 0; r < k; ++r) {
    // lane-local best among untaken slots (larger value, then lower index)
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int e = lane + 64 * j;
      bool ok = e < E && !((taken >> j) & 1u);
      if (ok && (v[j] > bv || (v[j] == bv && e < bi))) {
        bv = v[j];
        bi = e;
      }
    }
    // the wave's best: the largest value, then among the lanes holding it the lowest index
    const uint32_t kb = order_key(bv);
    const uint32_t kmax = wave_max_u32(kb);
    bi = (int)wave_min_u32(kb == kmax ? (uint32_t)bi : 0x7FFFFFFFu);
    bv = __uint_as_float((kmax & 0x80000000u) ? (kmax & 0x7FFFFFFFu) : ~kmax);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) {
      vsel = bv;
      isel = bi;
    }
  }
  // the chosen experts' softmax probabilities, lane r for round r (out of the selection
  // loop, whose rounds depend on each other), and their sum in round order
  const float w = lane < k ? expf(vsel - mx) / sum : 0.0f;
  float wsum = 0.0f;
  if (renorm)
    for (int r = 0; r < k; ++r) wsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), r));
  if (lane < k) {
    topk_idx[t * k + lane] = isel;
    topk_w[t * k + lane] = renorm ? w / wsum : w;
  }
}

// Pass 1: per-chunk histogram of the E experts and the bucket of dropped pairs
// (counts [nchunks][E + 1]).
__global__ void __launch_bounds__(256) perm_hist(const int32_t *__restrict__ idx, int64_t R, int E,
                                                 int32_t *__restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e <= E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  int64_t b = (int64_t)blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
    int64_t f = b + i;
    if (f < R) atomicAdd(&hist[bucket_of(idx[f], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) counts[(int64_t)blockIdx.x * (E + 1) + e] = hist[e];
}

// Pass 2 (one block): base[c][e] = offsets[e] + sum_{c' < c} counts[c'][e];
// offsets = exclusive prefix of the per-expert totals; the dropped bucket E starts
// at offsets[E].  Optionally the prefixes
// of ceil(count / bm) and ceil(count / bm2) (row tiles per expert) for the grouped
// GEMMs; with bm2 < 0 the second prefix instead counts one tile per expert whose rows
// past its last full bm-row tile number between 1 and -bm2 (rem_tile).  The prefixes over experts are a wave-level inclusive scan plus the totals
// of the waves before.
__global__ void __launch_bounds__(1024) perm_scan(int32_t *__restrict__ counts, int nchunks, int E,
                                                  int32_t *__restrict__ offsets, int bm,
                                                  int32_t *__restrict__ tile_off, int bm2,
                                                  int32_t *__restrict__ tile_off2) {
  __shared__ int32_t wsum[16][3];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const int64_t ld = E + 1;
  int32_t run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      int32_t v = counts[c * ld + e];
      counts[c * ld + e] = run;
      run += v;
    }
  }
  const int32_t tiles = (e < E && bm > 0) ? (run + bm - 1) / bm : 0;
  const int32_t tiles2 = e < E ? tiles_2(run, bm, bm2) : 0;
  int32_t v = run, u = tiles, u2 = tiles2;  // inclusive prefixes within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t tv = __shfl_up(v, off, 64), tu = __shfl_up(u, off, 64), tu2 = __shfl_up(u2, off, 64);
    if (lane >= off) {
      v += tv;
      u += tu;
      u2 += tu2;
    }
  }
  if (lane == 63) {
    wsum[wave][0] = v;
    wsum[wave][1] = u;
    wsum[wave][2] = u2;
  }
  __syncthreads();
  int32_t bv = 0, bu = 0, bu2 = 0;  // totals of the waves before this one
  for (int q = 0; q < wave; ++q) {
    bv += wsum[q][0];
    bu += wsum[q][1];
    bu2 += wsum[q][2];
  }
  const int32_t ex = bv + v - run, ext = bu + u - tiles, ext2 = bu2 + u2 - tiles2;  // exclusive prefixes
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) counts[c * ld + e] += ex;
    offsets[e] = ex;
    if (tile_off) tile_off[e] = ext;
    if (tile_off2) tile_off2[e] = ext2;
  }
  if (e == E - 1) {
    offsets[E] = ex + run;
    if (tile_off) tile_off[E] = ext + tiles;
    if (tile_off2) tile_off2[E] = ext2 + tiles2;
    // the dropped pairs follow every expert's rows, chunk by chunk
    int32_t drun = ex + run;
    for (int c = 0; c < nchunks; ++c) {
      const int32_t v = counts[c * ld + E];
      counts[c * ld + E] = drun;
      drun += v;
    }
  }
}

// Pass 3: one wave scatters its chunk in order, 64 pairs at a time; equal experts
// inside a group are ranked by lane, so the result is the stable order.
__global__ void __launch_bounds__(64) perm_scatter(const int32_t *__restrict__ idx, int64_t R, int E,
                                                   const int32_t *__restrict__ base,
                                                   int32_t *__restrict__ perm,
                                                   int32_t *__restrict__ inv, const float *__restrict__ w_in,
                                                   float *__restrict__ w_out) {
  extern __shared__ int32_t cnt[];
  const int lane = threadIdx.x;
  for (int e = lane; e <= E; e += 64) cnt[e] = base[(int64_t)blockIdx.x * (E + 1) + e];
  const int64_t b = (int64_t)blockIdx.x * kChunk;
  if (w_in)  // this chunk's routing weights, copied on the way (16 bytes per lane and step)
    for (int64_t f = b + 4 * lane; f < b + kChunk && f < R; f += 256) {
      if (f + 4 <= R)
        *reinterpret_cast<float4 *>(w_out + f) = *reinterpret_cast<const float4 *>(w_in + f);
      else
        for (int64_t g = f; g < R; ++g) w_out[g] = w_in[g];
    }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull, upto = lane == 63 ? ~0ull : (2ull << lane) - 1ull;
  for (int s = 0; s < kChunk && b + s < R; s += 64) {
    int64_t f = b + s + lane;
    int e = f < R ? bucket_of(idx[f], E) : -1;
    const uint64_t same = lanes_equal(e + 1);  // pairs past R (e = -1) match only each other
    const int rank = __popcll(same & below);
    const bool last = (same & ~upto) == 0ull;
    int pos = 0;
    if (e >= 0) pos = cnt[e] + rank;
    __syncthreads();
    if (e >= 0) {
      perm[pos] = (int32_t)f;
      inv[f] = pos;
      if (last) cnt[e] = pos + 1;
    }
    __syncthreads();
  }
}

// One chunk (R <= kChunk): the three passes in one launch of one workgroup
__global__ void __launch_bounds__(1024) perm_one(const int32_t *__restrict__ idx, int R, int E,
                                                 int32_t *__restrict__ offsets, int bm, int32_t *__restrict__ tile_off,
                                                 int bm2, int32_t *__restrict__ tile_off2, int32_t *__restrict__ perm,
                                                 int32_t *__restrict__ inv, const float *__restrict__ w_in,
                                                 float *__restrict__ w_out) {
  extern __shared__ int32_t cnt[];  // E + 1 buckets
  perm_one_body(idx, R, E, offsets, bm, tile_off, bm2, tile_off2, perm, inv, w_in, w_out, cnt);
}

}  // namespace

size_t permute_ws_bytes(int64_t R, int E) {
  return (size_t)cdiv(R, kChunk) * (size_t)(E + 1) * sizeof(int32_t);
}

bqm_status permute_launch(const int32_t *topk_idx, int64_t R, int E, int32_t *perm, int32_t *inv,
                          int32_t *offsets, int32_t *counts_ws, int bm, int32_t *tile_off, int bm2,
                          int32_t *tile_off2, hipStream_t s, const float *w_in, float *w_out) {
  if (R > 0 && R <= kChunk) {
    perm_one<<<1, 1024, (E + 1) * sizeof(int32_t), s>>>(topk_idx, (int)R, E, offsets, bm, tile_off, bm2, tile_off2,
                                                         perm, inv, w_in, w_out);
    return launch_status("perm_one");
  }
  const int nchunks = (int)cdiv(R, kChunk);
  if (R > 0) {
    perm_hist<<<nchunks, 256, (E + 1) * sizeof(int32_t), s>>>(topk_idx, R, E, counts_ws);
    bqm_status st = launch_status("perm_hist");
    if (st != BQM_OK) return st;
  }
  perm_scan<<<1, 1024, 0, s>>>(counts_ws, nchunks, E, offsets, bm, tile_off, bm2, tile_off2);
  bqm_status st = launch_status("perm_scan");
  if (st != BQM_OK) return st;
  if (R > 0) {
    perm_scatter<<<nchunks, 64, (E + 1) * sizeof(int32_t), s>>>(topk_idx, R, E, counts_ws, perm, inv, w_in, w_out);
    st = launch_status("perm_scatter");
  }
  return st;
}

}  // namespace bqm

using namespace bqm;

extern "C" bqm_status bqm_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t renorm,
                                int32_t *topk_idx, float *topk_w, void *stream) {
  BQM_REQUIRE(T >= 0, BQM_ERR_INVALID_ARG, "bqm_route: T < 0");
  BQM_REQUIRE(E >= 1 && E <= 1024, BQM_ERR_SHAPE, "bqm_route: E=%d outside [1, 1024]", E);
  BQM_REQUIRE(k >= 1 && k <= E && k <= 16, BQM_ERR_SHAPE, "bqm_route: k=%d outside [1, min(E,16)]",
              k);
  if (T == 0) return BQM_OK;
  BQM_REQUIRE(logits && topk_idx && topk_w, BQM_ERR_INVALID_ARG, "bqm_route: NULL pointer");
  BQM_REQUIRE(aligned16(logits) && aligned16(topk_idx) && aligned16(topk_w), BQM_ERR_ALIGN,
              "bqm_route: pointer not 16-byte aligned");
  const unsigned grid = (unsigned)cdiv(T, 4);
  hipStream_t s = as_stream(stream);
  if (E <= 64)
    route_kernel<1><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, topk_w);
  else if (E <= 128)
    route_kernel<2><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, topk_w);
  else if (E <= 256)
    route_kernel<4><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, topk_w);
  else if (E <= 512)
    route_kernel<8><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, topk_w);
  else
    route_kernel<16><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, topk_idx, topk_w);
  return launch_status("route_kernel");
}

extern "C" size_t bqm_permute_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return permute_ws_bytes(T * k, E);
}

extern "C" bqm_status bqm_permute(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k,
                                  int32_t *perm, int32_t *inv, int32_t *offsets, void *ws,
                                  size_t ws_bytes, void *stream) {
  BQM_REQUIRE(T >= 0, BQM_ERR_INVALID_ARG, "bqm_permute: T < 0");
  BQM_REQUIRE(E >= 1 && E <= 1024, BQM_ERR_SHAPE, "bqm_permute: E=%d outside [1, 1024]", E);
  BQM_REQUIRE(k >= 1 && k <= E, BQM_ERR_SHAPE, "bqm_permute: k=%d outside [1, E]", k);
  BQM_REQUIRE(offsets, BQM_ERR_INVALID_ARG, "bqm_permute: offsets is NULL");
  BQM_REQUIRE(aligned16(offsets), BQM_ERR_ALIGN, "bqm_permute: offsets not 16-byte aligned");
  const int64_t R = T * k;
  size_t need = permute_ws_bytes(R, E);
  BQM_REQUIRE((need == 0 || ws) && ws_bytes >= need, BQM_ERR_WORKSPACE,
              "bqm_permute: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  BQM_REQUIRE(!ws || aligned16(ws), BQM_ERR_ALIGN, "bqm_permute: ws not 16-byte aligned");
  if (R > 0) {
    BQM_REQUIRE(topk_idx && perm && inv, BQM_ERR_INVALID_ARG, "bqm_permute: NULL pointer");
    BQM_REQUIRE(aligned16(topk_idx) && aligned16(perm) && aligned16(inv), BQM_ERR_ALIGN,
                "bqm_permute: pointer not 16-byte aligned");
  }
  return permute_launch(topk_idx, R, E, perm, inv, offsets, reinterpret_cast<int32_t *>(ws), 0,
                        nullptr, 0, nullptr, as_stream(stream));
}
