// Device helpers of the stable counting-sort permutation of routed pairs by expert,
// shared by the permutation kernels and the decode path's launch that fuses the
// one-workgroup permutation with the first LoRA projection.
#pragma once
#include <cstdint>
#include <hip/hip_runtime.h>

namespace bqm {
namespace {

// Expert index of a routed pair, with every index outside [0, E) sent to bucket E:
// such a pair belongs to no expert, and the sort places it after offsets[E].
__device__ __forceinline__ int bucket_of(int32_t e, int E) { return (uint32_t)e < (uint32_t)E ? e : E; }

// row tiles of an expert with n rows for the second prefix: ceil(n / bm2), or with
// bm2 < 0 one remainder tile when 0 < n mod bm <= -bm2
__device__ __forceinline__ int32_t tiles_2(int32_t n, int bm, int bm2) {
  if (bm2 > 0) return (n + bm2 - 1) / bm2;
  if (bm2 < 0 && bm > 0) {
    const int32_t r = n % bm;
    return r > 0 && r <= -bm2 ? 1 : 0;
  }
  return 0;
}

// lanes of the wave whose value equals this lane's (0 <= value < 2048: eleven bits)
__device__ __forceinline__ uint64_t lanes_equal(int v) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    const bool bit = (v >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// One chunk (R <= 2048 pairs, decode-sized batches): the histogram, the scans and
// the ordered scatter of the three-pass permutation in one workgroup of 1024
// threads.  Expert counts, offsets, tile prefixes, perm and inv are those of the
// three passes.  cnt: E + 1 ints of LDS.
__device__ __forceinline__ void perm_one_body(const int32_t *__restrict__ idx, int R, int E,
                                                 int32_t *__restrict__ offsets, int bm, int32_t *__restrict__ tile_off,
                                                 int bm2, int32_t *__restrict__ tile_off2, int32_t *__restrict__ perm,
                                                 int32_t *__restrict__ inv, const float *__restrict__ w_in,
                                                 float *__restrict__ w_out, int32_t *cnt) {
  __shared__ int32_t wsum[16][3];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (w_in)
    for (int f = t; f < R; f += 1024) w_out[f] = w_in[f];
  for (int e = t; e <= E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int f = t; f < R; f += 1024) atomicAdd(&cnt[bucket_of(idx[f], E)], 1);
  __syncthreads();
  const int e = t;
  const int32_t run = e < E ? cnt[e] : 0;
  const int32_t tiles = (e < E && bm > 0) ? (run + bm - 1) / bm : 0;
  const int32_t tiles2 = e < E ? tiles_2(run, bm, bm2) : 0;
  int32_t v = run, u = tiles, u2 = tiles2;
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
  int32_t bv = 0, bu = 0, bu2 = 0;
  for (int q = 0; q < wave; ++q) {
    bv += wsum[q][0];
    bu += wsum[q][1];
    bu2 += wsum[q][2];
  }
  const int32_t ex = bv + v - run, ext = bu + u - tiles, ext2 = bu2 + u2 - tiles2;
  if (e < E) {
    offsets[e] = ex;
    if (tile_off) tile_off[e] = ext;
    if (tile_off2) tile_off2[e] = ext2;
  }
  if (e == E - 1) {
    offsets[E] = ex + run;
    if (tile_off) tile_off[E] = ext + tiles;
    if (tile_off2) tile_off2[E] = ext2 + tiles2;
  }
  __syncthreads();  // every count has been read
  if (e < E) cnt[e] = ex;
  if (e == E - 1) cnt[E] = ex + run;  // the dropped pairs follow every expert's rows
  __syncthreads();
  // wave 0 places the pairs in order, 64 at a time (equal experts ranked by lane)
  const uint64_t below = (1ull << lane) - 1ull, upto = lane == 63 ? ~0ull : (2ull << lane) - 1ull;
  for (int s0 = 0; s0 < R; s0 += 64) {
    int pos = 0, bk = -1;
    bool last = false;
    if (wave == 0) {
      const int f = s0 + lane;
      bk = f < R ? bucket_of(idx[f], E) : -1;
      const uint64_t same = lanes_equal(bk + 1);
      const int rank = __popcll(same & below);
      last = (same & ~upto) == 0ull;
      if (bk >= 0) pos = cnt[bk] + rank;
    }
    __syncthreads();
    if (wave == 0 && bk >= 0) {
      perm[pos] = s0 + lane;
      inv[s0 + lane] = pos;
      if (last) cnt[bk] = pos + 1;
    }
    __syncthreads();
  }
}


}  // namespace
}  // namespace bqm
