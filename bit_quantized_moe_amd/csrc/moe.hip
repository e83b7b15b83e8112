// The routed-expert MoE layer over rowwise 4-bit expert weights with a bf16 LoRA:
// forward, dgrad through DQ(Q(W)) and the LoRA weight gradients, on gfx950.
//
// Forward (nf4moe page, the QuantizedNaiveMoe forward): for each routed pair
// (t, j) with expert e, h = X~ W~_gu^T + s (X A_gu^T) B_gu^T, a = silu(gate) * up
// (the chunk(2, -1) halves of h), y = a~ W~_dn^T + s (a A_dn^T) B_dn^T, and the
// layer output adds y times the routing weight back onto token t.  Dgrad (GLM
// page, section "The 4-bit base that was actually using 8-bit memory"): the
// input gradient contracts the output dimension of each weight, so it reads
// the single rowwise copy transposed, dequantized to bf16; no columnwise copy
// exists.  Only experts that received rows are ever read.
//
// Structure: the routed pairs are sorted by expert (route.hip), so each expert
// owns a contiguous segment of rows.  Two grouped-GEMM kernels (namespace fq) run
// the four weight contractions: a 256 x 256 output tile of one expert per
// workgroup of four waves (one per SIMD, each owning 256 rows x 64 columns), a K
// loop in steps of 64 through three LDS stages filled by direct-to-LDS copies two
// steps ahead, bf16 MFMA 32x32x16 with FP32 accumulation, then the LoRA
// up-projection as a short second segment and a fused epilogue (SwiGLU, routing
// weight, SwiGLU backward).  The weights go to LDS as stored (4-bit codes and
// their block scales) and are decoded in registers right before the MFMAs:
//   - gemm_fwd_q4 reads the codes K-major (forward, and a dgrad over a columnwise
//     copy); NVFP4 as e2m1 * e4m3 (exact in bf16; the FP32 per-tensor scale goes
//     on the accumulator), NF4 through a per-column 16-entry table of
//     bf16(level * absmax) looked up with byte permutes;
//   - gemm_dgrad_q4 reads the single rowwise copy transposed (4-bit transposing
//     LDS read, NVFP4), or for NF4 decodes its rows into a per-wave bf16 tile read
//     back with the 16-bit transposing read.
// With at most one routed row per expert on average (decode-sized batches), the
// forward GEMMs run gv::fwd_stream instead: no LDS stages for the weights, whose codes
// stream from HBM straight into registers, 16x16x32 MFMAs over up to 16 rows per pass.
// The LoRA down-projections (N = r) stream through lp::gemm_lora_proj; the LoRA
// weight gradients through lora_wgrad.  Workgroups are mapped so that each of the
// 8 XCDs walks a contiguous range of tiles: the tiles in flight on one XCD share
// an expert's activation rows and weight rows in that XCD's L2.
#include "common.h"
#include "internal.h"
#include "perm_dev.h"
#include "nf4_levels.inc"

#include <type_traits>

namespace bqm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int BM = 256;       // output rows per tile (routed rows of one expert)
constexpr int BK = 64;        // K step (one NF4 block, four NVFP4 blocks)
constexpr int NTHR = 256;

// A operand rows: bf16 activations gathered by token (A_GATHER) or in routed order
// (A_ROWS); the _Q forms are per-row NVFP4 activations expanded to bf16 val * sb
// (exact), whose per-row decode scales (Seg::a_sd) multiply the accumulator.
enum ASrc { A_GATHER = 0, A_ROWS = 1, A_GATHER_Q = 2, A_ROWS_Q = 3 };
enum Epi { EPI_GATEUP = 0, EPI_STORE = 1, EPI_DOWN_DGRAD = 2, EPI_STORE_SPLIT = 4 };

// One K segment of a contraction: A rows times one expert slice of a B stack.
struct Seg {
  const void *a;        // bf16 rows
  const float *a_sd;    // per-row decode scales of the _Q sources
  int64_t a_ld;         // elements per A row
  const void *b;        // B stack: 4-bit codes or bf16
  const void *b_sc;     // NVFP4 E4M3 scales / NF4 absmax
  const float *b_sd;    // NVFP4 per-expert decode scales
  int64_t b_rows, b_cols;  // one expert slice of the B stack is [b_rows, b_cols]
  int64_t b_estride;       // bf16 B: elements from one expert's slice to the next (0: one matrix for all)
  int b_nested;            // NF4: the absmax is the nested code (b_sc uint8, b_sd [offset, group scales])
  int K;
  int kmod;  // > 0: B is indexed at k mod kmod (A holds a hi/lo pair of K = 2*kmod)
};

struct GemmParams {
  const int32_t *perm, *offsets, *tile_off;
  int E, k;
  int N;   // output columns
  int I;   // gate/up split point
  int NT;  // output column tiles
  Seg s1, s2;  // s2.K == 0: no second segment
  float out_scale;
  const float *div_e;     // EPI_STORE_SPLIT: per-expert divisor of the output (NULL: none)
  uint16_t *out0, *out1;  // bf16 outputs
  float *outf;            // FP32 output (the gate/up activations h)
  const float *h_in;      // saved FP32 gate/up activations (dgrad epilogue)
  const float *tw;        // routing weight of pair f (dgrad epilogue)
  // Remainder tiles (the training-size forward): an expert whose rows past its last full
  // 256-row tile number at most 64 has those rows computed by the 64-row kernel.
  // tile_rem: the prefix of those tiles (one per such expert); the 256-row kernel then
  // skips them (its tiles per expert: tile_off minus tile_rem), and the 64-row kernel,
  // with rem_rows set, takes tile_rem as its tile prefix and starts each expert's rows
  // after its full 256-row tiles.
  const int32_t *tile_rem;
  int rem_rows;
  int rows_pass;  // the weight-streaming forward: rows per pass (its activation rows in LDS)
  // EPI_DOWN_DGRAD: per routed row and output column tile, the sum over the tile's columns
  // of da_u * a (the routing-weight gradient's share of the tile), [R][NT]; NULL: none
  float *dtw_part;
};

__constant__ float c_nf4[16] = BQM_NF4_LEVELS;

// ---------------------------------------------------------------------------
// tile-column -> weight-row mapping
// ---------------------------------------------------------------------------
// Gate/up interleave: in each 64-column group of the tile the first 32 columns
// are gate rows i and the next 32 the matching up rows I + i, so the epilogue
// finds g and u of the same element in the same lane and register.
template <int EPI, int BN>
__device__ __forceinline__ int64_t b_row_of_col(int j, int nt, int N, int I) {
  if constexpr (EPI == EPI_GATEUP) {
    int i = nt * (BN / 2) + (j >> 6) * 32 + (j & 31);
    if (i >= I) return -1;
    return (j & 32) ? (int64_t)I + i : (int64_t)i;
  } else {
    int n = nt * BN + j;
    return n < N ? n : -1;
  }
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// E4M3 scale byte -> float (hardware OCP E4M3 decode; exact, subnormals included)
template <int SEL>
__device__ __forceinline__ float e4m3_hw(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

// ---------------------------------------------------------------------------
// exact 4-bit -> bf16 conversion with the hardware FP4 converter
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) float f32x2;

// bf16 bits of two exactly representable floats, packed (lo, hi)
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
  // bytes 2,3 of lo then bytes 2,3 of hi: (lo >> 16) | (hi & 0xFFFF0000) in one byte permute
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// byte `sel` of c holds two E2M1 codes (low nibble first) -> their values times sb
template <int SEL>
__device__ __forceinline__ f32x2 fp4pair(uint32_t c, float sb) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, SEL);
  return v * sb;  // exact: <= 6 significant bits
}

// Nested NF4: absmax' of every block of a stack, fl(fl(e4m3(q) * s2[group]) + offset)
// in FP32 (the same two roundings as nf4_absmax_load), written to a workspace buffer so
// that the GEMMs read it as plain FP32 absmax.  Matrix blockIdx.y, nb blocks per
// matrix, G groups of 256 blocks per matrix; four blocks per thread when nb % 4 == 0.
template <bool VEC4>
__global__ void __launch_bounds__(256) nf4_unnest(const uint8_t *__restrict__ q, const float *__restrict__ sd,
                                                  int64_t nb, int64_t G, float *__restrict__ out) {
#pragma clang fp contract(off)
  const int64_t m = blockIdx.y;
  const float *sdm = sd + m * (1 + G);
  const float off = sdm[0];
  const uint8_t *qm = q + m * nb;
  float *om = out + m * nb;
  if constexpr (VEC4) {
    for (int64_t b = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; b < nb; b += (int64_t)gridDim.x * 1024) {
      const uint32_t c = *reinterpret_cast<const uint32_t *>(qm + b);
      const float s2 = sdm[1 + (b >> 8)];  // the four blocks share a group (256 % 4 == 0)
      float4 v;
      v.x = __builtin_amdgcn_cvt_f32_fp8(c, 0) * s2;
      v.y = __builtin_amdgcn_cvt_f32_fp8(c, 1) * s2;
      v.z = __builtin_amdgcn_cvt_f32_fp8(c, 2) * s2;
      v.w = __builtin_amdgcn_cvt_f32_fp8(c, 3) * s2;
      v.x = v.x + off;
      v.y = v.y + off;
      v.z = v.z + off;
      v.w = v.w + off;
      *reinterpret_cast<float4 *>(om + b) = v;
    }
  } else {
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nb; b += (int64_t)gridDim.x * 256) {
      const float prod = __builtin_amdgcn_cvt_f32_fp8(qm[b], 0) * sdm[1 + (b >> 8)];
      om[b] = prod + off;
    }
  }
}

// A wave-uniform float loaded once into a scalar register.  Loaded into a vector
// register instead, its first use sits inside the epilogue's per-element branches,
// and the wait for the load is then repeated before every store (each such wait
// also drains the stores already issued).
__device__ __forceinline__ float uniform_load(const float *ptr) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(*ptr)));
}

// logistic function with the hardware exponential and reciprocal (about 2 ulp)
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// ---------------------------------------------------------------------------
// the grouped GEMM
// ---------------------------------------------------------------------------
// B fragment (8 consecutive k of one column per lane) from a natural [k][n] tile
// Fragment (8 consecutive rows k of one column per lane) from a natural
// [k][col] tile with row stride STRIDE bf16, via the transposing LDS read.
template <int STRIDE>
__device__ __forceinline__ bf16x8 b_frag_trans_s(const uint16_t *Bs, int kbase, int nbase, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = kbase + 8 * (g >> 1) + (s >> 2);
  const int col = nbase + 16 * (g & 1) + 4 * (s & 3);
  const uint16_t *p0 = Bs + row * STRIDE + col;
  const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0));
  const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 4 * STRIDE));
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  const s16x8 v = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// epilogues: acc[tm][tn] element v of a wave holds row row0 + tm*32 + 8(v/4) +
// 4(lane/32) + v%4 and column col0 + tn*32 + lane%32 of the tile
// ---------------------------------------------------------------------------
// FULL: every row and column of this wave's block is inside the output (the common
// case), so the per-element bounds tests and their branches are left out.
template <int TM, int TN, int BN, int EPI, bool FULL>
__device__ __forceinline__ void epilogue_body(const GemmParams &p, const f32x16 (&acc)[TM][TN], float osc, int nt,
                                              int m0, int n_e, int rb, int row0, int col0, int lane, float esc) {
  const float sc = esc * p.out_scale;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int pos = m0 + row0 + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (!FULL && pos >= n_e) continue;
      const int64_t grow = rb + pos;
      if constexpr (EPI == EPI_GATEUP) {
        // in each 64-column group of the tile: 32 gate columns, then the matching up columns
#pragma unroll
        for (int q = 0; q < TN / 2; ++q) {
          const int i = nt * (BN / 2) + col0 / 2 + q * 32 + (lane & 31);
          if (!FULL && i >= p.I) continue;
          const float g = acc[tm][2 * q][v] * esc, u = acc[tm][2 * q + 1][v] * esc;
          const float a = g * sigmoid_f(g) * u;
          p.outf[grow * 2 * p.I + i] = g;
          p.outf[grow * 2 * p.I + p.I + i] = u;
          p.out1[grow * p.I + i] = (uint16_t)f32_to_bf16(a);
        }
      } else if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int n = nt * BN + col0 + tn * 32 + (lane & 31);
          if (FULL || n < p.N) p.out0[grow * p.N + n] = (uint16_t)f32_to_bf16(acc[tm][tn][v] * sc);
        }
      } else if constexpr (EPI == EPI_STORE_SPLIT) {
        // FP32 value kept as an unevaluated pair of bf16 (hi in columns [0, N), lo in [N, 2N))
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int n = nt * BN + col0 + tn * 32 + (lane & 31);
          if (FULL || n < p.N) {
            const float val = acc[tm][tn][v] * osc;
            const uint32_t hb = f32_to_bf16(val);
            const float lo2 = val - __uint_as_float(hb << 16);
            p.out0[grow * 2 * p.N + n] = (uint16_t)hb;
            p.out0[grow * 2 * p.N + p.N + n] = (uint16_t)f32_to_bf16(lo2);
          }
        }
      }
    }
  }
}

template <int TM, int TN, int BN, int EPI>
__device__ __forceinline__ void epilogue(const GemmParams &p, const f32x16 (&acc)[TM][TN], int e, int nt, int m0,
                                         int n_e, int rb, int row0, int col0, int lane, float esc) {
  const bool rows_in = m0 + row0 + TM * 32 <= n_e;
  const float osc = p.div_e ? p.out_scale / uniform_load(p.div_e + e) : p.out_scale;
  const bool cols_in = EPI == EPI_GATEUP ? nt * (BN / 2) + col0 / 2 + (TN / 2) * 32 <= p.I
                                         : nt * BN + col0 + TN * 32 <= p.N;
  if (rows_in && cols_in)
    epilogue_body<TM, TN, BN, EPI, true>(p, acc, osc, nt, m0, n_e, rb, row0, col0, lane, esc);
  else
    epilogue_body<TM, TN, BN, EPI, false>(p, acc, osc, nt, m0, n_e, rb, row0, col0, lane, esc);
}

// Epilogue of the accumulator transposed: the grouped GEMMs of namespace fq issue
// their MFMAs as weights x activations, so element v of lane L holds output column
// 8(v/4) + 4(L/32) + v%4 of row L%32.  Each lane then owns one row per 32-row tile
// and 4 consecutive columns per group of 4 registers: one 8- or 16-byte store (or
// load) per 4 values instead of one per value, and one routing weight per row.
template <int TM, int TN, int BN, int EPI, bool FULL>
__device__ __forceinline__ void epilogue_t_body(const GemmParams &p, const f32x16 (&acc)[TM][TN], int nt, int m0,
                                                int n_e, int rb, int row0, int col0, int lane, float esc,
                                                float (&dp)[TM], bool dtw) {
  static_assert(EPI == EPI_STORE || EPI == EPI_GATEUP || EPI == EPI_DOWN_DGRAD, "transposed epilogues");
  const int g = lane >> 5;
  const float sc = esc * p.out_scale;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int pos = m0 + row0 + tm * 32 + (lane & 31);
    const bool row_ok = FULL || pos < n_e;
    const int64_t grow = rb + (FULL ? pos : min(pos, n_e - 1));
    if constexpr (EPI == EPI_STORE) {
      if (row_ok) {
        uint16_t *__restrict__ out = p.out0 + grow * p.N;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = nt * BN + col0 + tn * 32 + 8 * q + 4 * g;
            if (FULL || n < p.N) {
              const uint32_t lo = f32_to_bf16(acc[tm][tn][4 * q] * sc) | (f32_to_bf16(acc[tm][tn][4 * q + 1] * sc) << 16);
              const uint32_t hi = f32_to_bf16(acc[tm][tn][4 * q + 2] * sc) | (f32_to_bf16(acc[tm][tn][4 * q + 3] * sc) << 16);
              *reinterpret_cast<uint2 *>(out + n) = make_uint2(lo, hi);
            }
          }
      }
    } else if constexpr (EPI == EPI_GATEUP) {
      // each 64-column group of the tile: 32 gate columns (tile tn = 2 qq), then the
      // matching 32 up columns (tn = 2 qq + 1)
      if (row_ok) {
#pragma unroll
        for (int qq = 0; qq < TN / 2; ++qq)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = nt * (BN / 2) + col0 / 2 + qq * 32 + 8 * q + 4 * g;
            if (FULL || i < p.I) {
              float gv[4], uv[4];
              uint32_t a2[2];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                gv[t] = acc[tm][2 * qq][4 * q + t] * esc;
                uv[t] = acc[tm][2 * qq + 1][4 * q + t] * esc;
              }
#pragma unroll
              for (int t = 0; t < 2; ++t)
                a2[t] = f32_to_bf16(gv[2 * t] * sigmoid_f(gv[2 * t]) * uv[2 * t]) |
                        (f32_to_bf16(gv[2 * t + 1] * sigmoid_f(gv[2 * t + 1]) * uv[2 * t + 1]) << 16);
              float *hrow = p.outf + grow * 2 * p.I;
              *reinterpret_cast<float4 *>(hrow + i) = make_float4(gv[0], gv[1], gv[2], gv[3]);
              *reinterpret_cast<float4 *>(hrow + p.I + i) = make_float4(uv[0], uv[1], uv[2], uv[3]);
              *reinterpret_cast<uint2 *>(p.out1 + grow * p.I + i) = make_uint2(a2[0], a2[1]);
            }
          }
      }
    } else {  // EPI_DOWN_DGRAD: da = w * da_u, SwiGLU backward -> dh = [dg, du]
      const float *__restrict__ hrow = p.h_in + grow * 2 * p.I;
      const float w = p.tw[p.perm[grow]];
      float4 gv[TN][4], uv[TN][4];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int i = nt * BN + col0 + tn * 32 + 8 * q + 4 * g;
          i = (FULL || i < p.N) ? i : 0;
          gv[tn][q] = *reinterpret_cast<const float4 *>(hrow + i);
          uv[tn][q] = *reinterpret_cast<const float4 *>(hrow + p.I + i);
        }
      if (row_ok) {
        uint16_t *__restrict__ out = p.out0 + grow * 2 * p.I;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = nt * BN + col0 + tn * 32 + 8 * q + 4 * g;
            if (FULL || i < p.N) {
              const float gg[4] = {gv[tn][q].x, gv[tn][q].y, gv[tn][q].z, gv[tn][q].w};
              const float uu[4] = {uv[tn][q].x, uv[tn][q].y, uv[tn][q].z, uv[tn][q].w};
              uint32_t dg2[2], du2[2];
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                float dgv[2], duv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  const int j = 2 * t + h;
                  const float sg = sigmoid_f(gg[j]);
                  const float dau = acc[tm][tn][4 * q + j] * esc;
                  const float da = w * dau;
                  dgv[h] = da * uu[j] * sg * (1.0f + gg[j] * (1.0f - sg));
                  duv[h] = da * gg[j] * sg;
                  // routing-weight gradient: da_u times the forward's bf16 a (the same
                  // expression and rounding as the gate_up epilogue)
                  if (dtw) dp[tm] += dau * __uint_as_float(f32_to_bf16(gg[j] * sg * uu[j]) << 16);
                }
                dg2[t] = f32_to_bf16(dgv[0]) | (f32_to_bf16(dgv[1]) << 16);
                du2[t] = f32_to_bf16(duv[0]) | (f32_to_bf16(duv[1]) << 16);
              }
              *reinterpret_cast<uint2 *>(out + i) = make_uint2(dg2[0], dg2[1]);
              *reinterpret_cast<uint2 *>(out + p.I + i) = make_uint2(du2[0], du2[1]);
            }
          }
      }
    }
  }
}

// dp (EPI_DOWN_DGRAD with p.dtw_part set): per 32-row tile, this lane's sum of da_u * a
// over its columns, added to dp[tm]
template <int TM, int TN, int BN, int EPI>
__device__ __forceinline__ void epilogue_t(const GemmParams &p, const f32x16 (&acc)[TM][TN], int nt, int m0, int n_e,
                                           int rb, int row0, int col0, int lane, float esc, float (&dp)[TM]) {
  const bool rows_in = m0 + row0 + TM * 32 <= n_e;
  const bool cols_in = EPI == EPI_GATEUP ? nt * (BN / 2) + col0 / 2 + (TN / 2) * 32 <= p.I
                                         : nt * BN + col0 + TN * 32 <= p.N;
  const bool dtw = EPI == EPI_DOWN_DGRAD && p.dtw_part != nullptr;
  if (rows_in && cols_in)
    epilogue_t_body<TM, TN, BN, EPI, true>(p, acc, nt, m0, n_e, rb, row0, col0, lane, esc, dp, dtw);
  else
    epilogue_t_body<TM, TN, BN, EPI, false>(p, acc, nt, m0, n_e, rb, row0, col0, lane, esc, dp, dtw);
}
template <int TM, int TN, int BN, int EPI>
__device__ __forceinline__ void epilogue_t(const GemmParams &p, const f32x16 (&acc)[TM][TN], int nt, int m0, int n_e,
                                           int rb, int row0, int col0, int lane, float esc) {
  float dp[TM];
  epilogue_t<TM, TN, BN, EPI>(p, acc, nt, m0, n_e, rb, row0, col0, lane, esc, dp);
}

// The routing-weight gradient's partial sums of one output tile (4 waves of 64 columns,
// TM 32-row tiles): lanes L and L ^ 32 hold the two halves of a wave's columns for row
// L % 32, the four waves' sums are added in wave order through LDS (lds: TM * 128 floats,
// free: the caller has finished its stages), and the tile's rows get part[row][nt].
template <int TM>
__device__ __forceinline__ void dtw_tile(const GemmParams &p, float (&dp)[TM], int nt, int m0, int n_e, int rb,
                                         int wn, int lane, float *lds) {
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) dp[tm] += __shfl_xor(dp[tm], 32, 64);
  __syncthreads();
  if (lane < 32) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) lds[wn * TM * 32 + tm * 32 + lane] = dp[tm];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < TM * 32; i += blockDim.x) {
    const int pos = m0 + i;
    if (pos < n_e) {
      float s = lds[i];
      for (int q = 1; q < 4; ++q) s += lds[q * TM * 32 + i];
      p.dtw_part[(int64_t)(rb + pos) * p.NT + nt] = s;
    }
  }
}

// x *= s on an accumulator element that stays in its AGPR (VALU arithmetic cannot
// read AGPRs; going through the compiler moves the whole accumulator into VGPRs)
__device__ __forceinline__ void scale_acc(float &x, float s) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %1, %0\n\t"
      "v_mul_f32 %1, %2, %1\n\t"
      "v_accvgpr_write_b32 %0, %1"
      : "+a"(x), "=&v"(t)
      : "v"(s));
}

// valid 32-row tiles of a wave: a run-time count (ragged tail)
constexpr int VT_DYN = -1;

// ---------------------------------------------------------------------------
// Forward grouped GEMM over K-major NVFP4 weights (gate_up and down forward)
// ---------------------------------------------------------------------------
// The 4-bit codes and E4M3 scales of the weight tile go global -> LDS with the
// direct-to-LDS load (8 KB + 1 KB per 64-deep K step, instead of 32 KB of
// dequantized bf16 written by the waves), and every wave decodes its own MFMA
// B fragments in registers right before use.  The four waves each own a
// 256 x 64 slab of the 256 x 256 tile, so no two waves decode the same columns.
// bf16 A rows are copied global -> LDS the same way, into 128-byte rows whose
// 16-byte chunk c sits at position c ^ ((row >> 1) & 7), so the 16 lanes of a
// fragment read hit 16 different bank groups.
// Inside a K step, lane group g of a fragment covers k = 32g + 8kk .. +8 in
// slice kk (one fixed permutation of k for A and B alike), so a lane's four
// slices of one weight column are 16 contiguous code bytes and two scale bytes.
namespace fq {
constexpr int BM = 256, BN = 256, NTHR = 256, ACH = 8;
constexpr int WMG = 1, WNG = 4;  // wave grid: WMG x WNG waves of TM x TN 32x32 tiles
constexpr int TM = BM / WMG / 32, TN = BN / WNG / 32;

constexpr int NST = 3;  // LDS stages: copies run two K steps ahead

typedef __attribute__((address_space(3))) void lds_void;

constexpr int DQS = 72;  // row stride (bf16) of the dgrad's decoded NF4 tiles

struct Smem {
  static constexpr int NS = NST, NSG = 0;
  static constexpr int lora_b_bytes = 2 * BM * BK * 2;  // stages 1 and 2 of a[] (seg_lora_n)
  uint16_t a[NST][BM * BK];  // bf16, swizzled 128-byte rows
  uint8_t b[NST][BN * 32];   // codes: 32 bytes per output column (forward), 128 per weight row (dgrad)
  uint32_t s[NST][BN];       // E4M3 block scales of the K step (NF4: FP32 absmax)
  uint8_t t[BN / 64][256];   // dgrad: each wave's scales regrouped per 16-column block
  uint16_t dq[BN / 64][BK * DQS];  // NF4 dgrad: each wave's decoded 64 x 64 weight tile
};

// LDS byte addresses of a stage's A, B and scale areas and the wave index, all
// computed in scalar registers (the copies take their LDS address from M0)
__device__ __forceinline__ uint32_t wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
template <class SM>
__device__ __forceinline__ uint32_t smem_u32(const SM &sm) { return (uint32_t)(uintptr_t)(const lds_void *)&sm; }
template <class SM>
__device__ __forceinline__ uint32_t lds_a(const SM &sm, int st) {
  return smem_u32(sm) + (uint32_t)offsetof(SM, a) + (uint32_t)st * (uint32_t)sizeof(sm.a[0]);
}
template <class SM>
__device__ __forceinline__ uint32_t lds_b(const SM &sm, int st) {
  return smem_u32(sm) + (uint32_t)offsetof(SM, b) + (uint32_t)st * (uint32_t)sizeof(sm.b[0]);
}
template <class SM>
__device__ __forceinline__ uint32_t lds_s(const SM &sm, int st) {
  return smem_u32(sm) + (uint32_t)offsetof(SM, s) + (uint32_t)st * (uint32_t)sizeof(sm.s[0]);
}

// Workgroup barrier that orders LDS (waits for this wave's LDS operations, then
// s_barrier) without waiting for outstanding global loads: __syncthreads() also
// drains vmcnt, which would wait for the copies issued for later steps.  The
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt with vmcnt(n) and no wait on the other counters
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ int a_off(int r, int c) { return r * BK + 8 * (c ^ ((r >> 1) & 7)); }

// row of the tile owned by this thread's j-th A chunk (NC chunks of 8 rows per wave,
// 32 NC rows per tile)
template <int NC = ACH>
__device__ __forceinline__ int a_row(int j) { return 8 * NC * (threadIdx.x >> 6) + 8 * j + ((threadIdx.x & 63) >> 3); }

// A row of this lane's direct copy j when a tile holds VT valid 32-row tiles: each wave
// copies 8 VT rows (VT copies of 8 rows), so a tile copies only the 32 VT rows its
// MFMAs read
template <int VT>
__device__ __forceinline__ int dma_row(int j) { return 8 * VT * (threadIdx.x >> 6) + 8 * j + ((threadIdx.x & 63) >> 3); }

// source rows of the direct copies (routed rows past the expert's segment clamped; their
// results are dropped)
template <int ASRC, int VT>
__device__ __forceinline__ void dma_rows(const GemmParams &p, int rb, int n_e, int m0, int64_t (&arow)[ACH]) {
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int pos = min(m0 + dma_row<VT>(j), n_e - 1);
    arow[j] = (ASRC == A_GATHER || ASRC == A_GATHER_Q) ? (int64_t)(p.perm[rb + pos] / p.k) : (int64_t)(rb + pos);
  }
}


// Direct-to-LDS copies (lane i's 16 or 4 bytes land at lds + 16 i or 4 i), written as
// inline assembly: the compiler's wait-count bookkeeping treats its own form of this
// copy as an LDS event of unknown order and then drains every outstanding LDS read
// (lgkmcnt(0)) before each use of an LDS result, exposing the read latency.  The
// copies are waited for explicitly (wait_vm) before their stage is read.
// lds: the wave-uniform LDS byte address (M0), kept in a scalar register
__device__ __forceinline__ void dma_b128(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}

// A rows through registers (the LoRA segment; k >= K zeroed when MASKK)
template <int NC = ACH>
struct ARegs {
  u32x4 v[NC];
};

template <int ASRC, bool MASKK, int NC = ACH>
__device__ __forceinline__ void a_load(const Seg &s, const int64_t (&arow)[ACH], int k0, ARegs<NC> &r) {
  const int tid = threadIdx.x;
  const uint16_t *a = reinterpret_cast<const uint16_t *>(s.a);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int kk = k0 + (tid & 7) * 8;
    const bool ok = !MASKK || kk < s.K;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(a + arow[i] * s.a_ld + (ok ? kk : 0));
    r.v[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int ASRC, int NC = ACH>
__device__ __forceinline__ void a_store(uint16_t *As, const ARegs<NC> &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NC; ++i) *reinterpret_cast<u32x4 *>(As + a_off(a_row<NC>(i), tid & 7)) = r.v[i];
}

// A fragments of slice kk for row tiles 0..TMA-1
template <int TMA = TM>
__device__ __forceinline__ void a_frags(const uint16_t *As, int kk, int row0, int lane, bf16x8 (&af)[TMA]) {
#pragma unroll
  for (int tm = 0; tm < TMA; ++tm)
    af[tm] = *reinterpret_cast<const bf16x8 *>(As + a_off(row0 + tm * 32 + (lane & 31), 4 * (lane >> 5) + kk));
}

// Weight formats of the register-decode kernels
enum WFmt { WF_NVFP4 = 0, WF_NF4 = 1 };

// this lane's codes (4 slices) and the two block scales of its weight columns
// (NVFP4), or the decode table of each column's 64-block (NF4: the low and high
// bytes of the 16 bf16 values bf16(level[c] * absmax), four entries per register)
struct BCodes {
  u32x4 c[TN];
  float s[TN][2];
  uint32_t lo[TN][4], hi[TN][4];
};

// ---- NF4 in registers ----
// A 64-block of one weight column shares one FP32 absmax a, so its 16 possible
// operands T[c] = bf16(fl(level[c] * a)) (the dequantized value, rounded to nearest
// even) are computed once per column and K step, and every code is a table lookup
// done with byte permutes: the 16 entries' low bytes sit in four registers, their
// high bytes in four more, and v_perm picks four bytes at a time by code.
constexpr float kNF4Levels[16] = BQM_NF4_LEVELS;

__device__ __forceinline__ void nf4_table(float a, uint32_t (&lo)[4], uint32_t (&hi)[4]) {
  uint32_t pr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pr[j] = pack_bf16_rne(kNF4Levels[2 * j] * a, kNF4Levels[2 * j + 1] * a);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = __builtin_amdgcn_perm(pr[2 * i + 1], pr[2 * i], 0x06040200u);
    hi[i] = __builtin_amdgcn_perm(pr[2 * i + 1], pr[2 * i], 0x07050301u);
  }
}

// byte i of the result = plane byte x_i, for x_i = 0..15 in byte i of the code word:
// s = x & 7 picks within entries 0-7 and 8-15, sel = i + 4 * bit3(x_i) chooses between them
__device__ __forceinline__ uint32_t nf4_lut(const uint32_t (&t)[4], uint32_t s, uint32_t sel) {
  const uint32_t a = __builtin_amdgcn_perm(t[1], t[0], s);
  const uint32_t b = __builtin_amdgcn_perm(t[3], t[2], s);
  return __builtin_amdgcn_perm(b, a, sel);
}

// the 8 codes of one slice (element 2j in the low nibble of byte j) -> 4 bf16 pairs, in
// four parts so that the work can sit between MFMAs: part 0 and 1 look up the even
// and odd elements' bytes, parts 2 and 3 interleave them into pairs (e0,e1) .. (e6,e7)
struct NF4Tmp {
  uint32_t so, xo, le, he, lo, ho;
};

template <int PART>
__device__ __forceinline__ void nf4_part(uint32_t c, const uint32_t (&lo)[4], const uint32_t (&hi)[4], NF4Tmp &t,
                                         u32x4 &out) {
  if constexpr (PART == 0) {
    // even elements: the low nibbles (bits 0-2 pick within a half, bit 3 the half)
    const uint32_t se = c & 0x07070707u, xe = ((c >> 1) & 0x04040404u) | 0x03020100u;
    t.so = (c >> 4) & 0x07070707u;
    t.xo = ((c >> 5) & 0x04040404u) | 0x03020100u;
    t.le = nf4_lut(lo, se, xe);
    t.he = nf4_lut(hi, se, xe);
  } else if constexpr (PART == 1) {
    t.lo = nf4_lut(lo, t.so, t.xo);
    t.ho = nf4_lut(hi, t.so, t.xo);
  } else if constexpr (PART == 2) {
    const uint32_t e01 = __builtin_amdgcn_perm(t.he, t.le, 0x05010400u), o01 = __builtin_amdgcn_perm(t.ho, t.lo, 0x05010400u);
    out[0] = __builtin_amdgcn_perm(o01, e01, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(o01, e01, 0x07060302u);
  } else {
    const uint32_t e23 = __builtin_amdgcn_perm(t.he, t.le, 0x07030602u), o23 = __builtin_amdgcn_perm(t.ho, t.lo, 0x07030602u);
    out[2] = __builtin_amdgcn_perm(o23, e23, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(o23, e23, 0x07060302u);
  }
}

template <int PART>
__device__ __forceinline__ void nf4_step(const BCodes &b, int tn, int kk, NF4Tmp &t, u32x4 &out) {
  nf4_part<PART>(b.c[tn][kk], b.lo[tn], b.hi[tn], t, out);
}


template <int VT, int TMA = TM>
__device__ __forceinline__ void mfmas(const bf16x8 (&af)[TMA], const bf16x8 (&bf)[TN], int vt,
                                      f32x16 (&acc)[TMA][TN]) {
#pragma unroll
  for (int tm = 0; tm < TMA; ++tm) {
    if (VT != VT_DYN || tm < vt) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[tn], af[tm], acc[tm][tn], 0, 0, 0);
    }
  }
}

// ---- Segment 1 with A rows copied straight to LDS: software-pipelined K loop ----
// One wave per SIMD has no other wave to hide its waits behind, so the step is
// written out in issue order: each 32-row tile's two MFMAs of slice kk are followed
// by that tile's A-fragment read for slice kk+1 and one bf16 pair of the slice-kk+1
// weight decode (and, in slice 0, one copy of step ks+2), pinned in that order by
// scheduling barriers.  The reads then have a whole slice of MFMAs to land, and the
// decode and address arithmetic issue in the shadow of the matrix pipe.

// per-thread copy sources at K step 0 (advanced by the step's K offset)
struct DmaSrc {
  const uint16_t *a[ACH];
  const uint8_t *c[2];
  const uint8_t *s;
};

template <int EPI, int VT>
__device__ __forceinline__ void dma_src(const Seg &s, const int64_t (&arow)[ACH], int e, int nt, int N, int I,
                                        DmaSrc &d) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint16_t *a = reinterpret_cast<const uint16_t *>(s.a);
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int r = dma_row<VT>(j);
    d.a[j] = a + arow[j] * s.a_ld + 8 * ((lane & 7) ^ ((r >> 1) & 7));
  }
  const int64_t slice = s.b_rows * s.b_cols;
  const uint8_t *codes = reinterpret_cast<const uint8_t *>(s.b) + e * (slice / 2);
  const uint8_t *scales = reinterpret_cast<const uint8_t *>(s.b_sc) + e * (slice / 16);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int64_t wr = b_row_of_col<EPI, BN>((2 * w + j) * 32 + (lane >> 1), nt, N, I);
    wr = wr < 0 ? 0 : wr;
    d.c[j] = codes + wr * (s.b_cols / 2) + 16 * (lane & 1);
  }
  int64_t wr = b_row_of_col<EPI, BN>(64 * w + lane, nt, N, I);
  wr = wr < 0 ? 0 : wr;
  d.s = scales + wr * (s.b_cols / 16);
}

// copies j < VT + 2 (A rows and codes) of the K step at k0 into stage st
template <int VT, class SM>
__device__ __forceinline__ void dma_ac(const DmaSrc &d, int j, int k0, const SM &sm, int st) {
  const uint32_t w = wave_id();
  if (j < VT)
    dma_b128(d.a[j] + k0, lds_a(sm, st) + (8 * VT * w + 8 * j) * BK * 2);
  else
    dma_b128(d.c[j - VT] + k0 / 2, lds_b(sm, st) + (2 * w + j - VT) * 1024);
}

// copy number j (0..VT+2) of the K step at k0 into stage st: A rows (j < VT), codes, scales
template <int VT, class SM>
__device__ __forceinline__ void dma_one(const DmaSrc &d, int j, int k0, const SM &sm, int st) {
  const uint32_t w = wave_id();
  if (j < VT + 2)
    dma_ac<VT>(d, j, k0, sm, st);
  else
    dma_b32(d.s + k0 / 16, lds_s(sm, st) + 256 * w);
}

// Scale groups (the few-rows configuration): the E4M3 scales (NF4: FP32 absmax) of four
// consecutive K steps, 16 bytes of one weight row, go to LDS with one 16-byte copy lane
// per column instead of one 4-byte copy per column and step, so a quarter of the copy
// instructions carry the scales, and each touches a column's cache line once per four
// steps.  The group of step ks lives in buffer (ks / 4) % NSG; the last group of a K
// range is shifted back to end at the row's end (K >= 256, so that it starts >= 0).
template <class SM>
__device__ __forceinline__ uint32_t lds_sg(const SM &sm, int buf) {
  return smem_u32(sm) + (uint32_t)offsetof(SM, sg) + (uint32_t)buf * (uint32_t)sizeof(sm.sg[0]);
}
__device__ __forceinline__ int sg_first(int g, int nk) { return min(4 * g, nk - 4); }
// the group that starts at the K step at k0
template <class SM>
__device__ __forceinline__ void dma_sg(const DmaSrc &d, int k0, int nk, const SM &sm) {
  const int g = k0 / (4 * BK);
  dma_b128(d.s + 4 * sg_first(g, nk), lds_sg(sm, g % SM::NSG) + 1024 * wave_id());
}
// the scale word of column 0 for step ks (column c at index 4 c)
template <class SM>
__device__ __forceinline__ const uint32_t *sg_words(const SM &sm, int ks, int nk) {
  const int g = ks >> 2;
  return sm.sg[g % SM::NSG] + (ks - sg_first(g, nk));
}

// copy j (0 .. VT+2) of the K step at k0: A rows (j < VT), codes (two), then the scale
// word, or with scale groups the group's copy, issued with the group's first step only
template <int VT, bool SG, class SM>
__device__ __forceinline__ void dma_any(const DmaSrc &d, int j, int k0, int nk, const SM &sm, int st) {
  if constexpr (SG) {
    if (j < VT + 2)
      dma_ac<VT>(d, j, k0, sm, st);
    else if (((k0 / BK) & 3) == 0)
      dma_sg(d, k0, nk, sm);
  } else {
    dma_one<VT>(d, j, k0, sm, st);
  }
}

// Where the VT + 3 copies of step ks+2 are issued inside step ks: the VT copies of A
// rows spread over the MFMA pairs of slices 0-2 (position 8 kk + tm), the code and
// scale copies in slice 3, so the four waves' copies do not queue up behind each
// other.  Stage (ks+2) % 3 was last read in step ks-1, so any point of step ks may
// write it.  The A copies come before the wait in slice 3, which lets exactly those
// (VT of them) stay in flight.  -1: none here.
template <int VT>
__device__ __forceinline__ constexpr int dma_slot(int kk, int tm) {
  if (kk < 3) {
    for (int j = 0; j < VT; ++j)
      if ((24 * j) / VT == 8 * kk + tm) return j;
    return -1;
  }
  return tm == 1 ? VT : (tm == 4 ? VT + 1 : (tm == 7 ? VT + 2 : -1));
}

__device__ __forceinline__ bf16x8 a_frag(const uint16_t *As, int kk, int row, int lane) {
  return *reinterpret_cast<const bf16x8 *>(As + a_off(row + (lane & 31), 4 * (lane >> 5) + kk));
}

// raw codes and scale words of this lane's weight columns (LDS reads only)
struct BRaw {
  u32x4 c[TN];
  uint32_t sw[TN];
};

// SST: dwords between the scale words of consecutive columns
template <int SST = 1>
__device__ __forceinline__ void b_raw(const uint8_t *Bs, const uint32_t *Ss, int wn, int lane, BRaw &r) {
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int col = wn * TN * 32 + tn * 32 + (lane & 31);
    r.c[tn] = *reinterpret_cast<const u32x4 *>(Bs + col * 32 + 16 * (lane >> 5));
    r.sw[tn] = Ss[col * SST];
  }
}

__device__ __forceinline__ void b_cook(const BRaw &r, int lane, BCodes &b) {
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    b.c[tn] = r.c[tn];
    const uint32_t sw = r.sw[tn] >> (16 * (lane >> 5));  // blocks 2g, 2g+1
    b.s[tn][0] = e4m3_hw<0>(sw);
    b.s[tn][1] = e4m3_hw<1>(sw);
  }
}

// NF4: the scale word of a column is its FP32 absmax for the K step (one 64-block)
__device__ __forceinline__ void b_cook_nf4(const BRaw &r, int tn, BCodes &b) {
  b.c[tn] = r.c[tn];
  nf4_table(__uint_as_float(r.sw[tn]), b.lo[tn], b.hi[tn]);
}

// bf16 pair p (0..3) of column tile tn's fragment of slice kk
__device__ __forceinline__ uint32_t dec_pair(const BCodes &b, int tn, int kk, int p) {
  const uint32_t c = b.c[tn][kk];
  f32x2 v;
  if (p == 0)
    v = fp4pair<0>(c, b.s[tn][kk >> 1]);
  else if (p == 1)
    v = fp4pair<1>(c, b.s[tn][kk >> 1]);
  else if (p == 2)
    v = fp4pair<2>(c, b.s[tn][kk >> 1]);
  else
    v = fp4pair<3>(c, b.s[tn][kk >> 1]);
  return pack_exact(v.x, v.y);
}

__device__ __forceinline__ void mfma1(const bf16x8 &a, const u32x4 &b, f32x16 &acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), a, acc, 0, 0, 0);
}

#define FQ_PIN() __builtin_amdgcn_sched_barrier(0)

// One K step.  On entry af[0] / bf[0] hold slice 0 of stage `cur` and bc its codes.
// DMA: issue the copies of the step at k2 into stage n2.  NEXT: a following step
// exists (stage nx), whose slice 0 is loaded into af[0] / bf[0] at the end; before
// reading it the wave lets WV of its copies stay in flight (those of later steps).
// TMA: row tiles of the accumulator (VT <= TMA of them are valid).
// SG: scale groups (nk: K steps of the segment; sgn: the scale words of the next step)
template <int VT, bool DMA, bool NEXT, int WF, int WV, int TMA, bool SG = false, class SM>
__device__ __forceinline__ void step_q4(SM &sm, int cur, int nx, int n2, int k2, const DmaSrc &d, int wn, int row0,
                                        int lane, bf16x8 (&af)[2][TMA], u32x4 (&bf)[2][TN], BCodes &bc,
                                        f32x16 (&acc)[TMA][TN], int nk = 0, const uint32_t *sgn = nullptr) {
  const uint16_t *As = sm.a[cur];
  NF4Tmp nt;
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    const int c = kk & 1, n = c ^ 1;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if (tm < VT) mfma1(af[c][tm], bf[c][0], acc[tm][0]);
      if (tm < VT) af[n][tm] = a_frag(As, kk + 1, row0 + 32 * tm, lane);
      if (DMA && dma_slot<VT>(kk, tm) >= 0) dma_any<VT, SG>(d, dma_slot<VT>(kk, tm), k2, nk, sm, n2);
      FQ_PIN();
      if (tm < VT) mfma1(af[c][tm], bf[c][1], acc[tm][1]);
      if constexpr (WF == WF_NVFP4) {
        bf[n][tm >> 2][tm & 3] = dec_pair(bc, tm >> 2, kk + 1, tm & 3);
      } else {
        // the four parts of column tile tm / 4's slice kk+1
        if ((tm & 3) == 0) nf4_step<0>(bc, tm >> 2, kk + 1, nt, bf[n][tm >> 2]);
        if ((tm & 3) == 1) nf4_step<1>(bc, tm >> 2, kk + 1, nt, bf[n][tm >> 2]);
        if ((tm & 3) == 2) nf4_step<2>(bc, tm >> 2, kk + 1, nt, bf[n][tm >> 2]);
        if ((tm & 3) == 3) nf4_step<3>(bc, tm >> 2, kk + 1, nt, bf[n][tm >> 2]);
      }
      FQ_PIN();
    }
  }
  // slice 3: its MFMAs around the step boundary, then the next step's slice 0
  BRaw raw;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    if (tm < VT) mfma1(af[1][tm], bf[1][0], acc[tm][0]);
    if (NEXT && tm >= 2 && tm - 2 < VT) af[0][tm - 2] = a_frag(sm.a[nx], 0, row0 + 32 * (tm - 2), lane);
    if (NEXT && tm == 7) {
      if constexpr (VT > 6) af[0][6] = a_frag(sm.a[nx], 0, row0 + 192, lane);
      if constexpr (VT > 7) af[0][7] = a_frag(sm.a[nx], 0, row0 + 224, lane);
    }
    FQ_PIN();
    if (tm < VT) mfma1(af[1][tm], bf[1][1], acc[tm][1]);
    if (NEXT && tm == 0) {
      // stage nx has landed for every wave, and every wave is done reading stage
      // cur (its last reads were issued in slice 2 and are drained here), so the
      // next step may copy into it
      FQ_PIN();
      wait_vm<WV>();
      barrier_lds();
      FQ_PIN();
      if constexpr (SG)
        b_raw<4>(sm.b[nx], sgn, wn, lane, raw);
      else
        b_raw(sm.b[nx], sm.s[nx], wn, lane, raw);
    }
    if (DMA && dma_slot<VT>(3, tm) >= 0) dma_any<VT, SG>(d, dma_slot<VT>(3, tm), k2, nk, sm, n2);
    if constexpr (WF == WF_NVFP4) {
      if (NEXT && tm == 3) b_cook(raw, lane, bc);
      if (NEXT && tm >= 4) {
        const int q = 2 * (tm - 4);  // pairs q, q+1 of slice 0
        bf[0][q >> 2][q & 3] = dec_pair(bc, q >> 2, 0, q & 3);
        bf[0][(q + 1) >> 2][(q + 1) & 3] = dec_pair(bc, (q + 1) >> 2, 0, (q + 1) & 3);
      }
    } else {
      // tables of column tiles 0 and 1, then the four parts of each one's slice 0
      if (NEXT && tm == 3) b_cook_nf4(raw, 0, bc);
      if (NEXT && tm == 4) nf4_step<0>(bc, 0, 0, nt, bf[0][0]);
      if (NEXT && tm == 5) {
        b_cook_nf4(raw, 1, bc);
        nf4_step<1>(bc, 0, 0, nt, bf[0][0]);
      }
      if (NEXT && tm == 6) {
        nf4_step<2>(bc, 0, 0, nt, bf[0][0]);
        nf4_step<3>(bc, 0, 0, nt, bf[0][0]);
        nf4_step<0>(bc, 1, 0, nt, bf[0][1]);
      }
      if (NEXT && tm == 7) {
        nf4_step<1>(bc, 1, 0, nt, bf[0][1]);
        nf4_step<2>(bc, 1, 0, nt, bf[0][1]);
        nf4_step<3>(bc, 1, 0, nt, bf[0][1]);
      }
    }
    FQ_PIN();
  }
}

// Copies a wave has in flight after those of a K step: the waits below count L later
// steps as L sets of VT A-row copies and two code copies (and the scale word without
// scale groups), leaving out scale groups, which only makes a wait longer.
template <int VT, bool SG>
__device__ __forceinline__ constexpr int later_copies(int L) {
  return L * (VT + (SG ? 2 : 3));
}

// The last steps of the K loop, which issue no copies: tail step J (of D) waits until
// the copies of at most D - 2 - J later steps are in flight.  Steps J < j0 do not
// exist (K shorter than D steps).  (The step of tail step J is nk - D + J.)
template <int VT, int WF, int TMA, bool SG, int J, int D, class SM>
__device__ __forceinline__ void tail_q4(SM &sm, int &cur, int j0, int nk, const DmaSrc &d, int wn, int row0, int lane,
                                        bf16x8 (&af)[2][TMA], u32x4 (&bf)[2][TN], BCodes &bc,
                                        f32x16 (&acc)[TMA][TN]) {
  if constexpr (J < D) {
    if (J >= j0) {
      const int nx = cur == SM::NS - 1 ? 0 : cur + 1;
      constexpr bool kNext = J + 1 < D;
      const uint32_t *sgn = nullptr;
      if constexpr (SG && kNext) sgn = sg_words(sm, nk - D + J + 1, nk);
      step_q4<VT, false, kNext, WF, kNext ? later_copies<VT, SG>(D - 2 - J) : 0, TMA, SG>(
          sm, cur, nx, 0, 0, d, wn, row0, lane, af, bf, bc, acc, nk, sgn);
      cur = nx;
    }
    tail_q4<VT, WF, TMA, SG, J + 1, D>(sm, cur, j0, nk, d, wn, row0, lane, af, bf, bc, acc);
  }
}

// Segment 1: the K loop over the 4-bit weight with copies issued D = NS - 1 steps
// ahead.  SG: scale groups (the segment's K is then at least 256).
template <int EPI, int VT, int WF, int TMA, bool SG = false, class SM>
__device__ __forceinline__ void seg_q4_direct(const Seg &s, int e, int nt, int N, int I, const int64_t (&arow)[ACH],
                                              SM &sm, f32x16 (&acc)[TMA][TN]) {
  constexpr int NDMA = VT + 3, D = SM::NS - 1;
  static_assert(D >= 2 && later_copies<VT, SG>(D) + 1 < 64, "copies in flight fit the wait counter");
  static_assert(!SG || D <= 4 * (SM::NSG - 1), "a scale group is written after its buffer's last reader");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wn = wid % WNG, row0 = (wid / WNG) * TMA * 32;
  const int nk = s.K / BK;
  DmaSrc d;
  dma_src<EPI, VT>(s, arow, e, nt, N, I, d);
  // prologue: stage j <- step j for j < D; wait for stage 0 only
#pragma unroll
  for (int j = 0; j < NDMA; ++j) dma_any<VT, SG>(d, j, 0, nk, sm, 0);
  if (nk >= D) {
#pragma unroll
    for (int st = 1; st < D; ++st)
#pragma unroll
      for (int j = 0; j < NDMA; ++j) dma_any<VT, SG>(d, j, st * BK, nk, sm, st);
    wait_vm<later_copies<VT, SG>(D - 1)>();
  } else {
    if constexpr (D > 2) {
      for (int st = 1; st < nk; ++st)
#pragma unroll
        for (int j = 0; j < NDMA; ++j) dma_any<VT, SG>(d, j, st * BK, nk, sm, st);
    }
    wait_vm<0>();
  }
  barrier_lds();
  bf16x8 af[2][TMA];
  u32x4 bf[2][TN];
  BCodes bc;
  {
    BRaw raw;
    if constexpr (SG)
      b_raw<4>(sm.b[0], sg_words(sm, 0, nk), wn, lane, raw);
    else
      b_raw(sm.b[0], sm.s[0], wn, lane, raw);
#pragma unroll
    for (int tm = 0; tm < VT; ++tm) af[0][tm] = a_frag(sm.a[0], 0, row0 + 32 * tm, lane);
    if constexpr (WF == WF_NVFP4) {
      b_cook(raw, lane, bc);
#pragma unroll
      for (int q = 0; q < 4 * TN; ++q) bf[0][q >> 2][q & 3] = dec_pair(bc, q >> 2, 0, q & 3);
    } else {
      NF4Tmp t;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        b_cook_nf4(raw, tn, bc);
        nf4_step<0>(bc, tn, 0, t, bf[0][tn]);
        nf4_step<1>(bc, tn, 0, t, bf[0][tn]);
        nf4_step<2>(bc, tn, 0, t, bf[0][tn]);
        nf4_step<3>(bc, tn, 0, t, bf[0][tn]);
      }
    }
  }
  int cur = 0, ks = 0;
  for (; ks + D < nk; ++ks) {
    const int nx = cur == SM::NS - 1 ? 0 : cur + 1;
    // stage of step ks + D, last read in step ks - 1
    const int nd = D == 2 ? (nx == SM::NS - 1 ? 0 : nx + 1) : (cur == 0 ? SM::NS - 1 : cur - 1);
    const uint32_t *sgn = nullptr;
    if constexpr (SG) sgn = sg_words(sm, ks + 1, nk);
    step_q4<VT, true, true, WF, later_copies<VT, SG>(D - 2) + VT, TMA, SG>(sm, cur, nx, nd, (ks + D) * BK, d, wn, row0,
                                                                       lane, af, bf, bc, acc, nk, sgn);
    cur = nx;
  }
  if constexpr (D == 2) {
    if (ks + 1 < nk) {
      const int nx = cur == SM::NS - 1 ? 0 : cur + 1;
      const uint32_t *sgn = nullptr;
      if constexpr (SG) sgn = sg_words(sm, ks + 1, nk);
      step_q4<VT, false, true, WF, 0, TMA, SG>(sm, cur, nx, 0, 0, d, wn, row0, lane, af, bf, bc, acc, nk, sgn);
      cur = nx;
    }
    step_q4<VT, false, false, WF, 0, TMA, SG>(sm, cur, 0, 0, 0, d, wn, row0, lane, af, bf, bc, acc, nk, nullptr);
  } else {
    tail_q4<VT, WF, TMA, SG, 0, D>(sm, cur, nk >= D ? 0 : D - nk, nk, d, wn, row0, lane, af, bf, bc, acc);
  }
  __syncthreads();  // the stages are reused by the next segment
}
#undef FQ_PIN

// Segment 2 (LoRA up-projection): A = hi/lo pair rows through registers (k >= K
// zeroed), B = the bf16 LoRA matrix [N rows][kmod], fragments loaded straight
// from global memory (it is small and stays in L2).  The loads of step ks+1 are
// issued before the MFMAs of step ks, alternating between two LDS A buffers, so
// the segment waits for global memory once, not once per slice.
template <int NC = ACH>
struct LoraRegs {
  ARegs<NC> a;
  bf16x8 b[4][TN];
};

template <int EPI, int NC>
__device__ __forceinline__ void lora_load(const Seg &s, const int64_t (&arow)[ACH], const uint16_t *bsrc,
                                          const int64_t (&wr)[TN], int ks, int lane, LoraRegs<NC> &r) {
  a_load<A_ROWS, true, NC>(s, arow, ks * BK, r.a);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int kb = (ks * BK + 32 * (lane >> 5) + 8 * kk) % s.kmod;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) r.b[kk][tn] = *reinterpret_cast<const bf16x8 *>(bsrc + wr[tn] * s.b_cols + kb);
  }
}

// TMA row tiles of 32 (arow: the A rows of this thread's TMA chunks, a_row<TMA>)
template <int EPI, int TMA = TM, class SM>
__device__ __forceinline__ void seg_lora(const Seg &s, int e, int nt, int N, int I, const int64_t (&arow)[ACH],
                                         SM &sm, int vt, f32x16 (&acc)[TMA][TN]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wn = wid % WNG;
  const int row0 = (wid / WNG) * TMA * 32;
  const int nk = (s.K + BK - 1) / BK;
  const uint16_t *bsrc = reinterpret_cast<const uint16_t *>(s.b) + e * s.b_estride;
  int64_t wr[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    int64_t w = b_row_of_col<EPI, BN>(wn * TN * 32 + tn * 32 + (lane & 31), nt, N, I);
    wr[tn] = w < 0 ? 0 : w;
  }
  // the loads of the first two steps are in flight together (K = 2r: one wait, not two);
  // step ks + 2 is loaded into the registers step ks has finished with
  LoraRegs<TMA> r[2];
  lora_load<EPI>(s, arow, bsrc, wr, 0, lane, r[0]);
  if (nk > 1) lora_load<EPI>(s, arow, bsrc, wr, 1, lane, r[1]);
  for (int ks = 0; ks < nk; ks += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (ks + h >= nk) break;
      a_store<A_ROWS, TMA>(sm.a[h], r[h].a);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 af[TMA];
        a_frags<TMA>(sm.a[h], kk, row0, lane, af);
        mfmas<VT_DYN, TMA>(af, r[h].b[kk], vt, acc);
      }
      if (ks + h + 2 < nk) lora_load<EPI>(s, arow, bsrc, wr, ks + h + 2, lane, r[h]);
    }
  }
  __syncthreads();
}

// ---- dgrad over the rowwise NVFP4 weight, read transposed ----
// dX[r, h] = sum_j dH[r, j] DQ(W)[j, h]: the contraction runs over the weight's rows
// j, while its 16-element scale blocks run along h.  Each K step copies 64 weight
// rows of the tile's 256 columns (64 x 128 code bytes, 16-byte chunk c of row j at
// position c ^ (j & 7)) and their 64 x 16 scale bytes to LDS as they are stored.
// The gfx950 4-bit transposing LDS read then hands every lane of a 16-lane group
// one column (= one scale block) with 16 consecutive rows of codes; the 16 scales
// of those rows are regrouped per block in a small per-wave LDS area.  A step's k
// order: slice kk = 2m + t, lane group g covers rows 32m + 16g + 8t .. +8, for the
// A fragments and the weight alike.

struct DmaSrcD {
  const uint16_t *a[ACH];
  const uint8_t *c[2];
  const uint8_t *s;
  int64_t cstride, sstride;  // bytes per weight row: codes, scales
};

template <int VT>
__device__ __forceinline__ void dma_src_d(const Seg &s, const int64_t (&arow)[ACH], int e, int nt, int N,
                                          DmaSrcD &d) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint16_t *a = reinterpret_cast<const uint16_t *>(s.a);
#pragma unroll
  for (int j = 0; j < VT; ++j) {
    const int r = dma_row<VT>(j);
    d.a[j] = a + arow[j] * s.a_ld + 8 * ((lane & 7) ^ ((r >> 1) & 7));
  }
  const int64_t slice = s.b_rows * s.b_cols;
  d.cstride = s.b_cols / 2;
  d.sstride = s.b_cols / 16;
  const uint8_t *codes = reinterpret_cast<const uint8_t *>(s.b) + e * (slice / 2);
  const uint8_t *scales = reinterpret_cast<const uint8_t *>(s.b_sc) + e * (slice / 16);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * w + 8 * j + (lane >> 3);
    int c = (lane & 7) ^ (row & 7);                 // the chunk that lands at this lane's position
    if (nt * BN + 32 * c >= N) c = 0;               // columns past N: any valid bytes (dropped)
    d.c[j] = codes + row * d.cstride + nt * (BN / 2) + 16 * c;
  }
  const int row = 16 * w + (lane >> 2);
  int q = lane & 3;
  if (nt * (BN / 16) + 4 * q >= N / 16) q = 0;
  d.s = scales + row * d.sstride + nt * (BN / 16) + 4 * q;
}

// copy j (0..VT+2) of the K step at k0 into stage st: A rows (j < VT), codes, scales
template <int VT, class SM>
__device__ __forceinline__ void dma_one_d(const DmaSrcD &d, int j, int k0, const SM &sm, int st) {
  const uint32_t w = wave_id();
  if (j < VT)
    dma_b128(d.a[j] + k0, lds_a(sm, st) + (8 * VT * w + 8 * j) * BK * 2);
  else if (j < VT + 2)
    dma_b128(d.c[j - VT] + k0 * d.cstride, lds_b(sm, st) + (16 * w + 8 * (j - VT)) * 128);
  else
    dma_b32(d.s + k0 * d.sstride, lds_s(sm, st) + 256 * w);
}

__device__ __forceinline__ bf16x8 a_frag_d(const uint16_t *As, int kk, int row, int lane) {
  const int c = 4 * (kk >> 1) + 2 * (lane >> 5) + (kk & 1);
  return *reinterpret_cast<const bf16x8 *>(As + a_off(row + (lane & 31), c));
}

typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// this lane's codes of column tile tn for rows 32m + 16g .. +16 (nibble i = row +i)
__device__ __forceinline__ i32x2 codes_tr(const uint8_t *Bs, int wn, int tn, int m, int lane) {
  const int q = lane >> 4, row = 32 * m + 16 * (q >> 1) + (lane & 15);
  const int c = 2 * wn + tn;  // 16-byte chunk of the wave's column tile; half q & 1
  const uint8_t *p = Bs + row * 128 + 16 * (c ^ (row & 7)) + 8 * (q & 1);
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)(p));
}

struct DRaw {
  i32x2 c[TN][2];   // codes per column tile and row half-step m
  u32x4 s[TN][2];   // the 16 scale bytes of those rows, in row order
};

// bf16 pair p of column tile tn's fragment of slice kk
__device__ __forceinline__ uint32_t dec_pair_d(const DRaw &r, int tn, int kk, int p) {
  const int m = kk >> 1, t = kk & 1;
  const uint32_t c = (uint32_t)r.c[tn][m][t];
  const uint32_t sw = r.s[tn][m][2 * t + (p >> 1)];
  f32x2 v;
  if (p == 0)
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  else if (p == 1)
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
  else if (p == 2)
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
  else
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
  const f32x2 sc = (p & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)sw, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)sw, false);
  v = v * sc;  // exact: <= 6 significant bits
  return pack_exact(v.x, v.y);
}

#define FQ_PIN() __builtin_amdgcn_sched_barrier(0)

template <int VT, bool DMA, bool NEXT, int TMA, class SM>
__device__ __forceinline__ void step_dq(SM &sm, int cur, int nx, int n2, int k2, const DmaSrcD &d, int wn, int row0,
                                        int lane, bf16x8 (&af)[2][TMA], u32x4 (&bf)[2][TN], DRaw &raw,
                                        f32x16 (&acc)[TMA][TN]) {
  const uint16_t *As = sm.a[cur];
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    const int c = kk & 1, n = c ^ 1;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if (tm < VT) mfma1(af[c][tm], bf[c][0], acc[tm][0]);
      if (tm < VT) af[n][tm] = a_frag_d(As, kk + 1, row0 + 32 * tm, lane);
      if (DMA && dma_slot<VT>(kk, tm) >= 0) dma_one_d<VT>(d, dma_slot<VT>(kk, tm), k2, sm, n2);
      FQ_PIN();
      if (tm < VT) mfma1(af[c][tm], bf[c][1], acc[tm][1]);
      bf[n][tm >> 2][tm & 3] = dec_pair_d(raw, tm >> 2, kk + 1, tm & 3);
      FQ_PIN();
    }
  }
  // slice 3 around the step boundary; then slice 0 of the next step
  uint32_t sw = 0;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    if (tm < VT) mfma1(af[1][tm], bf[1][0], acc[tm][0]);
    if (NEXT) {
      if (tm == 1 || tm == 4 || tm == 5) {
        const int i = tm == 1 ? 0 : (tm == 4 ? 4 : 6);
        if (i < VT) af[0][i] = a_frag_d(sm.a[nx], 0, row0 + 32 * i, lane);
        if (i + 1 < VT) af[0][i + 1] = a_frag_d(sm.a[nx], 0, row0 + 32 * (i + 1), lane);
      }
      if (tm == 2 && 2 < VT) af[0][2] = a_frag_d(sm.a[nx], 0, row0 + 64, lane);
      if (tm == 3 && 3 < VT) af[0][3] = a_frag_d(sm.a[nx], 0, row0 + 96, lane);
      if (tm == 2) {
        // regroup this wave's 4 x 64 scale bytes per column block
        uint8_t *t = sm.t[wn];
#pragma unroll
        for (int b = 0; b < 4; ++b) t[64 * b + lane] = (uint8_t)(sw >> (8 * b));
      }
      if (tm == 3) {
        const uint8_t *t = sm.t[wn];
        const int q = lane >> 4;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            raw.s[tn][m] = *reinterpret_cast<const u32x4 *>(t + 64 * (2 * tn + (q & 1)) + 32 * m + 16 * (q >> 1));
      }
    }
    FQ_PIN();
    if (tm < VT) mfma1(af[1][tm], bf[1][1], acc[tm][1]);
    if (DMA && dma_slot<VT>(3, tm) >= 0) dma_one_d<VT>(d, dma_slot<VT>(3, tm), k2, sm, n2);
    if (NEXT && tm == 0) {
      // stage nx has landed for every wave and every wave is done reading stage cur
      FQ_PIN();
      if (DMA)
        wait_vm<VT>();
      else
        wait_vm<0>();
      barrier_lds();
      FQ_PIN();
      sw = sm.s[nx][16 * lane / 4 + wn];  // scale dword (row lane, blocks 4wn .. 4wn+3)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int m = 0; m < 2; ++m) raw.c[tn][m] = codes_tr(sm.b[nx], wn, tn, m, lane);
    }
    if (NEXT && tm >= 6) {
      const int tn = tm - 6;
#pragma unroll
      for (int q = 0; q < 4; ++q) bf[0][tn][q] = dec_pair_d(raw, tn, 0, q);
    }
    FQ_PIN();
  }
}

template <int EPI, int VT, int TMA, class SM>
__device__ __forceinline__ void seg_dq_direct(const Seg &s, int e, int nt, int N, const int64_t (&arow)[ACH], SM &sm,
                                              f32x16 (&acc)[TMA][TN]) {
  static_assert(SM::NS == 3, "the copies run two K steps ahead through three stages");
  constexpr int NDMA = VT + 3;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wn = wid % WNG, row0 = (wid / WNG) * TMA * 32;
  const int nk = s.K / BK;
  DmaSrcD d;
  dma_src_d<VT>(s, arow, e, nt, N, d);
#pragma unroll
  for (int j = 0; j < NDMA; ++j) dma_one_d<VT>(d, j, 0, sm, 0);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) dma_one_d<VT>(d, j, BK, sm, 1);
    wait_vm<NDMA>();
  } else {
    wait_vm<0>();
  }
  barrier_lds();
  bf16x8 af[2][TMA];
  u32x4 bf[2][TN];
  DRaw raw;
  {
    const uint32_t sw = sm.s[0][16 * lane / 4 + wn];
    uint8_t *t = sm.t[wn];
#pragma unroll
    for (int b = 0; b < 4; ++b) t[64 * b + lane] = (uint8_t)(sw >> (8 * b));
    const int q = lane >> 4;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        raw.c[tn][m] = codes_tr(sm.b[0], wn, tn, m, lane);
        raw.s[tn][m] = *reinterpret_cast<const u32x4 *>(t + 64 * (2 * tn + (q & 1)) + 32 * m + 16 * (q >> 1));
      }
#pragma unroll
    for (int tm = 0; tm < VT; ++tm) af[0][tm] = a_frag_d(sm.a[0], 0, row0 + 32 * tm, lane);
#pragma unroll
    for (int q2 = 0; q2 < 4 * TN; ++q2) bf[0][q2 >> 2][q2 & 3] = dec_pair_d(raw, q2 >> 2, 0, q2 & 3);
  }
  int cur = 0, ks = 0;
  for (; ks + 2 < nk; ++ks) {
    const int nx = cur == NST - 1 ? 0 : cur + 1;
    const int n2 = nx == NST - 1 ? 0 : nx + 1;
    step_dq<VT, true, true, TMA>(sm, cur, nx, n2, (ks + 2) * BK, d, wn, row0, lane, af, bf, raw, acc);
    cur = nx;
  }
  if (ks + 1 < nk) {
    const int nx = cur == NST - 1 ? 0 : cur + 1;
    step_dq<VT, false, true, TMA>(sm, cur, nx, 0, 0, d, wn, row0, lane, af, bf, raw, acc);
    cur = nx;
  }
  step_dq<VT, false, false, TMA>(sm, cur, 0, 0, 0, d, wn, row0, lane, af, bf, raw, acc);
  __syncthreads();  // the stages are reused by the next segment
}

// ---- dgrad over NF4 weights ----
// NF4 blocks run along the weight's columns, which are the dgrad's output, so along the
// contraction every value has its own absmax and the lane-wise table of the forward does
// not apply.  Each K step's weight rows are decoded row-major instead, one slice (16 rows)
// ahead of the MFMAs, into a per-wave bf16 tile in LDS (64 rows x the wave's 64 columns,
// row stride DQS), and the B fragments are read from it with the 16-bit transposing LDS
// read.  Lane 4r+q decodes row r's columns 16q..16q+15: the wave's 64 columns are one NF4
// block, so the four lanes of a row share one absmax and build its table together (each
// computes four entries, gathered with quad DPP broadcasts).  k order: slice kk holds rows
// 16kk..16kk+15 and lane group g rows 16kk+8g..+8, for the A fragments and the weight alike.

// quad-shared table: lane q of a quad computes entries 4q..4q+3 from lv = levels[4q..4q+3]
__device__ __forceinline__ void nf4_table_quad(float a, const float4 &lv, uint32_t (&lo)[4], uint32_t (&hi)[4]) {
  const int pa = (int)pack_bf16_rne(lv.x * a, lv.y * a), pb = (int)pack_bf16_rne(lv.z * a, lv.w * a);
  uint32_t pr[8];  // quad_perm(i, i, i, i): lane i of the quad to all four
  pr[0] = (uint32_t)__builtin_amdgcn_mov_dpp(pa, 0x00, 0xF, 0xF, true);
  pr[1] = (uint32_t)__builtin_amdgcn_mov_dpp(pb, 0x00, 0xF, 0xF, true);
  pr[2] = (uint32_t)__builtin_amdgcn_mov_dpp(pa, 0x55, 0xF, 0xF, true);
  pr[3] = (uint32_t)__builtin_amdgcn_mov_dpp(pb, 0x55, 0xF, 0xF, true);
  pr[4] = (uint32_t)__builtin_amdgcn_mov_dpp(pa, 0xAA, 0xF, 0xF, true);
  pr[5] = (uint32_t)__builtin_amdgcn_mov_dpp(pb, 0xAA, 0xF, 0xF, true);
  pr[6] = (uint32_t)__builtin_amdgcn_mov_dpp(pa, 0xFF, 0xF, 0xF, true);
  pr[7] = (uint32_t)__builtin_amdgcn_mov_dpp(pb, 0xFF, 0xF, 0xF, true);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = __builtin_amdgcn_perm(pr[2 * i + 1], pr[2 * i], 0x06040200u);
    hi[i] = __builtin_amdgcn_perm(pr[2 * i + 1], pr[2 * i], 0x07050301u);
  }
}

// a lane's share of one slice: its row's codes (16 columns) and absmax, the table, the pairs
struct DnRow {
  uint32_t c[2];
  float a;
  uint32_t lo[4], hi[4];
  NF4Tmp t;
  u32x4 o[2];
};

// codes and absmax of slice kk's row for this lane from stage (codes, absmax) in LDS
__device__ __forceinline__ void dn_load(const uint8_t *Bs, const uint32_t *Ss, int wn, int kk, int lane, DnRow &r) {
  const int row = 16 * kk + (lane >> 2), q = lane & 3;
  const int c = 2 * wn + (q >> 1);
  const i32x2 v = *reinterpret_cast<const i32x2 *>(Bs + row * 128 + 16 * (c ^ (row & 7)) + 8 * (q & 1));
  r.c[0] = (uint32_t)v[0];
  r.c[1] = (uint32_t)v[1];
  r.a = __uint_as_float(Ss[row * 4 + wn]);
}

// part p (0..5) of decoding and storing this lane's 16 values of slice kk into the wave's tile
template <int P>
__device__ __forceinline__ void dn_part(DnRow &r, const float4 &lv, uint16_t *Dq, int kk, int lane) {
  if constexpr (P == 0) {
    nf4_table_quad(r.a, lv, r.lo, r.hi);
  } else if constexpr (P == 1) {
    nf4_part<0>(r.c[0], r.lo, r.hi, r.t, r.o[0]);
    nf4_part<1>(r.c[0], r.lo, r.hi, r.t, r.o[0]);
  } else if constexpr (P == 2) {
    nf4_part<2>(r.c[0], r.lo, r.hi, r.t, r.o[0]);
    nf4_part<3>(r.c[0], r.lo, r.hi, r.t, r.o[0]);
    nf4_part<0>(r.c[1], r.lo, r.hi, r.t, r.o[1]);
  } else if constexpr (P == 3) {
    nf4_part<1>(r.c[1], r.lo, r.hi, r.t, r.o[1]);
    nf4_part<2>(r.c[1], r.lo, r.hi, r.t, r.o[1]);
    nf4_part<3>(r.c[1], r.lo, r.hi, r.t, r.o[1]);
    uint16_t *dst = Dq + (16 * kk + (lane >> 2)) * DQS + 16 * (lane & 3);
    *reinterpret_cast<u32x4 *>(dst) = r.o[0];
    *reinterpret_cast<u32x4 *>(dst + 8) = r.o[1];
  }
}

__device__ __forceinline__ bf16x8 a_frag_n(const uint16_t *As, int kk, int row, int lane) {
  return *reinterpret_cast<const bf16x8 *>(As + a_off(row + (lane & 31), 2 * kk + (lane >> 5)));
}


// One K step of the NF4 dgrad.  On entry af[0] / bf[0] hold slice 0 of stage cur.  In each
// slice, after its MFMA pairs: the next slice's rows are decoded (from stage cur, or for the
// next step's slice 0 from stage nx after the step barrier), written to the wave's tile and
// read back transposed as the next slice's B fragments.
template <int VT, bool DMA, bool NEXT>
__device__ __forceinline__ void step_dn(Smem &sm, int cur, int nx, int n2, int k2, const DmaSrcD &d, int wn, int row0,
                                        int lane, const float4 &lv, bf16x8 (&af)[2][TM], u32x4 (&bf)[2][TN],
                                        f32x16 (&acc)[TM][TN]) {
  const uint16_t *As = sm.a[cur];
  uint16_t *Dq = sm.dq[wn];
  DnRow r;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int c = kk & 1, n = c ^ 1;
    const bool last = kk == 3;
    const int kn = last ? 0 : kk + 1;  // the slice decoded and loaded here
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if (tm < VT) mfma1(af[c][tm], bf[c][0], acc[tm][0]);
      if (!last) {
        if (tm < VT) af[n][tm] = a_frag_n(As, kn, row0 + 32 * tm, lane);
      } else if (NEXT && tm >= 1) {
        if (tm - 1 < VT) af[n][tm - 1] = a_frag_n(sm.a[nx], 0, row0 + 32 * (tm - 1), lane);
        if (tm == 7 && 7 < VT) af[n][7] = a_frag_n(sm.a[nx], 0, row0 + 224, lane);
      }
      if (DMA && dma_slot<VT>(kk, tm) >= 0) dma_one_d<VT>(d, dma_slot<VT>(kk, tm), k2, sm, n2);
      FQ_PIN();
      if (tm < VT) mfma1(af[c][tm], bf[c][1], acc[tm][1]);
      if (last && tm == 0 && NEXT) {
        // stage nx has landed for every wave, and every wave is done with stage cur
        FQ_PIN();
        if (DMA)
          wait_vm<VT>();
        else
          wait_vm<0>();
        barrier_lds();
        FQ_PIN();
      }
      if (!last || NEXT) {
        if (tm == 0) dn_load(last ? sm.b[nx] : sm.b[cur], last ? sm.s[nx] : sm.s[cur], wn, kn, lane, r);
        if (tm == 1) dn_part<0>(r, lv, Dq, kn, lane);
        if (tm == 2) dn_part<1>(r, lv, Dq, kn, lane);
        if (tm == 3) dn_part<2>(r, lv, Dq, kn, lane);
        if (tm == 4) dn_part<3>(r, lv, Dq, kn, lane);
        if (tm == 5) bf[n][0] = __builtin_bit_cast(u32x4, b_frag_trans_s<DQS>(Dq, 16 * kn, 0, lane));
        if (tm == 6) bf[n][1] = __builtin_bit_cast(u32x4, b_frag_trans_s<DQS>(Dq, 16 * kn, 32, lane));
      }
      FQ_PIN();
    }
  }
}

template <int EPI, int VT>
__device__ __forceinline__ void seg_dn_direct(const Seg &s, int e, int nt, int N, const int64_t (&arow)[ACH], Smem &sm,
                                              f32x16 (&acc)[TM][TN]) {
  constexpr int NDMA = VT + 3;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wn = wid % WNG, row0 = (wid / WNG) * TM * 32;
  const int nk = s.K / BK;
  const float4 lv = reinterpret_cast<const float4 *>(c_nf4)[lane & 3];
  DmaSrcD d;
  dma_src_d<VT>(s, arow, e, nt, N, d);
#pragma unroll
  for (int j = 0; j < NDMA; ++j) dma_one_d<VT>(d, j, 0, sm, 0);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) dma_one_d<VT>(d, j, BK, sm, 1);
    wait_vm<NDMA>();
  } else {
    wait_vm<0>();
  }
  barrier_lds();
  bf16x8 af[2][TM];
  u32x4 bf[2][TN];
  {
    uint16_t *Dq = sm.dq[wn];
    DnRow r;
    dn_load(sm.b[0], sm.s[0], wn, 0, lane, r);
    dn_part<0>(r, lv, Dq, 0, lane);
    dn_part<1>(r, lv, Dq, 0, lane);
    dn_part<2>(r, lv, Dq, 0, lane);
    dn_part<3>(r, lv, Dq, 0, lane);
    bf[0][0] = __builtin_bit_cast(u32x4, b_frag_trans_s<DQS>(Dq, 0, 0, lane));
    bf[0][1] = __builtin_bit_cast(u32x4, b_frag_trans_s<DQS>(Dq, 0, 32, lane));
#pragma unroll
    for (int tm = 0; tm < VT; ++tm) af[0][tm] = a_frag_n(sm.a[0], 0, row0 + 32 * tm, lane);
  }
  int cur = 0, ks = 0;
  for (; ks + 2 < nk; ++ks) {
    const int nx = cur == NST - 1 ? 0 : cur + 1;
    const int n2 = nx == NST - 1 ? 0 : nx + 1;
    step_dn<VT, true, true>(sm, cur, nx, n2, (ks + 2) * BK, d, wn, row0, lane, lv, af, bf, acc);
    cur = nx;
  }
  if (ks + 1 < nk) {
    const int nx = cur == NST - 1 ? 0 : cur + 1;
    step_dn<VT, false, true>(sm, cur, nx, 0, 0, d, wn, row0, lane, lv, af, bf, acc);
    cur = nx;
  }
  step_dn<VT, false, false>(sm, cur, 0, 0, 0, d, wn, row0, lane, lv, af, bf, acc);
  __syncthreads();  // the stages are reused by the next segment
}
#undef FQ_PIN

// Segment 2 of the dgrad (LoRA): A = hi/lo pair rows (k >= K zeroed), B = the bf16
// LoRA matrix [kmod rows][N cols] taken at row k mod kmod; its 64 x 256 tile is
// staged in natural layout (row stride BN + 8) and read with the 16-bit
// transposing LDS read.
constexpr int LSTR = BN + 8;

template <int NC = ACH>
__device__ __forceinline__ void lora_n_load(const Seg &s, const int64_t (&arow)[ACH], const uint16_t *bsrc, int nt,
                                            int N, int ks, ARegs<NC> &a, u32x4 (&bv)[8]) {
  const int tid = threadIdx.x;
  a_load<A_ROWS, true, NC>(s, arow, ks * BK, a);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + NTHR * i, row = c >> 5, col = nt * BN + 8 * (c & 31);
    const int kb = (ks * BK + row) % s.kmod;
    bv[i] = *reinterpret_cast<const u32x4 *>(bsrc + (int64_t)kb * s.b_cols + (col < N ? col : 0));
  }
}

// TMA row tiles of 32 (arow: the A rows of this thread's TMA chunks, a_row<TMA>); the
// LoRA-B tile sits from stage 1's A area on (SM::lora_b_fits: it fits the stages after it)
template <int TMA = TM, class SM>
__device__ __forceinline__ void seg_lora_n(const Seg &s, int e, int nt, int N, const int64_t (&arow)[ACH], SM &sm,
                                           int vt, f32x16 (&acc)[TMA][TN]) {
  static_assert(SM::lora_b_bytes >= BK * LSTR * 2, "LoRA tile fits the stages");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wn = wid % WNG, row0 = (wid / WNG) * TMA * 32;
  const int nk = (s.K + BK - 1) / BK;
  const uint16_t *bsrc = reinterpret_cast<const uint16_t *>(s.b) + e * s.b_estride;
  uint16_t *Bt = sm.a[1];
  ARegs<TMA> ar;
  u32x4 bv[8];
  lora_n_load<TMA>(s, arow, bsrc, nt, N, 0, ar, bv);
  for (int ks = 0; ks < nk; ++ks) {
    a_store<A_ROWS, TMA>(sm.a[0], ar);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + NTHR * i;
      *reinterpret_cast<u32x4 *>(Bt + (c >> 5) * LSTR + 8 * (c & 31)) = bv[i];
    }
    if (ks + 1 < nk) lora_n_load<TMA>(s, arow, bsrc, nt, N, ks + 1, ar, bv);  // lands during this step's MFMAs
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[TMA], bl[TN];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) bl[tn] = b_frag_trans_s<LSTR>(Bt, 16 * kk, wn * TN * 32 + tn * 32, lane);
#pragma unroll
      for (int tm = 0; tm < TMA; ++tm)
        af[tm] = *reinterpret_cast<const bf16x8 *>(sm.a[0] + a_off(row0 + tm * 32 + (lane & 31), 2 * kk + (lane >> 5)));
      mfmas<VT_DYN, TMA>(af, bl, vt, acc);
    }
    __syncthreads();
  }
}

template <int ASRC, int EPI, int WF = WF_NVFP4>
__global__ void __launch_bounds__(NTHR, 1) gemm_dgrad_q4(GemmParams p) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  // the tile prefix: 256-row tiles, less the remainder tiles the 64-row kernel takes
  auto toff = [&](int e) { return p.tile_off[e] - (p.tile_rem ? p.tile_rem[e] : 0); };
  const int total = toff(p.E) * p.NT;
  const int per = (total + 7) / 8;
  const int li = blockIdx.x >> 3;
  if (li >= per) return;
  const int L = (blockIdx.x & 7) * per + li;
  if (L >= total) return;
  const int mt = L / p.NT, nt = L % p.NT;
  int lo = 0, hi = p.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (toff(mid) <= mt)
      lo = mid;
    else
      hi = mid;
  }
  const int e = lo;
  const int rb = p.offsets[e];
  const int n_e = p.offsets[e + 1] - rb;
  const int m0 = (mt - toff(e)) * BM;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wn = wid % WNG, row0 = (wid / WNG) * TM * 32;
  const int rows_left = n_e - m0 - row0;
  const int vt = rows_left <= 0 ? 0 : (rows_left >= TM * 32 ? TM : (rows_left + 31) / 32);
  int64_t arow[ACH];
  f32x16 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tm][tn][v] = 0.0f;
  // row tiles rounded up to even counts; the copies cover the tile's 32 vt rows only
  const int vtu = __builtin_amdgcn_readfirstlane(vt);  // every wave starts at row 0: vt is the tile's
  if constexpr (WF == WF_NF4) {
    if (vtu > 6) {
      dma_rows<ASRC, 8>(p, rb, n_e, m0, arow);
      seg_dn_direct<EPI, 8>(p.s1, e, nt, p.N, arow, sm, acc);
    } else if (vtu > 4) {
      dma_rows<ASRC, 6>(p, rb, n_e, m0, arow);
      seg_dn_direct<EPI, 6>(p.s1, e, nt, p.N, arow, sm, acc);
    } else if (vtu > 2) {
      dma_rows<ASRC, 4>(p, rb, n_e, m0, arow);
      seg_dn_direct<EPI, 4>(p.s1, e, nt, p.N, arow, sm, acc);
    } else {
      dma_rows<ASRC, 2>(p, rb, n_e, m0, arow);
      seg_dn_direct<EPI, 2>(p.s1, e, nt, p.N, arow, sm, acc);
    }
  } else {
    if (vtu > 6) {
      dma_rows<ASRC, 8>(p, rb, n_e, m0, arow);
      seg_dq_direct<EPI, 8>(p.s1, e, nt, p.N, arow, sm, acc);
    } else if (vtu > 4) {
      dma_rows<ASRC, 6>(p, rb, n_e, m0, arow);
      seg_dq_direct<EPI, 6>(p.s1, e, nt, p.N, arow, sm, acc);
    } else if (vtu > 2) {
      dma_rows<ASRC, 4>(p, rb, n_e, m0, arow);
      seg_dq_direct<EPI, 4>(p.s1, e, nt, p.N, arow, sm, acc);
    } else {
      dma_rows<ASRC, 2>(p, rb, n_e, m0, arow);
      seg_dq_direct<EPI, 2>(p.s1, e, nt, p.N, arow, sm, acc);
    }
  }
  // the per-expert FP32 decode scale multiplies the whole accumulator (the LoRA
  // segment's A operand was stored divided by it); NF4 values are the weights themselves
  const float esc = WF == WF_NF4 ? 1.0f : uniform_load(p.s1.b_sd + e);
  if (p.s2.K > 0) {
    int64_t arow2[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) arow2[i] = rb + min(m0 + a_row(i), n_e - 1);
    seg_lora_n(p.s2, e, nt, p.N, arow2, sm, vt, acc);
  }
  float dp[TM] = {};  // EPI_DOWN_DGRAD: the routing-weight gradient's partial sums
  if (vt > 0) epilogue_t<TM, TN, BN, EPI>(p, acc, nt, m0, n_e, rb, row0, wn * TN * 32, lane, esc, dp);
  if constexpr (EPI == EPI_DOWN_DGRAD)
    if (p.dtw_part) dtw_tile<TM>(p, dp, nt, m0, n_e, rb, wn, lane, reinterpret_cast<float *>(&sm));
}

// LORN: the LoRA term takes an N-major B ([K = r rows][N cols], the dgrad's A_gu / A_dn)
// through seg_lora_n; used when a dgrad runs on this K-major kernel over a columnwise copy
template <int ASRC, int EPI, bool LORN = false, int WF = WF_NVFP4>
__global__ void __launch_bounds__(NTHR, 1) gemm_fwd_q4(GemmParams p) {
  static_assert(WF == WF_NVFP4 || (ASRC == A_GATHER || ASRC == A_ROWS), "NF4 weights take bf16 activations");
  __shared__ __attribute__((aligned(16))) Smem sm;
  // the tile prefix: 256-row tiles, less the remainder tiles the 64-row kernel takes
  auto toff = [&](int e) { return p.tile_off[e] - (p.tile_rem ? p.tile_rem[e] : 0); };
  // tile decode: XCD x (= blockIdx % 8) walks tiles [x*per, (x+1)*per)
  const int total = toff(p.E) * p.NT;
  const int per = (total + 7) / 8;
  const int li = blockIdx.x >> 3;
  if (li >= per) return;
  const int L = (blockIdx.x & 7) * per + li;
  if (L >= total) return;
  const int mt = L / p.NT, nt = L % p.NT;
  int lo = 0, hi = p.E;  // largest e with toff(e) <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (toff(mid) <= mt)
      lo = mid;
    else
      hi = mid;
  }
  const int e = lo;
  const int rb = p.offsets[e];
  const int n_e = p.offsets[e + 1] - rb;
  const int m0 = (mt - toff(e)) * BM;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wn = wid % WNG, row0 = (wid / WNG) * TM * 32;
  const int rows_left = n_e - m0 - row0;  // this wave's valid 32-row tiles: vt (0 skips every MFMA)
  const int vt = rows_left <= 0 ? 0 : (rows_left >= TM * 32 ? TM : (rows_left + 31) / 32);

  constexpr bool kQA = ASRC == A_GATHER_Q || ASRC == A_ROWS_Q;
  int64_t arow[ACH];

  f32x16 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tm][tn][v] = 0.0f;

  // row tiles rounded up to even counts (rows past the segment are dropped); the copies
  // cover the tile's 32 vt rows only
  const int vtu = __builtin_amdgcn_readfirstlane(vt);  // every wave starts at row 0: vt is the tile's
  if (vtu > 6) {
    dma_rows<ASRC, 8>(p, rb, n_e, m0, arow);
    seg_q4_direct<EPI, 8, WF>(p.s1, e, nt, p.N, p.I, arow, sm, acc);
  } else if (vtu > 4) {
    dma_rows<ASRC, 6>(p, rb, n_e, m0, arow);
    seg_q4_direct<EPI, 6, WF>(p.s1, e, nt, p.N, p.I, arow, sm, acc);
  } else if (vtu > 2) {
    dma_rows<ASRC, 4>(p, rb, n_e, m0, arow);
    seg_q4_direct<EPI, 4, WF>(p.s1, e, nt, p.N, p.I, arow, sm, acc);
  } else {
    dma_rows<ASRC, 2>(p, rb, n_e, m0, arow);
    seg_q4_direct<EPI, 2, WF>(p.s1, e, nt, p.N, p.I, arow, sm, acc);
  }

  // FP32 decode scales of segment 1: per expert in the epilogue,
  // per row and expert (NVFP4 activations, val * sb rows) before the LoRA segment
  float esc = 1.0f;  // NF4: the table values are the dequantized weights themselves
  if constexpr (!kQA && WF == WF_NVFP4) esc = uniform_load(p.s1.b_sd + e);
  if constexpr (kQA) {
    const float sb = p.s1.b_sd[e];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      // the accumulator is transposed: lane L holds row L % 32 of the tile
      float sc = sb;
      const int pos = m0 + row0 + tm * 32 + (lane & 31);
      if (pos < n_e) {
        const int64_t src = ASRC == A_GATHER_Q ? (int64_t)(p.perm[rb + pos] / p.k) : (int64_t)(rb + pos);
        sc = sb * p.s1.a_sd[src];
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = acc[tm][tn][v];
          scale_acc(x, sc);
          acc[tm][tn][v] = x;
        }
    }
  }

  if (p.s2.K > 0) {
    int64_t arow2[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) arow2[i] = rb + min(m0 + a_row(i), n_e - 1);
    if constexpr (LORN)
      seg_lora_n(p.s2, e, nt, p.N, arow2, sm, vt, acc);
    else
      seg_lora<EPI>(p.s2, e, nt, p.N, p.I, arow2, sm, vt, acc);
  }

  float dp[TM] = {};  // EPI_DOWN_DGRAD: the routing-weight gradient's partial sums
  if (vt > 0) epilogue_t<TM, TN, BN, EPI>(p, acc, nt, m0, n_e, rb, row0, wn * TN * 32, lane, esc, dp);
  if constexpr (EPI == EPI_DOWN_DGRAD)
    if (p.dtw_part) dtw_tile<TM>(p, dp, nt, m0, n_e, rb, wn, lane, reinterpret_cast<float *>(&sm));
}

// ---- Few routed rows per expert (decode-sized batches) ----
// With a handful of rows per expert the forward is a stream of the hit experts'
// weights, and what bounds it is how many weight bytes each CU keeps in flight.
// This configuration runs the same K loop on 64-row tiles (one or two valid 32-row
// tiles) with NS LDS stages of 17 KB, so that NS - 1 K steps of copies are in flight
// per workgroup instead of two, and OCC workgroups per CU.
constexpr int BMN = 64, TMN = BMN / 32;

template <int NS_>
struct SmemN {
  static constexpr int NS = NS_, NSG = 2;
  uint16_t a[NS_][BMN * BK];
  uint8_t b[NS_][BN * 32];
  uint32_t sg[NSG][BN * 4];  // scale groups: column c's 16 bytes at 16 c
};

// tile_off: prefix over experts of ceil(rows / BMN)
template <int ASRC, int EPI, int WF, int NS, int OCC>
__global__ void __launch_bounds__(NTHR, OCC) gemm_fwd_q4n(GemmParams p) {
  static_assert(WF == WF_NVFP4 || (ASRC == A_GATHER || ASRC == A_ROWS), "NF4 weights take bf16 activations");
  __shared__ __attribute__((aligned(16))) SmemN<NS> sm;
  const int total = p.tile_off[p.E] * p.NT;
  const int per = (total + 7) / 8;
  const int li = blockIdx.x >> 3;
  if (li >= per) return;
  const int L = (blockIdx.x & 7) * per + li;
  if (L >= total) return;
  const int mt = L / p.NT, nt = L % p.NT;
  int lo = 0, hi = p.E;  // largest e with tile_off[e] <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_off[mid] <= mt)
      lo = mid;
    else
      hi = mid;
  }
  const int e = lo;
  const int rb = p.offsets[e];
  const int n_e = p.offsets[e + 1] - rb;
  const int m0 = (p.rem_rows ? n_e / BM * BM : 0) + (mt - p.tile_off[e]) * BMN;
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) % WNG;
  const int rows_left = n_e - m0;  // >= 1: the tile exists
  const int vt = rows_left >= BMN ? TMN : (rows_left + 31) / 32;
  constexpr bool kQA = ASRC == A_GATHER_Q || ASRC == A_ROWS_Q;
  int64_t arow[ACH];
  f32x16 acc[TMN][TN];
#pragma unroll
  for (int tm = 0; tm < TMN; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tm][tn][v] = 0.0f;
  if (__builtin_amdgcn_readfirstlane(vt) > 1) {
    dma_rows<ASRC, 2>(p, rb, n_e, m0, arow);
    seg_q4_direct<EPI, 2, WF, TMN, true>(p.s1, e, nt, p.N, p.I, arow, sm, acc);
  } else {
    dma_rows<ASRC, 1>(p, rb, n_e, m0, arow);
    seg_q4_direct<EPI, 1, WF, TMN, true>(p.s1, e, nt, p.N, p.I, arow, sm, acc);
  }
  float esc = 1.0f;
  if constexpr (!kQA && WF == WF_NVFP4) esc = uniform_load(p.s1.b_sd + e);
  if constexpr (kQA) {
    const float sb = p.s1.b_sd[e];
#pragma unroll
    for (int tm = 0; tm < TMN; ++tm) {
      float sc = sb;
      const int pos = m0 + tm * 32 + (lane & 31);
      if (pos < n_e) {
        const int64_t src = ASRC == A_GATHER_Q ? (int64_t)(p.perm[rb + pos] / p.k) : (int64_t)(rb + pos);
        sc = sb * p.s1.a_sd[src];
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = acc[tm][tn][v];
          scale_acc(x, sc);
          acc[tm][tn][v] = x;
        }
    }
  }
  if (p.s2.K > 0) {
    int64_t arow2[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) arow2[i] = rb + min(m0 + a_row<TMN>(i < TMN ? i : 0), n_e - 1);
    seg_lora<EPI, TMN>(p.s2, e, nt, p.N, p.I, arow2, sm, vt, acc);
  }
  epilogue_t<TMN, TN, BN, EPI>(p, acc, nt, m0, n_e, rb, 0, wn * TN * 32, lane, esc);
}

// The NVFP4 dgrad on 64-row tiles: the same transposed weight read and K loop as
// gemm_dgrad_q4 (three stages, copies two K steps ahead), with stages of 17 KB so that
// kOccD workgroups share a CU.  The LoRA segment's B tile (64 x LSTR bf16) takes the
// A stages 1 and 2 and the code stages after them.
struct SmemD {
  static constexpr int NS = NST, NSG = 0;
  static constexpr int lora_b_bytes = 2 * BMN * BK * 2 + NST * BN * 32;
  uint16_t a[NST][BMN * BK];
  uint8_t b[NST][BN * 32];  // 64 weight rows of 128 code bytes
  uint32_t s[NST][BN];
  uint8_t t[BN / 64][256];
};
static_assert(offsetof(SmemD, b) == sizeof(SmemD::a), "the LoRA tile runs from a[1] into b[]");
constexpr int kOccD = 2;

// tile_off: prefix over experts of the 64-row tiles (few rows), or of the remainder
// tiles when rem_rows is set (each expert's rows past its full 256-row tiles)
template <int ASRC, int EPI>
__global__ void __launch_bounds__(NTHR, kOccD) gemm_dgrad_q4n(GemmParams p) {
  __shared__ __attribute__((aligned(16))) SmemD sm;
  const int total = p.tile_off[p.E] * p.NT;
  const int per = (total + 7) / 8;
  const int li = blockIdx.x >> 3;
  if (li >= per) return;
  const int L = (blockIdx.x & 7) * per + li;
  if (L >= total) return;
  const int mt = L / p.NT, nt = L % p.NT;
  int lo = 0, hi = p.E;  // largest e with tile_off[e] <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_off[mid] <= mt)
      lo = mid;
    else
      hi = mid;
  }
  const int e = lo;
  const int rb = p.offsets[e];
  const int n_e = p.offsets[e + 1] - rb;
  const int m0 = (p.rem_rows ? n_e / BM * BM : 0) + (mt - p.tile_off[e]) * BMN;
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) % WNG;
  const int rows_left = n_e - m0;  // >= 1: the tile exists
  const int vt = rows_left >= BMN ? TMN : (rows_left + 31) / 32;
  int64_t arow[ACH];
  f32x16 acc[TMN][TN];
#pragma unroll
  for (int tm = 0; tm < TMN; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tm][tn][v] = 0.0f;
  if (__builtin_amdgcn_readfirstlane(vt) > 1) {
    dma_rows<ASRC, 2>(p, rb, n_e, m0, arow);
    seg_dq_direct<EPI, 2, TMN>(p.s1, e, nt, p.N, arow, sm, acc);
  } else {
    dma_rows<ASRC, 1>(p, rb, n_e, m0, arow);
    seg_dq_direct<EPI, 1, TMN>(p.s1, e, nt, p.N, arow, sm, acc);
  }
  const float esc = uniform_load(p.s1.b_sd + e);
  if (p.s2.K > 0) {
    int64_t arow2[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) arow2[i] = rb + min(m0 + a_row<TMN>(i < TMN ? i : 0), n_e - 1);
    seg_lora_n<TMN>(p.s2, e, nt, p.N, arow2, sm, vt, acc);
  }
  float dp[TMN] = {};  // EPI_DOWN_DGRAD: the routing-weight gradient's partial sums
  epilogue_t<TMN, TN, BN, EPI>(p, acc, nt, m0, n_e, rb, 0, wn * TN * 32, lane, esc, dp);
  if constexpr (EPI == EPI_DOWN_DGRAD)
    if (p.dtw_part) dtw_tile<TMN>(p, dp, nt, m0, n_e, rb, wn, lane, reinterpret_cast<float *>(&sm));
}
}  // namespace fq

// ---------------------------------------------------------------------------
// Weight-streaming forward for decode-sized batches (NVFP4 weights)
// ---------------------------------------------------------------------------
// With about one routed row per expert each weight byte feeds one or two rows, and
// the forward GEMMs are a stream of the hit experts' 4-bit weights.  This kernel keeps
// no stage in LDS and has no barrier in its K loop.  A workgroup of four waves takes
// up to 16 of one expert's rows per pass (the M of a 16x16x32 bf16 MFMA) and 32
// output columns: the gate and up columns of 16 consecutive i, or 32 consecutive
// columns.  The waves split K into 128-deep blocks (wave w takes blocks w, w + 4, ...).
// In a block, lane L loads 16 code bytes (32 consecutive k) and the two E4M3 scales
// of column L % 16 of each column set at k0 + 32 (L / 16), PF blocks ahead, straight
// into registers, and the same 32 activations of row L % 16 (small, and hot in L2);
// MFMA m of the block takes their k = 8m .. 8m + 7 (one permutation of k for both
// operands).  The four waves' FP32 partial sums are added in LDS in wave order, then
// the LoRA up-projection (split over the waves the same way, 32 deep per MFMA), the
// per-expert (and, for NVFP4 activations, per-row) decode scales and the epilogue.
namespace gv {
constexpr int NTHR = 256, NW = NTHR / 64;
constexpr int KB = 128;  // K per block
constexpr int RP = 16;   // rows per pass at most (the MFMA's M)
constexpr int PF = 4;    // blocks of loads in flight per wave
constexpr int OCC = 4;   // workgroups per CU (at most 128 registers per lane)
constexpr int COLS = 32; // output columns per workgroup (two sets of 16)
constexpr int LDS_BUDGET = 36 * 1024;  // LDS for the weight rows' scales and a pass's activation rows
constexpr int RED_BYTES = NW * 4 * 64 * 16;  // the waves' partial sums (aliasing the rows)
constexpr int LSL = 2;   // LoRA up-projection with KS > 1: 32-deep slices per wave (its K at most 32 KS LSL)
constexpr int KSPLIT_MIN = 4096;  // the waves split K from this K on
// word 3 of a raw buffer resource on this GPU family (32-bit elements, no swizzle)
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((ext_vector_type(4))) float f32x4;

// LDS bytes of the scales of the weight rows a workgroup reads (K / 16 bytes each):
// 32 rows per column block, NW / ks column blocks when ks waves split each one's K
__host__ __device__ constexpr int scale_lds_bytes(int64_t K, int ks) { return (int)(32 * (NW / ks) * (K / 16)); }

struct Blk {
  u32x4 c[2];  // 32 codes of this lane's column in each set (element 2b in the low nibble of byte b)
};

__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// the 8 weights of MFMA m (code word m, block scale m / 2) as bf16 pairs (exact)
template <int M>
__device__ __forceinline__ u32x4 dec8(const u32x4 &c, float sb) {
  u32x4 r;
  f32x2 v = fp4pair<0>(c[M], sb);
  r[0] = pack_exact(v.x, v.y);
  v = fp4pair<1>(c[M], sb);
  r[1] = pack_exact(v.x, v.y);
  v = fp4pair<2>(c[M], sb);
  r[2] = pack_exact(v.x, v.y);
  v = fp4pair<3>(c[M], sb);
  r[3] = pack_exact(v.x, v.y);
  return r;
}

// the codes of one block: byte offsets of the block in this lane's rows (the expert's
// slice is the buffer; a lane past K in a half block reads its row's start)
__device__ __forceinline__ void load_blk(Blk &b, __amdgpu_buffer_rsrc_t rc, const uint32_t (&oc)[2], int k) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    b.c[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc[j] + (uint32_t)(k / 2), 0, 0));
}

// one MFMA's weights decoded right before it (the scheduling barriers keep the decode
// of the whole block from being hoisted, which would hold 32 more registers); xr: this
// lane's activations at the block's k (LDS, zero past K)
// sw: the block's two E4M3 scales of this lane's column in each set (bytes 0, 1)
__device__ __forceinline__ void use_blk(const Blk &b, const uint32_t (&sw)[2], const uint16_t *xr, f32x4 (&acc)[2]) {
  float sb[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    sb[j][0] = e4m3_hw<0>(sw[j]);
    sb[j][1] = e4m3_hw<1>(sw[j]);
  }
  u32x4 x = *reinterpret_cast<const u32x4 *>(xr);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma16(x, dec8<0>(b.c[j], sb[j][0]), acc[j]);
  __builtin_amdgcn_sched_barrier(0);
  x = *reinterpret_cast<const u32x4 *>(xr + 8);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma16(x, dec8<1>(b.c[j], sb[j][0]), acc[j]);
  __builtin_amdgcn_sched_barrier(0);
  x = *reinterpret_cast<const u32x4 *>(xr + 16);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma16(x, dec8<2>(b.c[j], sb[j][1]), acc[j]);
  __builtin_amdgcn_sched_barrier(0);
  x = *reinterpret_cast<const u32x4 *>(xr + 24);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma16(x, dec8<3>(b.c[j], sb[j][1]), acc[j]);
  __builtin_amdgcn_sched_barrier(0);
}

// tile_off: the prefix of 64-row tiles per expert; NT: column blocks of COLS;
// rows_pass rows of K activations (rounded up to a block) fit the dynamic LDS.
// KS waves share a column block and split its K (wave w takes blocks w % KS,
// w % KS + KS, ...), adding their partial sums in LDS; the workgroup holds NW / KS
// column blocks, which share the activation rows.  KS = 1 gives each wave a whole
// column block (a long enough run of blocks when K is short); KS = NW splits long K
// four ways; KS = 2 halves each wave's run when there are too few workgroups to fill
// the chip with whole column blocks.
template <int ASRC, int EPI, int KS>
__global__ void __launch_bounds__(NTHR, OCC) fwd_stream(GemmParams p) {
  static_assert(EPI == EPI_GATEUP || EPI == EPI_STORE, "forward epilogues");
  static_assert(KS == 1 || KS == 2 || KS == NW, "waves per column block");
  constexpr bool kQA = ASRC == A_GATHER_Q || ASRC == A_ROWS_Q;
  constexpr bool kGather = ASRC == A_GATHER || ASRC == A_GATHER_Q;
  constexpr int WS = KS;  // block stride of a wave
  // dynamic LDS: the scales of the weight rows [32 NW / KS][K / 16], then the pass's
  // activation rows [rows_pass][Kp], which after the K loop (KS > 1) hold the waves'
  // partial sums [NW][4][64]: base sums of sets 0, 1, then LoRA sums of sets 0, 1
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ int tile_info[4];
  const int mt = blockIdx.x / p.NT, cbq = blockIdx.x % p.NT;
  // the expert of row tile mt, found by all threads at once: one load per expert
  {
    int hit = 0;
    for (int e = threadIdx.x; e < p.E; e += NTHR) {
      const int t0 = p.tile_off[e], t1 = p.tile_off[e + 1], o0 = p.offsets[e], o1 = p.offsets[e + 1];
      if (t0 <= mt && mt < t1) {
        tile_info[0] = e;
        tile_info[1] = o0;
        tile_info[2] = o1 - o0;
        tile_info[3] = t0;
        hit = 1;
      }
    }
    if (!__syncthreads_or(hit)) return;  // past the last tile: the grid is an upper bound
  }
  const int e = __builtin_amdgcn_readfirstlane(tile_info[0]);
  const int rb = __builtin_amdgcn_readfirstlane(tile_info[1]);
  const int n_e = __builtin_amdgcn_readfirstlane(tile_info[2]);
  const int m0 = (mt - __builtin_amdgcn_readfirstlane(tile_info[3])) * 64, mend = min(m0 + 64, n_e);
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the block loop branches on it
  const int cb = cbq * (NW / KS) + w / KS;  // this wave's column block
  const int kw0 = w % KS;                    // this wave's first block

  // this lane's weight column in each set (a wave past the last column block reads the
  // last 16 rows and stores nothing)
  const Seg &s = p.s1;
  int col[2], row0[2];  // row0: the first weight row of each set
  bool col_ok[2];
  if constexpr (EPI == EPI_GATEUP) {
    const int i = cb * 16 + c;
    row0[0] = min(cb * 16, p.I - 16);
    row0[1] = p.I + row0[0];
    col_ok[0] = col_ok[1] = i < p.I;
    col[0] = col_ok[0] ? i : row0[0];
    col[1] = col_ok[0] ? p.I + i : row0[1];
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = cb * COLS + 16 * j + c;
      row0[j] = min(cb * COLS + 16 * j, p.N - 16);
      col_ok[j] = n < p.N;
      col[j] = col_ok[j] ? n : row0[j];
    }
  }
  const int K = s.K;
  // the expert's slice of codes as a buffer (loads past it read 0)
  const int64_t slice = s.b_rows * s.b_cols;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const uint8_t *>(s.b) + e * (slice / 2)), 0, (int)(slice / 2), kRsrcWord3);
  uint32_t oc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) oc[j] = (uint32_t)col[j] * (uint32_t)(s.b_cols / 2) + 16 * g;
  const int nkb = (K + KB - 1) / KB;
  const int nb = nkb > kw0 ? (nkb - kw0 + WS - 1) / WS : 0;  // this wave's blocks kw0 + WS j
  const int Kp = nkb * KB, K8 = K / 8, Kp8 = Kp / 8;  // LDS row stride: K rounded up, zero past K
  // the E4M3 scales of the waves' weight rows (K / 16 bytes each, contiguous in HBM per
  // set of 16 rows) go to LDS once, by direct copies: 2-byte loads of each lane's own
  // scales would cost one memory transaction per row and block
  const int SB = K / 16;  // scale bytes per weight row (a multiple of 4)
  uint8_t *sc = reinterpret_cast<uint8_t *>(xs);
  uint8_t *scw = sc + (w / KS) * 32 * SB;  // this wave's rows
  uint16_t *xa = reinterpret_cast<uint16_t *>(sc + scale_lds_bytes(K, KS));  // the activation rows after them
  f32x4(*red)[4][64] = reinterpret_cast<f32x4(*)[4][64]>(xa);
  const float esc = kQA ? 1.0f : uniform_load(s.b_sd + e);
  const Seg &l = p.s2;
  const uint16_t *bl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) bl[j] = reinterpret_cast<const uint16_t *>(l.b) + e * l.b_estride + (int64_t)col[j] * l.b_cols;

  for (int r0 = m0; r0 < mend; r0 += p.rows_pass) {
    const int nr = min(p.rows_pass, mend - r0);
    // the pass's activation rows go global -> LDS by direct copies (1 KB per wave and
    // copy), then every lane's first PF blocks of weights and its LoRA operands are
    // requested, and only then is the copy waited for
    for (int q = threadIdx.x; q < nr * (Kp8 - K8); q += NTHR) {
      const int row = q / (Kp8 - K8), ch = K8 + q - row * (Kp8 - K8);
      *reinterpret_cast<u32x4 *>(xa + row * Kp + 8 * ch) = u32x4{0u, 0u, 0u, 0u};
    }
    if (r0 == m0) {
      // set j's 16 weight rows hold 16 SB contiguous bytes of scales (16-byte aligned)
      const uint8_t *sg = reinterpret_cast<const uint8_t *>(s.b_sc) + e * (slice / 16);
      for (int j = 0; j < 2; ++j) {
        const uint8_t *src = sg + (int64_t)row0[j] * SB;
        for (int c0 = 64 * kw0; c0 < SB; c0 += 64 * WS) {  // 16-byte chunks of the 16 SB bytes
          const uint32_t dst = (uint32_t)(uintptr_t)(const fq::lds_void *)(scw + 16 * j * SB + 16 * c0);
          if (c0 + lane < SB) fq::dma_b128(src + 16 * (c0 + lane), dst);
        }
      }
    }
    for (int row = 0; row < nr; ++row) {
      const int64_t src = kGather ? (int64_t)(p.perm[rb + r0 + row] / p.k) : (int64_t)(rb + r0 + row);
      const uint16_t *xg = reinterpret_cast<const uint16_t *>(s.a) + src * s.a_ld;
      for (int c0 = 64 * w; c0 < K8; c0 += 64 * NW) {
        const uint32_t dst = (uint32_t)(uintptr_t)(const fq::lds_void *)(xa + row * Kp + 8 * c0);
        if (c0 + lane < K8) fq::dma_b128(xg + 8 * (c0 + lane), dst);
      }
    }
    const bool xok = c < nr;
    const int pos = r0 + min(c, nr - 1);
    const uint16_t *xrow = xa + min(c, nr - 1) * Kp + 32 * g;
    // this lane's scale pair of a block at k: bytes (k + 32 g) / 16 of its rows (clamped
    // into the row past K, where the activations are zero)
    const uint8_t *srow0 = scw + (col[0] - row0[0]) * SB, *srow1 = scw + (16 + col[1] - row0[1]) * SB;
    auto scales = [&](int k, uint32_t(&sw)[2]) {
      const int o = min(k + 32 * g, K - 32) / 16;
      sw[0] = *reinterpret_cast<const uint16_t *>(srow0 + o);
      sw[1] = *reinterpret_cast<const uint16_t *>(srow1 + o);
    };

    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    Blk buf[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      if (u < nb) {
        const int k = (kw0 + WS * u) * KB;
        load_blk(buf[u], rc, oc, k + 32 * g < K ? k : 0);
      }
    }
    // LoRA up-projection operands (A = the hi/lo pair rows at k < s2.K, B = the expert's
    // LoRA matrix at k mod kmod): with KS > 1, this wave's 32-deep slices kw0, kw0 + KS,
    // ... requested now; otherwise every slice, after the K loop
    const uint16_t *ar = reinterpret_cast<const uint16_t *>(l.a) + (int64_t)(rb + pos) * l.a_ld;
    auto lora_ops = [&](int k, u32x4 &la, u32x4(&lb)[2]) {
      const bool ok = k < l.K;
      const u32x4 z = {0u, 0u, 0u, 0u};
      la = (ok && xok) ? *reinterpret_cast<const u32x4 *>(ar + k) : z;
      const int kb = ok ? k % l.kmod : 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) lb[j] = ok ? *reinterpret_cast<const u32x4 *>(bl[j] + kb) : z;
    };
    u32x4 la[KS > 1 ? LSL : 1], lb[KS > 1 ? LSL : 1][2];
    if constexpr (KS > 1) {
#pragma unroll
      for (int q = 0; q < LSL; ++q) lora_ops(32 * (kw0 + KS * q) + 8 * g, la[q], lb[q]);
    }
    // the direct copies are not tracked by the compiler's wait counts: wait for every load
    // issued so far (the row copies are the oldest), then the barrier
    fq::wait_vm<0>();
    __syncthreads();

    // steady state: every slot is refilled right after use, no branch between loads (so
    // that each use waits only for its own block); then the last blocks without refills
    int j0 = 0;
    auto use = [&](int u, int j) {
      const int k = (kw0 + WS * j) * KB;
      uint32_t sw[2];
      scales(k, sw);
      use_blk(buf[u], sw, xrow + k, acc);
    };
    for (; j0 + 2 * PF <= nb; j0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        use(u, j0 + u);
        const int kn = (kw0 + WS * (j0 + u + PF)) * KB;
        load_blk(buf[u], rc, oc, kn + 32 * g < K ? kn : 0);
      }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      if (j0 + u < nb) {
        use(u, j0 + u);
        if (j0 + u + PF < nb) {
          const int kn = (kw0 + WS * (j0 + u + PF)) * KB;
          load_blk(buf[u], rc, oc, kn + 32 * g < K ? kn : 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (j0 + PF + u < nb) use(u, j0 + PF + u);
    f32x4 lacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if constexpr (KS > 1) {
#pragma unroll
      for (int q = 0; q < LSL; ++q)
#pragma unroll
        for (int j = 0; j < 2; ++j) lacc[j] = mfma16(la[q], lb[q][j], lacc[j]);
    } else {
#pragma unroll 2
      for (int k0 = 0; k0 < l.K; k0 += 32) {
        lora_ops(k0 + 8 * g, la[0], lb[0]);
#pragma unroll
        for (int j = 0; j < 2; ++j) lacc[j] = mfma16(la[0], lb[0][j], lacc[j]);
      }
    }

    f32x4 v[2], lv[2];
    if constexpr (KS > 1) {
      // the partial sums of a column block's KS waves, added in wave order by its first
      __syncthreads();  // every wave is done reading the activation rows
      red[w][0][lane] = acc[0];
      red[w][1][lane] = acc[1];
      red[w][2][lane] = lacc[0];
      red[w][3][lane] = lacc[1];
      __syncthreads();
      if (kw0 == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          v[j] = red[w][j][lane];
          lv[j] = red[w][2 + j][lane];
#pragma unroll
          for (int q = 1; q < KS; ++q) {
            v[j] += red[w + q][j][lane];
            lv[j] += red[w + q][2 + j][lane];
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v[j] = acc[j];
        lv[j] = lacc[j];
      }
    }
    if (kw0 == 0) {
      // lane (c, g) holds rows 4 g + t (t = 0..3) of column c of each set
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = 4 * g + t;
        if (row >= nr) continue;
        const int64_t grow = rb + r0 + row;
        float val[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) val[j] = v[j][t];
        if constexpr (kQA) {
          const int64_t src = kGather ? (int64_t)(p.perm[grow] / p.k) : grow;
          const float sc = p.s1.b_sd[e] * p.s1.a_sd[src];
#pragma unroll
          for (int j = 0; j < 2; ++j) val[j] *= sc;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) val[j] += lv[j][t];
        if constexpr (EPI == EPI_GATEUP) {
          if (col_ok[0]) {
            const int i = cb * 16 + c;
            const float gv = val[0] * esc, uv = val[1] * esc;
            float *hrow = p.outf + grow * 2 * p.I;
            hrow[i] = gv;
            hrow[p.I + i] = uv;
            p.out1[grow * p.I + i] = (uint16_t)f32_to_bf16(gv * sigmoid_f(gv) * uv);
          }
        } else {
          const float sc = esc * p.out_scale;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (col_ok[j]) p.out0[grow * p.N + cb * COLS + 16 * j + c] = (uint16_t)f32_to_bf16(val[j] * sc);
        }
      }
    }
    __syncthreads();  // red and xs are reused by the next pass
  }
}
}  // namespace gv

// ---------------------------------------------------------------------------
// LoRA projections (N = r): U = s X A^T (A K-major [r][K]) and V = s dY B
// (B N-major [K][r]), per routed row, stored as hi/lo bf16 pairs.
// ---------------------------------------------------------------------------
// These stream the routed activation rows once (K = H, I or 2I deep, 64 columns),
// so they are bound by memory: a 256 x 64 tile per workgroup of 4 waves (64 rows
// each), two LDS stages of 40 KB filled by direct-to-LDS copies one step ahead, two
// workgroups per CU.  Rows are the same XOR-swizzled 128-byte rows as the GEMMs;
// an N-major B tile keeps its 64 k-rows of 128 bytes with 16-byte chunk c at
// c ^ (k & 7) and is read with the 16-bit transposing LDS read.
namespace lp {
constexpr int BM = 256, BN = 64, NTHR = 256, NST = 2, TM = 2, TN = 2, NDMA = 10;

struct Smem {
  uint16_t a[NST][BM * BK];
  uint16_t b[NST][BN * BK];
};

__device__ __forceinline__ uint32_t smem_u32(const Smem &sm) { return (uint32_t)(uintptr_t)(const fq::lds_void *)&sm; }

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// B fragment of an N-major swizzled tile: lane L gets column nbase + (L & 31) and
// rows kbase + 8 (L >> 5) + 0..7
__device__ __forceinline__ bf16x8 b_frag_nm(const uint16_t *Bs, int kbase, int nbase, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int row = kbase + 8 * (g >> 1) + (sl >> 2), col = nbase + 16 * (g & 1) + 4 * (sl & 3);
  const uint16_t *p0 = Bs + row * BK + 8 * ((col >> 3) ^ (row & 7)) + (col & 7);
  const uint16_t *p1 = Bs + (row + 4) * BK + 8 * ((col >> 3) ^ ((row + 4) & 7)) + (col & 7);
  const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p0));
  const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p1));
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  const s16x8 v = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int ASRC, bool BNM>
__global__ void __launch_bounds__(NTHR, 2) gemm_lora_proj(GemmParams p) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int total = p.tile_off[p.E] * p.NT;
  const int per = (total + 7) / 8;
  const int li = blockIdx.x >> 3;
  if (li >= per) return;
  const int L = (blockIdx.x & 7) * per + li;
  if (L >= total) return;
  const int mt = L / p.NT, nt = L % p.NT;
  int lo = 0, hi = p.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_off[mid] <= mt)
      lo = mid;
    else
      hi = mid;
  }
  const int e = lo;
  const int rb = p.offsets[e];
  const int n_e = p.offsets[e + 1] - rb;
  const int m0 = (mt - p.tile_off[e]) * BM;
  const int lane = threadIdx.x & 63;
  const uint32_t w = fq::wave_id();
  const int row0 = 64 * (int)w;
  const int rows_left = n_e - m0 - row0;
  const int vt = rows_left <= 0 ? 0 : (rows_left >= 64 ? 2 : (rows_left + 31) / 32);
  const Seg &s = p.s1;
  // copy sources at K step 0: 8 A chunks and 2 B chunks per thread
  const uint16_t *asrc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 64 * (int)w + 8 * j + (lane >> 3);
    const int pos = min(m0 + row, n_e - 1);
    const int64_t arow = ASRC == A_GATHER ? (int64_t)(p.perm[rb + pos] / p.k) : (int64_t)(rb + pos);
    asrc[j] = reinterpret_cast<const uint16_t *>(s.a) + arow * s.a_ld + 8 * ((lane & 7) ^ ((row >> 1) & 7));
  }
  const uint16_t *bsrc[2];
  const uint16_t *bbase = reinterpret_cast<const uint16_t *>(s.b) + e * s.b_estride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * (int)w + 8 * i + (lane >> 3);
    if constexpr (BNM) {  // row = k of the step; 8 columns per chunk
      int c = (lane & 7) ^ (row & 7);
      if (nt * BN + 8 * c >= p.N) c = 0;  // columns past r: any valid bytes (dropped)
      bsrc[i] = bbase + (int64_t)row * s.b_cols + nt * BN + 8 * c;
    } else {  // row = output column n
      int n = nt * BN + row;
      n = n < p.N ? n : 0;
      bsrc[i] = bbase + (int64_t)n * s.b_cols + 8 * ((lane & 7) ^ ((row >> 1) & 7));
    }
  }
  const int64_t bstep = BNM ? (int64_t)BK * s.b_cols : BK;  // elements per K step
  const uint32_t sbase = smem_u32(sm);
  auto issue = [&](int ks, int st) {
    const uint32_t la = sbase + (uint32_t)offsetof(Smem, a) + (uint32_t)st * (uint32_t)sizeof(sm.a[0]);
    const uint32_t lb = sbase + (uint32_t)offsetof(Smem, b) + (uint32_t)st * (uint32_t)sizeof(sm.b[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) fq::dma_b128(asrc[j] + ks * BK, la + (64 * w + 8 * j) * BK * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) fq::dma_b128(bsrc[i] + ks * bstep, lb + (16 * w + 8 * i) * BK * 2);
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tm][tn][v] = 0.0f;
  const int nk = s.K / BK;
  issue(0, 0);
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    if (ks + 1 < nk) {
      issue(ks + 1, st ^ 1);
      fq::wait_vm<NDMA>();
    } else {
      fq::wait_vm<0>();
    }
    fq::barrier_lds();
    const uint16_t *As = sm.a[st], *Bs = sm.b[st];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[TM], bf[TN];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if constexpr (BNM)
          bf[tn] = b_frag_nm(Bs, 16 * kk, tn * 32, lane);
        else
          bf[tn] = *reinterpret_cast<const bf16x8 *>(Bs + fq::a_off(tn * 32 + (lane & 31), 2 * kk + (lane >> 5)));
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        af[tm] = *reinterpret_cast<const bf16x8 *>(As + fq::a_off(row0 + tm * 32 + (lane & 31), 2 * kk + (lane >> 5)));
        if (tm < vt) {
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm], bf[tn], acc[tm][tn], 0, 0, 0);
        }
      }
    }
    fq::barrier_lds();  // the next step copies into this stage
  }
  if (vt > 0) epilogue<TM, TN, BN, EPI_STORE_SPLIT>(p, acc, e, nt, m0, n_e, rb, row0, 0, lane, 1.0f);
}
}  // namespace lp

// LoRA-A projection for a few rows per expert (decode-sized batches): out[row][n] =
// osc * sum_k A_row[k] * B[e][n][k] (B K-major [N][K]) stored as hi/lo bf16 pairs like
// the tiled projection above.  A workgroup takes expert e and 4 outputs for all of the
// expert's rows, one per wave; the lanes split K in 8-element pieces (four 512-wide
// slices' loads in flight at a time) and add their FP32 partial sums in a fixed
// butterfly.  The tiled kernel walks K in 64-deep steps with one 256-row tile per
// expert, which leaves most of the GPU idle when the batch is a few tokens.
// one wave: the dot product of activation row arow of s.a with the weight row brow
// over K = s.K; lane takes k = 8 lane + 512 j .. +8 and sums its products in order of
// k, four 512-wide slices' loads in flight at a time, then the lanes are added
__device__ __forceinline__ float lora_row_dot(const Seg &s, const uint16_t *brow, int64_t arow, int lane) {
  const int K = s.K;
  const uint16_t *ar = reinterpret_cast<const uint16_t *>(s.a) + arow * s.a_ld;
  float acc = 0.0f;
  int k0 = 8 * lane;
  for (; k0 + 3 * 512 < K; k0 += 4 * 512) {
    uint4 xa[4], ba[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xa[u] = *reinterpret_cast<const uint4 *>(ar + k0 + 512 * u);
      ba[u] = *reinterpret_cast<const uint4 *>(brow + k0 + 512 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t xv[4] = {xa[u].x, xa[u].y, xa[u].z, xa[u].w}, bv[4] = {ba[u].x, ba[u].y, ba[u].z, ba[u].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc += bf16_lo(xv[h]) * bf16_lo(bv[h]);
        acc += bf16_hi(xv[h]) * bf16_hi(bv[h]);
      }
    }
  }
  for (; k0 < K; k0 += 512) {
    const uint4 xa = *reinterpret_cast<const uint4 *>(ar + k0);
    const uint4 ba = *reinterpret_cast<const uint4 *>(brow + k0);
    const uint32_t xv[4] = {xa.x, xa.y, xa.z, xa.w}, bv[4] = {ba.x, ba.y, ba.z, ba.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc += bf16_lo(xv[h]) * bf16_lo(bv[h]);
      acc += bf16_hi(xv[h]) * bf16_hi(bv[h]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  return acc;
}

// output row `row`, column n of the [R, 2N] hi/lo pair layout (lane 0 stores)
__device__ __forceinline__ void lora_row_store(const GemmParams &p, int64_t row, int n, float val, int lane) {
  if (lane == 0) {
    const uint32_t hb = f32_to_bf16(val);
    const float lo2 = val - __uint_as_float(hb << 16);
    p.out0[row * 2 * p.N + n] = (uint16_t)hb;
    p.out0[row * 2 * p.N + p.N + n] = (uint16_t)f32_to_bf16(lo2);
  }
}

template <int ASRC>
__global__ void __launch_bounds__(256) lora_proj_rows(GemmParams p) {
  // workgroup row blockIdx.y: one 64-row tile of the prefix p.tile_off (at most 16 tokens:
  // one tile per expert with rows), its expert found by all threads at once
  __shared__ int tile_e;
  const int mt = blockIdx.y;
  {
    int hit = 0;
    for (int e = threadIdx.x; e < p.E; e += 256)
      if (p.tile_off[e] <= mt && mt < p.tile_off[e + 1]) {
        tile_e = e;
        hit = 1;
      }
    if (!__syncthreads_or(hit)) return;  // past the last tile: the grid is an upper bound
  }
  const int e = tile_e;
  const int m0 = (mt - p.tile_off[e]) * 64;
  const int rb = p.offsets[e] + m0, n_e = min(p.offsets[e + 1] - rb, 64);  // this tile's rows
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);  // one output column per wave
  if (n >= p.N) return;
  const Seg &s = p.s1;
  const uint16_t *brow = reinterpret_cast<const uint16_t *>(s.b) + e * s.b_estride + (int64_t)n * s.b_cols;
  const float osc = p.div_e ? p.out_scale / uniform_load(p.div_e + e) : p.out_scale;
  for (int i = 0; i < n_e; ++i) {
    const int64_t arow = ASRC == A_GATHER ? (int64_t)(p.perm[rb + i] / p.k) : (int64_t)(rb + i);
    lora_row_store(p, rb + i, n, lora_row_dot(s, brow, arow, lane) * osc, lane);
  }
}

// The one-workgroup permutation and the forward's first LoRA projection (U = s X A^T
// over gathered token rows) in one launch, for decode-sized batches (at most 1024
// routed pairs): workgroup 0 runs the permutation; every other workgroup takes one
// routed pair and 16 / wpc output columns, wpc waves per column (1, 2 or 4: as many as
// keep the grid within one round of the chip), each wave the 512-wide K slices
// q, q + wpc, ... (four slices' loads in flight at a time), the waves' sums added in
// order through LDS.  A projection workgroup places its
// pair's row itself, where the stable counting sort puts it (the number of pairs of
// lower experts plus the pair's rank among its expert's pairs), so it does not wait
// for workgroup 0; a dropped pair (expert index outside [0, E)) has no row.
struct PermArgs {
  const int32_t *idx;
  int R, E;
  int32_t *offsets;
  int bm;
  int32_t *tile_off;
  int bm2;
  int32_t *tile_off2;
  int32_t *perm, *inv;
  const float *w_in;
  float *w_out;
};
constexpr int kPermLoraWaves = 16;  // waves per projection workgroup

__global__ void __launch_bounds__(1024) perm_lora_rows(PermArgs a, GemmParams p, int wpc) {
  if (blockIdx.x == 0) {
    extern __shared__ int32_t cnt[];  // E + 1 buckets
    perm_one_body(a.idx, a.R, a.E, a.offsets, a.bm, a.tile_off, a.bm2, a.tile_off2, a.perm, a.inv, a.w_in, a.w_out,
                  cnt);
    return;
  }
  __shared__ float part[kPermLoraWaves];
  const int cols = kPermLoraWaves / wpc;  // output columns of this workgroup
  const int ncg = (p.N + cols - 1) / cols;
  const int f = (blockIdx.x - 1) / ncg;  // the routed pair (the grid holds R of them)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = ((blockIdx.x - 1) % ncg) * cols + wave % cols, kq = wave / cols;
  const int e = bucket_of(a.idx[f], a.E);
  const int q = threadIdx.x;  // one pair per thread: R <= 1024
  const int bq = q < a.R ? bucket_of(a.idx[q], a.E) : a.E + 1;
  const int lower = __syncthreads_count(bq < e);
  const int before = __syncthreads_count(q < f && bq == e);
  if (e >= a.E) return;  // the whole workgroup
  const bool ok = n < p.N;
  const Seg &s = p.s1;
  const int K = s.K;
  const uint16_t *brow = reinterpret_cast<const uint16_t *>(s.b) + e * s.b_estride + (int64_t)(ok ? n : 0) * s.b_cols;
  const uint16_t *ar = reinterpret_cast<const uint16_t *>(s.a) + (int64_t)(f / p.k) * s.a_ld;
  float acc = 0.0f;  // this lane's k = 8 lane + 512 (kq + wpc j) .. +8, in order of k
  const int step = 512 * wpc;
  for (int k0 = 8 * lane + 512 * kq; k0 < K; k0 += 4 * step) {
    uint4 xa[4], ba[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + step * u < K) {
        xa[u] = *reinterpret_cast<const uint4 *>(ar + k0 + step * u);
        ba[u] = *reinterpret_cast<const uint4 *>(brow + k0 + step * u);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + step * u < K) {
        const uint32_t xv[4] = {xa[u].x, xa[u].y, xa[u].z, xa[u].w}, bv[4] = {ba[u].x, ba[u].y, ba[u].z, ba[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc += bf16_lo(xv[h]) * bf16_lo(bv[h]);
          acc += bf16_hi(xv[h]) * bf16_hi(bv[h]);
        }
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (kq == 0 && ok) {
    float sum = part[wave];
    for (int i = 1; i < wpc; ++i) sum += part[wave + cols * i];
    const float osc = p.div_e ? p.out_scale / uniform_load(p.div_e + e) : p.out_scale;
    lora_row_store(p, lower + before, n, sum * osc, lane);
  }
}

// ---------------------------------------------------------------------------
// LoRA weight gradients: C[e] [M, N] = sum over the expert's rows of P[row][m] * Q[row][n]
// ---------------------------------------------------------------------------
struct WgradParams {
  const int32_t *perm, *offsets;
  const float *tw;  // routing weights by pair (scales P rows when scale_p)
  int k, M, N;
  const uint16_t *P;
  int64_t p_ld;
  int p_gather;     // P rows gathered by token
  int scale_p;      // multiply P rows by the routing weight
  const uint16_t *Q;
  int64_t q_ld;
  int q_gather;
  const float *c_scale;  // per-expert factor of the output (NULL: none)
  float *C;
  // > 0: one output for all experts (a shared LoRA-A) from `split` parts of the
  // experts; C is then [split][M][N] partial sums
  int split;
  int E;
  // per-expert outputs: row chunks (see wgrad_chunks) and the partial sums of the
  // experts with more than one chunk
  const int32_t *chunk_off, *slot_off;
  int chunk;
  float *part;
};

constexpr int WB = 64;  // wgrad tile (M and N) and row step

// One 64x64 tile of C[e] per workgroup; rows of the expert's segment in steps
// of 64.  All 256 threads load: each owns 2 16-byte chunks of the P rows and 2
// of the Q rows of a step (rows row = c / 8, 8 columns at 8 * (c % 8)), held in
// registers one step ahead; the routing weight that scales P rows is applied when
// the step is written to LDS, so the loads are not waited for before the MFMAs of
// the current step.  Tiles stay in their natural [row][col] layout in one LDS stage
// (18 KB, so eight workgroups share a CU and keep many loads in flight; two or three
// steps in flight per workgroup measured slower) and the MFMA fragments (8
// consecutive rows of one column) come from the gfx950 transposing LDS read.
constexpr int WS = WB + 8;  // LDS row stride in bf16 (64 columns + 16-byte pad)

struct WRegs {
  uint4 v[4];  // P chunks 0, 1; Q chunks 0, 1
  float w[2];  // routing weights of the two P rows (scale_p)
};

__device__ __forceinline__ void wgrad_load(const WgradParams &p, int rb, int n_e, int r0, int m0, int n0, WRegs &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool isq = i >= 2;
    const int c = tid + NTHR * (i & 1);  // 0..511: row c / 8, columns 8 * (c % 8)
    const int pos = r0 + (c >> 3);
    const int col = (isq ? n0 : m0) + 8 * (c & 7);
    const int lim = isq ? p.N : p.M;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (pos < n_e && col < lim) {
      const int64_t grow = rb + pos;
      const int gather = isq ? p.q_gather : p.p_gather;
      const int64_t srow = gather ? (int64_t)(p.perm[grow] / p.k) : grow;
      x = *reinterpret_cast<const uint4 *>((isq ? p.Q : p.P) + srow * (isq ? p.q_ld : p.p_ld) + col);
    }
    r.v[i] = x;
    if (!isq && p.scale_p) r.w[i] = pos < n_e ? p.tw[p.perm[rb + pos]] : 0.0f;
  }
}

__device__ __forceinline__ void wgrad_store(const WgradParams &p, uint16_t *Ps, uint16_t *Qs, const WRegs &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NTHR * (i & 1);
    uint4 x = r.v[i];
    if (i < 2 && p.scale_p) {
      const float s = r.w[i];
      uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) w[h] = f32_to_bf16(bf16_lo(w[h]) * s) | (f32_to_bf16(bf16_hi(w[h]) * s) << 16);
      x = make_uint4(w[0], w[1], w[2], w[3]);
    }
    *reinterpret_cast<uint4 *>((i >= 2 ? Qs : Ps) + (c >> 3) * WS + 8 * (c & 7)) = x;
  }
}

// acc = sum over the n_e rows from rb of P[row][m0 + .] (x) Q[row][n0 + .] for this
// wave's 32x32 quarter of the tile; the stage is free again on return
__device__ __forceinline__ void wgrad_rows(const WgradParams &p, int rb, int n_e, int m0, int n0, uint16_t *Ps,
                                           uint16_t *Qs, f32x16 &acc) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  const int nk = (n_e + WB - 1) / WB;
  if (nk == 0) return;
  WRegs r;
  wgrad_load(p, rb, n_e, 0, m0, n0, r);
  wgrad_store(p, Ps, Qs, r);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) wgrad_load(p, rb, n_e, (ks + 1) * WB, m0, n0, r);
#pragma unroll
    for (int kk = 0; kk < WB / 16; ++kk) {
      const bf16x8 a = b_frag_trans_s<WS>(Ps, kk * 16, wm * 32, lane);
      const bf16x8 b = b_frag_trans_s<WS>(Qs, kk * 16, wn * 32, lane);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading the stage
    if (ks + 1 < nk) {
      wgrad_store(p, Ps, Qs, r);
      __syncthreads();
    }
  }
}

// Row chunks of the per-expert gradients: an expert's rows are cut into chunks of
// p.chunk rows, one workgroup per chunk and output tile, so that the few experts with
// many rows under skewed routing do not keep one long K loop running after the rest.
// chunk_off[e] is the prefix of the chunk counts max(1, ceil(n_e / chunk)) (an expert
// without rows keeps one chunk, which writes its zero gradient); slot_off[e] the prefix
// of the counts of the experts with more than one chunk, whose chunks write FP32
// partial sums to slots slot_off[e] + j, added in chunk order by wgrad_sum_chunks.
// multi[0] is the number of such experts and multi[1 + i] the i-th of them.  One
// workgroup of 1024 threads, E <= 1024, inclusive scans in LDS.
__global__ void __launch_bounds__(1024) wgrad_chunks(const int32_t *__restrict__ offsets, int E, int chunk,
                                                     int32_t *__restrict__ chunk_off, int32_t *__restrict__ slot_off,
                                                     int32_t *__restrict__ multi) {
  __shared__ int32_t a[1024], b[1024], m[1024];
  const int t = threadIdx.x;
  int nc = 0, ns = 0;
  if (t < E) {
    const int n = offsets[t + 1] - offsets[t];
    nc = n > chunk ? (n + chunk - 1) / chunk : 1;
    ns = nc > 1 ? nc : 0;
  }
  a[t] = nc;
  b[t] = ns;
  m[t] = ns > 0;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int va = t >= d ? a[t - d] : 0, vb = t >= d ? b[t - d] : 0, vm = t >= d ? m[t - d] : 0;
    __syncthreads();
    a[t] += va;
    b[t] += vb;
    m[t] += vm;
    __syncthreads();
  }
  if (t == 0) {
    chunk_off[0] = slot_off[0] = 0;
    multi[0] = m[1023];
  }
  if (t < E) {
    chunk_off[t + 1] = a[t];
    slot_off[t + 1] = b[t];
    if (ns > 0) multi[m[t]] = t;  // 1 + (its rank among them)
  }
}

// C[e] = c_scale[e] times the sum of expert e's chunk partials in chunk order, for the
// experts with more than one chunk: blockIdx.y = the rank of e among them (multi, see
// wgrad_chunks), a grid-stride loop over the n4 float4 of the output
__global__ void __launch_bounds__(NTHR) wgrad_sum_chunks(const float4 *__restrict__ part,
                                                         const int32_t *__restrict__ chunk_off,
                                                         const int32_t *__restrict__ slot_off,
                                                         const int32_t *__restrict__ multi,
                                                         const float *__restrict__ c_scale, int64_t n4,
                                                         float4 *__restrict__ C) {
  if ((int)blockIdx.y >= multi[0]) return;
  const int e = multi[1 + blockIdx.y];
  const int nch = chunk_off[e + 1] - chunk_off[e];
  const float cs = c_scale ? c_scale[e] : 1.0f;
  const float4 *pe = part + (int64_t)slot_off[e] * n4;
  for (int64_t i = (int64_t)blockIdx.x * NTHR + threadIdx.x; i < n4; i += (int64_t)gridDim.x * NTHR) {
    float4 acc = pe[i];
    for (int j = 1; j < nch; ++j) {
      const float4 v = pe[(int64_t)j * n4 + i];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    acc.x *= cs;
    acc.y *= cs;
    acc.z *= cs;
    acc.w *= cs;
    C[(int64_t)e * n4 + i] = acc;
  }
}

// blockIdx.y: a row chunk of one expert (see wgrad_chunks): C[e] = c_scale[e] times
// its sum when the expert has one chunk, else the chunk's partial sum; or (SPLIT)
// the part e of the experts, [e E / split, (e+1) E / split), whose sums times their
// c_scale are added in FP32 in expert order into C[e], a partial sum of the one
// [M, N] output (the second accumulator lives only in this variant: the per-expert
// one stays within the registers of eight workgroups per CU)
template <bool SPLIT>
__global__ void __launch_bounds__(NTHR) lora_wgrad(WgradParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ps[WB * WS];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[WB * WS];
  int e = blockIdx.y;
  const int ntn = (p.N + WB - 1) / WB;
  const int mt = blockIdx.x / ntn, ntile = blockIdx.x % ntn;
  const int m0 = mt * WB, n0 = ntile * WB;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  f32x16 acc;
  float *out = nullptr;  // this workgroup's [M, N] output (set below)
  if constexpr (SPLIT) {
    const int e0 = (int)((int64_t)e * p.E / p.split), e1 = (int)((int64_t)(e + 1) * p.E / p.split);
    f32x16 tot;
#pragma unroll
    for (int v = 0; v < 16; ++v) tot[v] = 0.0f;
    for (int ex = e0; ex < e1; ++ex) {
      const int rb = p.offsets[ex];
      wgrad_rows(p, rb, p.offsets[ex + 1] - rb, m0, n0, Ps, Qs, acc);
      const float cs = p.c_scale ? p.c_scale[ex] : 1.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[v] += acc[v] * cs;
    }
    acc = tot;
    out = p.C + (int64_t)e * p.M * p.N;
  } else {
    const int c = blockIdx.y;
    if (c >= p.chunk_off[p.E]) return;
    int lo = 0, hi = p.E;  // the expert of chunk c: largest e with chunk_off[e] <= c
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.chunk_off[mid] <= c)
        lo = mid;
      else
        hi = mid;
    }
    e = lo;
    const int j = c - p.chunk_off[e], nch = p.chunk_off[e + 1] - p.chunk_off[e];
    const int rb = p.offsets[e], r0 = j * p.chunk;
    wgrad_rows(p, rb + r0, min(p.chunk, p.offsets[e + 1] - rb - r0), m0, n0, Ps, Qs, acc);
    if (nch > 1) {
      out = p.part + (int64_t)(p.slot_off[e] + j) * p.M * p.N;
    } else {
      const float cs = p.c_scale ? p.c_scale[e] : 1.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] *= cs;
      out = p.C + (int64_t)e * p.M * p.N;
    }
  }
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) {
    const int m = m0 + wm * 32 + 8 * (vv >> 2) + 4 * (lane >> 5) + (vv & 3);
    const int n = n0 + wn * 32 + (lane & 31);
    if (m < p.M && n < p.N) out[(int64_t)m * p.N + n] = acc[vv];
  }
}

// C[i] = sum of part[s][i] over s = 0, 1, ..., split-1 in that order (the split
// sums of lora_wgrad; n4 float4 per part)
__global__ void __launch_bounds__(NTHR) sum_parts(const float4 *__restrict__ part, int split, int64_t n4,
                                                  float4 *__restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * NTHR + threadIdx.x;
  if (i >= n4) return;
  float4 acc = part[i];
  for (int q = 1; q < split; ++q) {
    const float4 v = part[q * n4 + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  C[i] = acc;
}

// ---------------------------------------------------------------------------
// combine, routing-weight gradient
// ---------------------------------------------------------------------------
// out[t][c] = sum_j w[t,j] * rows[inv[t*k+j]][c] (w = 1 when tw == NULL), j ascending,
// FP32 accumulation over the bf16 routed rows; pairs placed at or after *n_valid (an
// expert index outside [0, E)) belong to no expert and add nothing
__global__ void __launch_bounds__(NTHR) combine_rows(const uint16_t *__restrict__ rows, const int32_t *__restrict__ inv,
                                                     const int32_t *__restrict__ n_valid, const float *__restrict__ tw,
                                                     int64_t T, int k, int64_t H, uint16_t *__restrict__ out) {
  const int64_t cpr = H / 8;
  const int32_t nv = *n_valid;
  for (int64_t it = (int64_t)blockIdx.x * NTHR + threadIdx.x; it < T * cpr; it += (int64_t)gridDim.x * NTHR) {
    const int64_t t = it / cpr, c = (it % cpr) * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // the token's row positions, then its rows, each set of loads in flight together
    // (k <= 16), then the sum in pair order
    int32_t pos[16];
    float w[16];
    uint4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) {
        pos[j] = inv[t * k + j];
        w[j] = tw ? tw[t * k + j] : 1.0f;
      }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k && pos[j] < nv) v[j] = *reinterpret_cast<const uint4 *>(rows + (int64_t)pos[j] * H + c);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k && pos[j] < nv) {
        const float wj = w[j];
        acc[0] += wj * bf16_lo(v[j].x); acc[1] += wj * bf16_hi(v[j].x);
        acc[2] += wj * bf16_lo(v[j].y); acc[3] += wj * bf16_hi(v[j].y);
        acc[4] += wj * bf16_lo(v[j].z); acc[5] += wj * bf16_hi(v[j].z);
        acc[6] += wj * bf16_lo(v[j].w); acc[7] += wj * bf16_hi(v[j].w);
      }
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) o[h] = f32_to_bf16(acc[2 * h]) | (f32_to_bf16(acc[2 * h + 1]) << 16);
    *reinterpret_cast<uint4 *>(out + t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// dtw[f] = <dy[t], y[inv[f]]>, one wave per routed pair (0 for a pair of no expert)
__global__ void __launch_bounds__(NTHR) dtopk_kernel(const uint16_t *__restrict__ dy, const uint16_t *__restrict__ y,
                                                     const int32_t *__restrict__ inv, const int32_t *__restrict__ n_valid,
                                                     int64_t R, int k, int64_t H, float *__restrict__ dtw) {
  const int lane = threadIdx.x & 63;
  const int64_t f = (int64_t)blockIdx.x * (NTHR / 64) + (threadIdx.x >> 6);
  if (f >= R) return;
  const int32_t pos = inv[f];
  if (pos >= *n_valid) {
    if (lane == 0) dtw[f] = 0.0f;
    return;
  }
  const uint16_t *a = dy + (f / k) * H;
  const uint16_t *b = y + (int64_t)pos * H;
  float s = 0.0f;
  for (int64_t c = lane * 8; c < H; c += 64 * 8) {
    const uint4 va = *reinterpret_cast<const uint4 *>(a + c), vb = *reinterpret_cast<const uint4 *>(b + c);
    s += bf16_lo(va.x) * bf16_lo(vb.x) + bf16_hi(va.x) * bf16_hi(vb.x) + bf16_lo(va.y) * bf16_lo(vb.y) +
         bf16_hi(va.y) * bf16_hi(vb.y);
    s += bf16_lo(va.z) * bf16_lo(vb.z) + bf16_hi(va.z) * bf16_hi(vb.z) + bf16_lo(va.w) * bf16_lo(vb.w) +
         bf16_hi(va.w) * bf16_hi(vb.w);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) dtw[f] = s;
}

// d(top-k w) from the down dgrad's partial sums: pair f's row inv[f] has nt partial sums
// of da_u * a (one per output column tile of I), added in tile order; a dropped pair
// (row past the experts' segments) gets 0.  The sum over i of da_u * a equals the sum over
// h of dy * y: y = a W~^T + the LoRA term is linear in a.
__global__ void __launch_bounds__(NTHR) dtopk_sum(const float *__restrict__ part, int nt,
                                                  const int32_t *__restrict__ inv, const int32_t *__restrict__ n_valid,
                                                  int64_t R, float *__restrict__ dtw) {
  const int64_t f = (int64_t)blockIdx.x * NTHR + threadIdx.x;
  if (f >= R) return;
  const int32_t pos = inv[f];
  float s = 0.0f;
  if (pos < *n_valid)
    for (int q = 0; q < nt; ++q) s += part[(int64_t)pos * nt + q];
  dtw[f] = s;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Layout {
  size_t perm, inv, off, tile_off, tile_off_n, counts, tw, ugu, udn, h, a, y, xq_c, xq_s, xq_d, xq_b, aq_c, aq_s, aq_d, aq_b, vdn, dh,
      vgu, dxr, part, wchunk, wpart, absx, dtwp;
  size_t total;
};

// parts of the experts whose shared-A gradient sums run side by side
int lora_split(int E) { return E < 64 ? E : 64; }

// rows per chunk of the per-expert LoRA gradients (wgrad_chunks): 2048, raised for very
// large batches so that the chunks (at most E + R / chunk) fit the grid's y dimension
int wgrad_chunk(int64_t R) { return (int)std::max<int64_t>(2048, cdiv(R, 32768)); }

Layout layout(const bqm_moe_desc *d) {
  const size_t T = d->T, H = d->H, I = d->I, E = d->E, k = d->k, r = d->r;
  const size_t R = T * k;
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.perm = take(R * 4);
  L.inv = take(R * 4);
  L.off = take((E + 1) * 4);
  L.tile_off = take((E + 1) * 4);
  L.tile_off_n = take((E + 1) * 4);
  L.counts = take(permute_ws_bytes((int64_t)R, (int)E));
  L.tw = take(R * 4);
  L.ugu = take(R * 2 * r * 2);
  L.udn = take(R * 2 * r * 2);
  L.h = take(R * 2 * I * 4);
  L.a = take(R * I * 2);
  L.y = take(R * H * 2);
  const bool aq = d->act_quant != 0;
  L.xq_c = take(aq ? T * H / 2 : 0);
  L.xq_s = take(aq ? T * H / 16 : 0);
  L.xq_d = take(aq ? T * 4 : 0);
  L.xq_b = take(aq ? T * H * 2 : 0);
  L.aq_c = take(aq ? R * I / 2 : 0);
  L.aq_s = take(aq ? R * I / 16 : 0);
  L.aq_d = take(aq ? R * 4 : 0);
  L.aq_b = take(aq ? R * I * 2 : 0);
  L.vdn = take(R * 2 * r * 2);
  L.dh = take(R * 2 * I * 2);
  L.vgu = take(R * 2 * r * 2);
  L.dxr = take(R * H * 2);
  // shared-A gradient: lora_split(R) partial sums of [r, max(H, I)] in FP32
  L.part = take(d->lora_shared_a && r > 0 ? (size_t)lora_split((int)E) * r * (H > I ? H : I) * 4 : 0);
  // per-expert gradients: chunk prefixes and the chunk partial sums (at most 2 R / chunk
  // of them, each at most [r, max(2I, H)])
  L.wchunk = take(r > 0 ? 3 * (E + 1) * 4 : 0);
  L.wpart = take(r > 0 ? 2 * (size_t)cdiv((int64_t)R, wgrad_chunk((int64_t)R)) * r * (2 * I > H ? 2 * I : H) * 4 : 0);
  // the routing-weight gradient's partial sums per routed row and down-dgrad column tile
  L.dtwp = take(d->act_quant ? 0 : (size_t)R * cdiv(I, 256) * 4);
  // nested NF4: FP32 absmax' of the larger stack (gate_up), rebuilt before each forward GEMM
  const bool nested = d->w_gu.fmt == BQM_FMT_NF4 && (d->w_gu.nested || d->w_dn.nested);
  L.absx = take(nested ? E * 2 * I * H / 64 * 4 : 0);
  L.total = o;
  return L;
}

bqm_status check_desc(const bqm_moe_desc *d, const char *who) {
  BQM_REQUIRE(d, BQM_ERR_INVALID_ARG, "%s: descriptor is NULL", who);
  BQM_REQUIRE(d->T >= 0 && d->H > 0 && d->I > 0, BQM_ERR_INVALID_ARG, "%s: bad T/H/I", who);
  BQM_REQUIRE(d->H % 64 == 0 && d->I % 64 == 0, BQM_ERR_SHAPE, "%s: H and I must be multiples of 64", who);
  BQM_REQUIRE(d->E >= 1 && d->E <= 1024, BQM_ERR_SHAPE, "%s: E=%d outside [1, 1024]", who, d->E);
  BQM_REQUIRE(d->k >= 1 && d->k <= d->E && d->k <= 16, BQM_ERR_SHAPE, "%s: k=%d outside [1, min(E,16)]", who, d->k);
  BQM_REQUIRE(d->r >= 0 && d->r <= 128 && d->r % 8 == 0, BQM_ERR_SHAPE,
              "%s: r=%d must be a multiple of 8 in [0, 128]", who, d->r);
  BQM_REQUIRE(d->T * d->k < (int64_t)1 << 31, BQM_ERR_SHAPE, "%s: too many routed rows", who);
  BQM_REQUIRE(d->lora_shared_a == 0 || d->lora_shared_a == 1, BQM_ERR_INVALID_ARG,
              "%s: lora_shared_a must be 0 or 1", who);
  const bqm_qtensor *w[2] = {&d->w_gu, &d->w_dn};
  const int64_t rows[2] = {2 * d->I, d->H}, cols[2] = {d->H, d->I};
  for (int i = 0; i < 2; ++i) {
    BQM_REQUIRE(w[i]->fmt == BQM_FMT_NVFP4 || w[i]->fmt == BQM_FMT_NF4, BQM_ERR_INVALID_ARG, "%s: bad weight format", who);
    BQM_REQUIRE(w[i]->fmt == d->w_gu.fmt, BQM_ERR_UNSUPPORTED, "%s: gate_up and down formats differ", who);
    BQM_REQUIRE(w[i]->n_mat == d->E && w[i]->rows == rows[i] && w[i]->cols == cols[i], BQM_ERR_SHAPE,
                "%s: %s stack must be [%d, %lld, %lld]", who, i ? "down" : "gate_up", d->E, (long long)rows[i],
                (long long)cols[i]);
    BQM_REQUIRE(w[i]->codes && w[i]->scales, BQM_ERR_INVALID_ARG, "%s: weight pointers NULL", who);
    BQM_REQUIRE(aligned16(w[i]->codes) && aligned16(w[i]->scales), BQM_ERR_ALIGN, "%s: weight pointers not aligned",
                who);
    if (w[i]->fmt == BQM_FMT_NVFP4) {
      BQM_REQUIRE(w[i]->scale_mode == BQM_SCALE_PER_TENSOR, BQM_ERR_UNSUPPORTED,
                  "%s: NVFP4 weights need one scale per expert matrix", who);
      BQM_REQUIRE(w[i]->s_dec && aligned16(w[i]->s_dec), BQM_ERR_INVALID_ARG, "%s: weight s_dec NULL/unaligned", who);
      BQM_REQUIRE(w[i]->nested == 0, BQM_ERR_INVALID_ARG, "%s: nested is for NF4 only", who);
    } else {
      BQM_REQUIRE(w[i]->nested == 0 || w[i]->nested == 1, BQM_ERR_INVALID_ARG, "%s: nested must be 0 or 1", who);
      if (w[i]->nested)
        BQM_REQUIRE(w[i]->s_dec && aligned16(w[i]->s_dec), BQM_ERR_INVALID_ARG,
                    "%s: nested NF4 weights need s_dec (offset and group scales)", who);
    }
  }
  BQM_REQUIRE(!d->act_quant || d->w_gu.fmt == BQM_FMT_NVFP4, BQM_ERR_UNSUPPORTED,
              "%s: act_quant needs NVFP4 weights", who);
  if (d->r > 0) {
    const void *l[4] = {d->A_gu, d->B_gu, d->A_dn, d->B_dn};
    for (int i = 0; i < 4; ++i) {
      BQM_REQUIRE(l[i], BQM_ERR_INVALID_ARG, "%s: LoRA pointer NULL with r > 0", who);
      BQM_REQUIRE(aligned16(l[i]), BQM_ERR_ALIGN, "%s: LoRA pointer not aligned", who);
    }
  }
  return BQM_OK;
}

struct Ws {
  char *base;
  Layout L;
  template <class T>
  T *at(size_t off) const {
    return reinterpret_cast<T *>(base + off);
  }
};

bqm_status check_ws(const bqm_moe_desc *d, void *ws, size_t ws_bytes, const char *who, Ws &w) {
  w.L = layout(d);
  BQM_REQUIRE(ws && ws_bytes >= w.L.total, BQM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who,
              w.L.total, ws_bytes);
  BQM_REQUIRE(aligned16(ws), BQM_ERR_ALIGN, "%s: workspace not 16-byte aligned", who);
  w.base = reinterpret_cast<char *>(ws);
  return BQM_OK;
}

// upper bound on the tiles of a grouped GEMM: every expert with rows adds at most
// one partial row tile, and at most min(E, R) experts have rows
int gemm_grid(int64_t R, int E, int NT, int bm = BM) {
  const int64_t mt = cdiv(R, bm) + std::min<int64_t>(E, R);
  const int64_t g = std::max<int64_t>(mt * NT, 1);
  return (int)((g + 7) / 8 * 8);
}

Seg seg_bf16(const void *a, int64_t a_ld, const void *b, int64_t b_rows, int64_t b_cols, int K) {
  Seg s{};
  s.a = a;
  s.a_ld = a_ld;
  s.b = b;
  s.b_rows = b_rows;
  s.b_cols = b_cols;
  s.b_estride = b_rows * b_cols;
  s.K = K;
  return s;
}

// A segment whose B is a LoRA-A: with a shared A (one [r, K] matrix read by every
// expert) the expert stride is 0.
Seg lora_a_seg(const bqm_moe_desc *d, Seg s) {
  if (d->lora_shared_a) s.b_estride = 0;
  return s;
}

// The LoRA up-projection segment: A = [R, 2r] hi/lo bf16 pairs, B indexed at k mod r.
// lora_k: the segment runs over K = 2r (hi and lo, FP32-accurate U and V) only in the
// forward with NVFP4 activations, where h decides the rounding of a and with it the
// per-token activation codes; elsewhere it reads the hi halves (K = r), a bf16 LoRA
// operand as in the pages' bf16 module, which is 0.39 ms less over the four GLM GEMMs.
Seg seg_lora(const void *pair_rows, const void *b, int64_t b_rows, int64_t b_cols, int r) {
  Seg s = seg_bf16(pair_rows, 2 * r, b, b_rows, b_cols, 2 * r);
  s.kmod = r;
  return s;
}

Seg seg_q(const void *a, int64_t a_ld, const bqm_qtensor &w, int K) {
  Seg s{};
  s.a = a;
  s.a_ld = a_ld;
  s.b = w.codes;
  s.b_sc = w.scales;
  s.b_sd = w.s_dec;
  s.b_rows = w.rows;
  s.b_cols = w.cols;
  s.b_nested = w.fmt == BQM_FMT_NF4 ? w.nested : 0;
  s.K = K;
  return s;
}

// NVFP4 weights with bf16 activations apply the per-expert s_dec to the whole
// accumulator in the epilogue, so the LoRA intermediates (U in the forward, V in
// the dgrad) that feed the same accumulator are stored divided by it.  With
// NVFP4 activations (forward only) segment 1 is rescaled in-kernel instead.
bool lora_folds_s_dec(const bqm_moe_desc *d, bool forward) {
  return d->w_gu.fmt == BQM_FMT_NVFP4 && !(forward && d->act_quant);
}

// Decode-sized batches: with at most this many routed rows per expert on average the
// forward GEMMs run on 64-row tiles (fq::gemm_fwd_q4n): kNSN LDS stages (76 KB) and
// kOccN workgroups per CU
constexpr int64_t kFewRowsPerExpert = 32;
constexpr int kNSN = 4, kOccN = 2;
bool few_rows(const bqm_moe_desc *d) { return d->T * d->k <= kFewRowsPerExpert * d->E; }

// Decode-sized batches (NVFP4 weights): a forward GEMM streams the weights
// (gv::fwd_stream) with at most this many routed rows per expert on average.  Measured
// on the GLM shape: gate_up streams faster up to 2 rows (its 12 KB activation rows fit
// two per pass), down up to at least 4.
constexpr int64_t kStreamRowsGateUp = 2, kStreamRowsDown = 4;
static_assert(kStreamRowsGateUp <= kFewRowsPerExpert && kStreamRowsDown <= kFewRowsPerExpert,
              "the streaming forward reads the 64-row tile prefix");
bool stream_rows(const bqm_moe_desc *d, int64_t per_expert) {
  return d->w_gu.fmt == BQM_FMT_NVFP4 && d->T * d->k <= per_expert * d->E;
}

// Training-size forward: an expert whose rows past its last full 256-row tile number at
// most kRemRows (rows spread around a multiple of 256) has those rows computed by the
// 64-row kernel (two workgroups per CU) rather than in a mostly empty 256-row tile.
// Both forward GEMMs need K >= 256 (the 64-row kernel's scale groups).
constexpr int kRemRows = 64;
bool rem_split(const bqm_moe_desc *d) { return !few_rows(d) && d->H >= 4 * BK && d->I >= 4 * BK; }

// forward GEMM over 4-bit weights: codes staged in LDS, decoded in registers.
// tile_off_n: the prefix of 64-row tiles per expert, to run the few-rows configuration
// tile_rem: the prefix of remainder tiles (rem_split), computed by the 64-row kernel
// after the 256-row kernel has taken the other tiles
template <int ASRC, int EPI, bool LORN = false, int WF = fq::WF_NVFP4>
bqm_status launch_fq(GemmParams p, int64_t R, hipStream_t s, const char *what, const int32_t *tile_off_n = nullptr,
                     const int32_t *tile_rem = nullptr) {
  static_assert(fq::BM == BM, "tile offsets are computed for BM rows");
  if constexpr (!LORN) {
    if (tile_off_n && p.s1.K >= 4 * BK) {  // scale groups of four K steps
      p.tile_off = tile_off_n;
      fq::gemm_fwd_q4n<ASRC, EPI, WF, kNSN, kOccN><<<gemm_grid(R, p.E, p.NT, fq::BMN), fq::NTHR, 0, s>>>(p);
      return launch_status(what);
    }
  }
  const bool rem = !LORN && tile_rem && p.s1.K >= 4 * BK;
  p.tile_rem = rem ? tile_rem : nullptr;
  const int grid = gemm_grid(R, p.E, p.NT);
  fq::gemm_fwd_q4<ASRC, EPI, LORN, WF><<<grid, fq::NTHR, 0, s>>>(p);
  const bqm_status st = launch_status(what);
  if (st != BQM_OK) return st;
  if constexpr (!LORN) {
    if (rem) {
      p.tile_off = tile_rem;
      p.tile_rem = nullptr;
      p.rem_rows = 1;
      const int64_t g = std::max<int64_t>(std::min<int64_t>(p.E, R) * p.NT, 1);
      fq::gemm_fwd_q4n<ASRC, EPI, WF, kNSN, kOccN><<<(int)((g + 7) / 8 * 8), fq::NTHR, 0, s>>>(p);
      return launch_status(what);
    }
  }
  return BQM_OK;
}

// compute units of the current device (cached per device)
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// weight-streaming forward (few rows per expert): tile_off_n is the prefix of 64-row
// tiles per expert; the output columns go in blocks of gv::COLS (gate_up: 16 i-values)
template <int ASRC, int EPI>
bqm_status launch_gv(GemmParams p, int64_t R, int64_t T, hipStream_t s, const char *what, const int32_t *tile_off_n) {
  p.tile_off = tile_off_n;
  const int NT = (int)(EPI == EPI_GATEUP ? cdiv(p.I, gv::COLS / 2) : cdiv(p.N, gv::COLS));
  // rows per pass: at most RP, as many as fit the LDS budget beside the scales, and never
  // more than T (an expert gets at most one row per token); a pass's rows live in LDS
  const int64_t K = p.s1.K;
  const int64_t Kp = cdiv(K, gv::KB) * gv::KB;
  // the four waves split K when K is long (enough blocks per wave); else each takes a
  // column block, or two waves share one when that leaves fewer workgroups than the
  // chip holds at once (one round: halving each wave's run of dependent blocks beats
  // the extra partial-sum step) and each of the two gets a block
  int ks = K >= gv::KSPLIT_MIN ? gv::NW : 1;
  if (ks == 1 && K >= 2 * gv::KB && p.s2.K <= 32 * 2 * gv::LSL &&
      gemm_grid(R, p.E, (int)cdiv(NT, gv::NW / 2), fq::BMN) <= device_cus() * gv::OCC)
    ks = 2;
  const int64_t xlds = gv::LDS_BUDGET - gv::scale_lds_bytes(K, ks);
  p.rows_pass = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)gv::RP, xlds / (2 * Kp), T}));
  const size_t xb = (size_t)p.rows_pass * Kp * 2;
  const size_t lds = gv::scale_lds_bytes(K, ks) + (ks > 1 ? std::max<size_t>(xb, gv::RED_BYTES) : xb);
  BQM_REQUIRE(ks == 1 || p.s2.K <= 32 * ks * gv::LSL, BQM_ERR_UNSUPPORTED,
              "%s: LoRA K %d above the streaming kernel's %d", what, p.s2.K, 32 * ks * gv::LSL);
  p.NT = (int)cdiv(NT, gv::NW / ks);
  const int grid = gemm_grid(R, p.E, p.NT, fq::BMN);
  if (ks == gv::NW)
    gv::fwd_stream<ASRC, EPI, gv::NW><<<grid, gv::NTHR, lds, s>>>(p);
  else if (ks == 2)
    gv::fwd_stream<ASRC, EPI, 2><<<grid, gv::NTHR, lds, s>>>(p);
  else
    gv::fwd_stream<ASRC, EPI, 1><<<grid, gv::NTHR, lds, s>>>(p);
  return launch_status(what);
}

// LoRA projections (N = r) streamed through LDS by direct copies
// Up to this many tokens the forward's LoRA-A projections run on lora_proj_rows (measured:
// at T = 1 / 8 0.024 / 0.049 ms against 0.066 / 0.067 for gate_up; slower from T = 64)
constexpr int64_t kFewTokens = 16;

template <int ASRC, bool BNM>
bqm_status launch_lp(const GemmParams &p, int64_t R, hipStream_t s, const char *what, int64_t T = -1,
                     const int32_t *tile_off_n = nullptr) {
  static_assert(lp::BM == BM, "tile offsets are computed for BM rows");
  if (!BNM && T >= 0 && T <= kFewTokens && tile_off_n) {
    // one workgroup row per 64-row tile of tile_off_n (one per expert with rows when
    // every token routes to distinct experts); the grid is an upper bound on the tiles
    GemmParams q = p;
    q.tile_off = tile_off_n;
    const int64_t tiles = std::max<int64_t>(cdiv(R, fq::BMN) + std::min<int64_t>(p.E, R), 1);
    lora_proj_rows<ASRC><<<dim3((unsigned)cdiv(p.N, 4), (unsigned)tiles), 256, 0, s>>>(q);
    return launch_status(what);
  }
  const int grid = gemm_grid(R, p.E, p.NT);
  lp::gemm_lora_proj<ASRC, BNM><<<grid, lp::NTHR, 0, s>>>(p);
  return launch_status(what);
}

// dgrad GEMM over the rowwise weight read transposed (codes staged in LDS); tile_off_n
// and tile_rem as for launch_fq (NVFP4 only: the NF4 dgrad keeps the 256-row tiles)
template <int ASRC, int EPI, int WF = fq::WF_NVFP4>
bqm_status launch_fd(GemmParams p, int64_t R, hipStream_t s, const char *what, const int32_t *tile_off_n = nullptr,
                     const int32_t *tile_rem = nullptr) {
  static_assert(fq::BM == BM, "tile offsets are computed for BM rows");
  constexpr bool kQ = WF == fq::WF_NVFP4;
  if (kQ && tile_off_n) {
    p.tile_off = tile_off_n;
    fq::gemm_dgrad_q4n<ASRC, EPI><<<gemm_grid(R, p.E, p.NT, fq::BMN), fq::NTHR, 0, s>>>(p);
    return launch_status(what);
  }
  const bool rem = kQ && tile_rem;
  p.tile_rem = rem ? tile_rem : nullptr;
  fq::gemm_dgrad_q4<ASRC, EPI, WF><<<gemm_grid(R, p.E, p.NT), fq::NTHR, 0, s>>>(p);
  const bqm_status st = launch_status(what);
  if (st != BQM_OK || !rem) return st;
  p.tile_off = tile_rem;
  p.tile_rem = nullptr;
  p.rem_rows = 1;
  const int64_t g = std::max<int64_t>(std::min<int64_t>(p.E, R) * p.NT, 1);
  fq::gemm_dgrad_q4n<ASRC, EPI><<<(int)((g + 7) / 8 * 8), fq::NTHR, 0, s>>>(p);
  return launch_status(what);
}

GemmParams base_params(const bqm_moe_desc *d, const Ws &w) {
  GemmParams p{};
  p.perm = w.at<int32_t>(w.L.perm);
  p.offsets = w.at<int32_t>(w.L.off);
  p.tile_off = w.at<int32_t>(w.L.tile_off);
  p.E = d->E;
  p.k = d->k;
  p.I = (int)d->I;
  p.out_scale = 1.0f;
  return p;
}

#define BQM_TRY(expr)                  \
  do {                                 \
    bqm_status st_ = (expr);           \
    if (st_ != BQM_OK) return st_;     \
  } while (0)

// Records the caller's stage event (start or end) if it asked for timing.
inline void mark(const bqm_moe_desc *d, int stage, int end, hipStream_t s) {
  if (d->stage_events && d->stage_events[2 * stage + end])
    (void)hipEventRecord(reinterpret_cast<hipEvent_t>(d->stage_events[2 * stage + end]), s);
}
#define BQM_STAGE(d, st, s, expr) \
  do {                            \
    mark(d, st, 0, s);            \
    BQM_TRY(expr);                \
    mark(d, st, 1, s);            \
  } while (0)

// rows [n_rows, cols] -> per-row NVFP4 (Four-Over-Six) into the given buffers, and the
// rows of val * sb in bf16 (exact) that the forward GEMMs multiply, their per-row s_dec
// applied to the accumulator (one pass: 4-bitter page, Method)
bqm_status quantize_rows(const uint16_t *x, int64_t n_rows, int64_t cols, uint8_t *codes, uint8_t *scales, float *sd,
                         uint16_t *expanded, hipStream_t s) {
  return nvfp4_quantize_rows_expand(x, n_rows, cols, codes, scales, sd, expanded, s);
}

// The forward GEMMs read NF4 absmax as FP32: a nested stack's absmax' is expanded into
// the workspace first and the segment points at it.
bqm_status nf4_fp32_absmax(const bqm_qtensor &q, const Ws &w, Seg &seg, hipStream_t s) {
  if (q.fmt != BQM_FMT_NF4 || !q.nested) return BQM_OK;
  const int64_t nb = q.rows * q.cols / 64, G = cdiv(nb, 256);
  float *out = w.at<float>(w.L.absx);
  const uint8_t *qs = reinterpret_cast<const uint8_t *>(q.scales);
  if (nb % 4 == 0)
    nf4_unnest<true><<<dim3((unsigned)std::min<int64_t>(cdiv(nb, 1024), 256), (unsigned)q.n_mat), 256, 0, s>>>(
        qs, q.s_dec, nb, G, out);
  else
    nf4_unnest<false><<<dim3((unsigned)std::min<int64_t>(cdiv(nb, 256), 256), (unsigned)q.n_mat), 256, 0, s>>>(
        qs, q.s_dec, nb, G, out);
  seg.b_sc = out;
  seg.b_nested = 0;
  return launch_status("nf4_unnest");
}

// U_gu = s X A_gu^T [R, r] (divided by the expert's s_dec when that folds)
GemmParams lora_a_gu_params(const bqm_moe_desc *d, const Ws &w, const uint16_t *x) {
  GemmParams p = base_params(d, w);
  p.N = d->r;
  p.NT = (int)cdiv(d->r, 64);
  p.s1 = lora_a_seg(d, seg_bf16(x, d->H, d->A_gu, d->r, d->H, (int)d->H));
  p.out_scale = d->lora_scale;
  p.div_e = lora_folds_s_dec(d, true) ? d->w_gu.s_dec : nullptr;
  p.out0 = w.at<uint16_t>(w.L.ugu);
  return p;
}

// Decode-sized batches: the permutation and U_gu in one launch (perm_lora_rows) where
// U_gu would run on the row kernel anyway (at most kFewTokens tokens) and the
// permutation is the one-workgroup form; at most 1024 routed pairs
bool fuse_perm_lora(const bqm_moe_desc *d) {
  const int64_t R = d->T * d->k;
  return d->r > 0 && d->T <= kFewTokens && R > 0 && R <= 1024 && few_rows(d);
}

// u_done: U_gu was computed with the permutation
template <int ASRC_X>
bqm_status fwd_gemms(const bqm_moe_desc *d, const Ws &w, const uint16_t *x, int64_t R, hipStream_t s, bool nf4,
                     bool u_done) {
  const int H = (int)d->H, I = (int)d->I, r = d->r;
  const float ls = d->lora_scale;
  uint16_t *ugu = w.at<uint16_t>(w.L.ugu), *udn = w.at<uint16_t>(w.L.udn);
  float *h = w.at<float>(w.L.h);
  uint16_t *y = w.at<uint16_t>(w.L.y);
  uint16_t *a = w.at<uint16_t>(w.L.a);
  const bool fold_fwd = lora_folds_s_dec(d, true);
  const int32_t *tn = few_rows(d) ? w.at<int32_t>(w.L.tile_off_n) : nullptr;
  const int32_t *trem = rem_split(d) ? w.at<int32_t>(w.L.tile_off_n) : nullptr;  // remainder tiles
  if (r > 0 && !u_done) {
    const GemmParams p = lora_a_gu_params(d, w, x);
    BQM_STAGE(d, BQM_STAGE_LORA_A_GU, s, (launch_lp<A_GATHER, false>(p, R, s, "lora_a gate_up", d->T, tn)));
  }
  // h = X~ W~_gu^T + U_gu B_gu^T; a = silu(g) u
  {
    GemmParams p = base_params(d, w);
    p.N = 2 * I;
    p.NT = (int)cdiv(I, 128);
    constexpr bool aq = ASRC_X == A_GATHER_Q;
    p.s1 = seg_q(aq ? (const void *)w.at<uint16_t>(w.L.xq_b) : (const void *)x, H, d->w_gu, H);
    if (aq) p.s1.a_sd = w.at<float>(w.L.xq_d);
    p.s2 = seg_lora(ugu, d->B_gu, 2 * I, r, r);
    if (!aq) p.s2.K = r;  // bf16 activations: the hi halves (see lora_k)
    p.outf = h;
    p.out1 = a;
    // (NF4 weights take bf16 activations only: check_desc rejects act_quant with them)
    if (nf4) {
      mark(d, BQM_STAGE_GATE_UP_FWD, 0, s);
      BQM_TRY(nf4_fp32_absmax(d->w_gu, w, p.s1, s));
      BQM_TRY((launch_fq<A_GATHER, EPI_GATEUP, false, fq::WF_NF4>(p, R, s, "gate_up fwd", tn, trem)));
      mark(d, BQM_STAGE_GATE_UP_FWD, 1, s);
    } else if (stream_rows(d, kStreamRowsGateUp))
      BQM_STAGE(d, BQM_STAGE_GATE_UP_FWD, s, (launch_gv<ASRC_X, EPI_GATEUP>(p, R, d->T, s, "gate_up fwd", tn)));
    else
      BQM_STAGE(d, BQM_STAGE_GATE_UP_FWD, s, (launch_fq<ASRC_X, EPI_GATEUP>(p, R, s, "gate_up fwd", tn, trem)));
  }
  constexpr bool aq = ASRC_X == A_GATHER_Q;
  if (aq)
    BQM_STAGE(d, BQM_STAGE_ACT_QUANT_A, s,
              quantize_rows(a, R, I, w.at<uint8_t>(w.L.aq_c), w.at<uint8_t>(w.L.aq_s), w.at<float>(w.L.aq_d),
                            w.at<uint16_t>(w.L.aq_b), s));
  // U_dn = s a A_dn^T  [R, r]
  if (r > 0) {
    GemmParams p = base_params(d, w);
    p.N = r;
    p.NT = (int)cdiv(r, 64);
    p.s1 = lora_a_seg(d, seg_bf16(a, I, d->A_dn, r, I, I));
    p.out_scale = ls;
    p.div_e = fold_fwd ? d->w_dn.s_dec : nullptr;
    p.out0 = udn;
    BQM_STAGE(d, BQM_STAGE_LORA_A_DN, s, (launch_lp<A_ROWS, false>(p, R, s, "lora_a down", d->T, tn)));
  }
  // y = a~ W~_dn^T + U_dn B_dn^T
  {
    GemmParams p = base_params(d, w);
    p.N = H;
    p.NT = (int)cdiv(H, 256);
    p.s1 = seg_q(aq ? (const void *)w.at<uint16_t>(w.L.aq_b) : (const void *)a, I, d->w_dn, I);
    if (aq) p.s1.a_sd = w.at<float>(w.L.aq_d);
    p.s2 = seg_lora(udn, d->B_dn, H, r, r);
    if (!aq) p.s2.K = r;
    p.out0 = y;
    if (nf4) {
      mark(d, BQM_STAGE_DOWN_FWD, 0, s);
      BQM_TRY(nf4_fp32_absmax(d->w_dn, w, p.s1, s));
      BQM_TRY((launch_fq<A_ROWS, EPI_STORE, false, fq::WF_NF4>(p, R, s, "down fwd", tn, trem)));
      mark(d, BQM_STAGE_DOWN_FWD, 1, s);
    } else if (stream_rows(d, kStreamRowsDown)) {
      if (aq)
        BQM_STAGE(d, BQM_STAGE_DOWN_FWD, s, (launch_gv<A_ROWS_Q, EPI_STORE>(p, R, d->T, s, "down fwd", tn)));
      else
        BQM_STAGE(d, BQM_STAGE_DOWN_FWD, s, (launch_gv<A_ROWS, EPI_STORE>(p, R, d->T, s, "down fwd", tn)));
    } else if (aq)
      BQM_STAGE(d, BQM_STAGE_DOWN_FWD, s, (launch_fq<A_ROWS_Q, EPI_STORE>(p, R, s, "down fwd", tn, trem)));
    else
      BQM_STAGE(d, BQM_STAGE_DOWN_FWD, s, (launch_fq<A_ROWS, EPI_STORE>(p, R, s, "down fwd", tn, trem)));
  }
  return BQM_OK;
}

}  // namespace
}  // namespace bqm

using namespace bqm;

extern "C" size_t bqm_moe_workspace_size(const bqm_moe_desc *d) {
  if (!d || d->T < 0 || d->k < 1 || d->E < 1 || d->r < 0) return 0;
  return layout(d).total;
}

extern "C" bqm_status bqm_moe_fwd(const bqm_moe_desc *d, const uint16_t *x, const int32_t *topk_idx,
                                  const float *topk_w, uint16_t *out, void *ws, size_t ws_bytes, void *stream) {
  BQM_TRY(check_desc(d, "bqm_moe_fwd"));
  Ws w;
  BQM_TRY(check_ws(d, ws, ws_bytes, "bqm_moe_fwd", w));
  const int64_t R = d->T * d->k;
  hipStream_t s = as_stream(stream);
  if (d->T > 0) {
    BQM_REQUIRE(x && topk_idx && topk_w && out, BQM_ERR_INVALID_ARG, "bqm_moe_fwd: NULL pointer");
    BQM_REQUIRE(aligned16(x) && aligned16(topk_idx) && aligned16(topk_w) && aligned16(out), BQM_ERR_ALIGN,
                "bqm_moe_fwd: pointer not 16-byte aligned");
  }
  const bool fused = fuse_perm_lora(d);
  if (fused) {
    // the permutation (and the copy of the routing weights) with U_gu
    PermArgs pa{topk_idx, (int)R, d->E, w.at<int32_t>(w.L.off), BM, w.at<int32_t>(w.L.tile_off),
                rem_split(d) ? -kRemRows : fq::BMN, w.at<int32_t>(w.L.tile_off_n), w.at<int32_t>(w.L.perm),
                w.at<int32_t>(w.L.inv), topk_w, w.at<float>(w.L.tw)};
    const GemmParams p = lora_a_gu_params(d, w, x);
    // waves per output column: the most that keep the grid within the chip's slots for
    // workgroups of 1024 threads (two per CU)
    int wpc = 4;
    while (wpc > 1 && 1 + R * cdiv(d->r, kPermLoraWaves / wpc) > 2 * (int64_t)device_cus()) wpc /= 2;
    const int grid = 1 + (int)R * (int)cdiv(d->r, kPermLoraWaves / wpc);
    mark(d, BQM_STAGE_PERMUTE, 0, s);
    perm_lora_rows<<<grid, 1024, (d->E + 1) * sizeof(int32_t), s>>>(pa, p, wpc);
    mark(d, BQM_STAGE_PERMUTE, 1, s);
    BQM_TRY(launch_status("permutation and lora_a gate_up"));
  } else {
    BQM_STAGE(d, BQM_STAGE_PERMUTE, s, permute_launch(topk_idx, R, d->E, w.at<int32_t>(w.L.perm), w.at<int32_t>(w.L.inv), w.at<int32_t>(w.L.off),
                           w.at<int32_t>(w.L.counts), BM, w.at<int32_t>(w.L.tile_off),
                           rem_split(d) ? -kRemRows : fq::BMN, w.at<int32_t>(w.L.tile_off_n), s, topk_w,
                           w.at<float>(w.L.tw)));  // (and the copy of the routing weights)
  }
  if (R == 0) return BQM_OK;
  const bool nf4 = d->w_gu.fmt == BQM_FMT_NF4;
  if (d->act_quant) {
    BQM_STAGE(d, BQM_STAGE_ACT_QUANT_X, s,
              quantize_rows(x, d->T, d->H, w.at<uint8_t>(w.L.xq_c), w.at<uint8_t>(w.L.xq_s), w.at<float>(w.L.xq_d),
                            w.at<uint16_t>(w.L.xq_b), s));
    BQM_TRY(fwd_gemms<A_GATHER_Q>(d, w, x, R, s, nf4, fused));
  } else {
    BQM_TRY(fwd_gemms<A_GATHER>(d, w, x, R, s, nf4, fused));
  }
  const int64_t items = d->T * (d->H / 8);
  mark(d, BQM_STAGE_COMBINE_FWD, 0, s);
  combine_rows<<<(int)std::min<int64_t>(cdiv(items, NTHR), 65536), NTHR, 0, s>>>(
      w.at<uint16_t>(w.L.y), w.at<int32_t>(w.L.inv), w.at<int32_t>(w.L.off) + d->E, w.at<float>(w.L.tw), d->T, d->k,
      d->H, out);
  mark(d, BQM_STAGE_COMBINE_FWD, 1, s);
  return launch_status("combine fwd");
}

namespace bqm {
namespace {
// The dgrad.  col_gu / col_dn NULL: the GEMMs read the rowwise weights of d transposed.
// Otherwise they read the columnwise copies (Q(W_gu^T) [E, H, 2I], Q(W_dn^T) [E, I, H])
// K-major on the forward kernel.
bqm_status dgrad_impl(const bqm_moe_desc *d, const bqm_qtensor *col_gu, const bqm_qtensor *col_dn, const uint16_t *dy,
                      void *ws, size_t ws_bytes, uint16_t *dx, float *dtopk_w, void *stream, const char *who) {
  BQM_TRY(check_desc(d, who));
  Ws w;
  BQM_TRY(check_ws(d, ws, ws_bytes, who, w));
  const bool col = col_gu != nullptr;
  const int64_t R = d->T * d->k;
  if (R == 0) return BQM_OK;
  BQM_REQUIRE(dy && dx, BQM_ERR_INVALID_ARG, "%s: NULL pointer", who);
  BQM_REQUIRE(aligned16(dy) && aligned16(dx) && (!dtopk_w || aligned16(dtopk_w)), BQM_ERR_ALIGN,
              "%s: pointer not 16-byte aligned", who);
  hipStream_t s = as_stream(stream);
  const int H = (int)d->H, I = (int)d->I, r = d->r;
  const float ls = d->lora_scale;
  const bool nf4 = d->w_gu.fmt == BQM_FMT_NF4;
  uint16_t *vdn = w.at<uint16_t>(w.L.vdn), *vgu = w.at<uint16_t>(w.L.vgu);
  uint16_t *dh = w.at<uint16_t>(w.L.dh);
  uint16_t *dxr = w.at<uint16_t>(w.L.dxr);
  // the 64-row tiles of the permutation, as in the forward
  const int32_t *tn = few_rows(d) ? w.at<int32_t>(w.L.tile_off_n) : nullptr;
  const int32_t *trem = rem_split(d) ? w.at<int32_t>(w.L.tile_off_n) : nullptr;
  // d(top-k w) = dy . y per routed pair.  With bf16 activations the down dgrad adds up
  // da_u * a per column tile in its epilogue (y is linear in a) and dtopk_sum adds the
  // tiles.  The rows of y are read back instead with NVFP4 activations (y's base term is
  // linear in the quantized a, its LoRA term in the bf16 a) and for the dgrad over
  // columnwise copies (whose DQ(Q(W^T))^T is not the forward's weight).
  const bool fused_dtw = dtopk_w && !d->act_quant && !col;
  if (dtopk_w && !fused_dtw) {
    mark(d, BQM_STAGE_DTOPK, 0, s);
    dtopk_kernel<<<(int)cdiv(R, NTHR / 64), NTHR, 0, s>>>(dy, w.at<uint16_t>(w.L.y), w.at<int32_t>(w.L.inv),
                                                          w.at<int32_t>(w.L.off) + d->E, R, d->k, d->H, dtopk_w);
    mark(d, BQM_STAGE_DTOPK, 1, s);
    BQM_TRY(launch_status("dtopk"));
  }
  // V_dn = s dY B_dn  [R, r]
  if (r > 0) {
    GemmParams p = base_params(d, w);
    p.N = r;
    p.NT = (int)cdiv(r, 64);
    p.s1 = seg_bf16(dy, H, d->B_dn, H, r, H);
    p.out_scale = ls;
    p.div_e = lora_folds_s_dec(d, false) ? (col ? col_dn->s_dec : d->w_dn.s_dec) : nullptr;
    p.out0 = vdn;
    BQM_STAGE(d, BQM_STAGE_LORA_B_DN, s, (launch_lp<A_GATHER, true>(p, R, s, "lora_b^T down")));
  }
  // da_u = dY W~_dn + V_dn A_dn; dh = SwiGLU'(w da_u)
  {
    GemmParams p = base_params(d, w);
    p.N = I;
    p.NT = (int)cdiv(I, 256);
    p.s1 = seg_q(dy, H, col ? *col_dn : d->w_dn, H);
    p.s2 = lora_a_seg(d, seg_lora(vdn, d->A_dn, r, I, r));
    p.s2.K = r;  // the hi halves of V (see lora_k)
    p.out0 = dh;
    p.h_in = w.at<float>(w.L.h);
    p.tw = w.at<float>(w.L.tw);
    p.dtw_part = fused_dtw ? w.at<float>(w.L.dtwp) : nullptr;
    if (col)
      BQM_STAGE(d, BQM_STAGE_DOWN_DGRAD, s, (launch_fq<A_GATHER, EPI_DOWN_DGRAD, true>(p, R, s, "down dgrad (columnwise)")));
    else if (nf4) {
      mark(d, BQM_STAGE_DOWN_DGRAD, 0, s);
      BQM_TRY(nf4_fp32_absmax(d->w_dn, w, p.s1, s));
      BQM_TRY((launch_fd<A_GATHER, EPI_DOWN_DGRAD, fq::WF_NF4>(p, R, s, "down dgrad")));
      mark(d, BQM_STAGE_DOWN_DGRAD, 1, s);
    }
    else
      BQM_STAGE(d, BQM_STAGE_DOWN_DGRAD, s, (launch_fd<A_GATHER, EPI_DOWN_DGRAD>(p, R, s, "down dgrad", tn, trem)));
    if (fused_dtw) {
      mark(d, BQM_STAGE_DTOPK, 0, s);
      dtopk_sum<<<(int)cdiv(R, NTHR), NTHR, 0, s>>>(w.at<float>(w.L.dtwp), p.NT, w.at<int32_t>(w.L.inv),
                                                    w.at<int32_t>(w.L.off) + d->E, R, dtopk_w);
      mark(d, BQM_STAGE_DTOPK, 1, s);
      BQM_TRY(launch_status("dtopk_sum"));
    }
  }
  // V_gu = s dh B_gu  [R, r]
  if (r > 0) {
    GemmParams p = base_params(d, w);
    p.N = r;
    p.NT = (int)cdiv(r, 64);
    p.s1 = seg_bf16(dh, 2 * I, d->B_gu, 2 * I, r, 2 * I);
    p.out_scale = ls;
    p.div_e = lora_folds_s_dec(d, false) ? (col ? col_gu->s_dec : d->w_gu.s_dec) : nullptr;
    p.out0 = vgu;
    BQM_STAGE(d, BQM_STAGE_LORA_B_GU, s, (launch_lp<A_ROWS, true>(p, R, s, "lora_b^T gate_up")));
  }
  // dX_row = dh W~_gu + V_gu A_gu
  {
    GemmParams p = base_params(d, w);
    p.N = H;
    p.NT = (int)cdiv(H, 256);
    p.s1 = seg_q(dh, 2 * I, col ? *col_gu : d->w_gu, 2 * I);
    p.s2 = lora_a_seg(d, seg_lora(vgu, d->A_gu, r, H, r));
    p.s2.K = r;
    p.out0 = dxr;
    if (col)
      BQM_STAGE(d, BQM_STAGE_GATE_UP_DGRAD, s, (launch_fq<A_ROWS, EPI_STORE, true>(p, R, s, "gate_up dgrad (columnwise)")));
    else if (nf4) {
      mark(d, BQM_STAGE_GATE_UP_DGRAD, 0, s);
      BQM_TRY(nf4_fp32_absmax(d->w_gu, w, p.s1, s));
      BQM_TRY((launch_fd<A_ROWS, EPI_STORE, fq::WF_NF4>(p, R, s, "gate_up dgrad")));
      mark(d, BQM_STAGE_GATE_UP_DGRAD, 1, s);
    }
    else
      BQM_STAGE(d, BQM_STAGE_GATE_UP_DGRAD, s, (launch_fd<A_ROWS, EPI_STORE>(p, R, s, "gate_up dgrad", tn, trem)));
  }
  const int64_t items = d->T * (d->H / 8);
  mark(d, BQM_STAGE_COMBINE_DGRAD, 0, s);
  combine_rows<<<(int)std::min<int64_t>(cdiv(items, NTHR), 65536), NTHR, 0, s>>>(
      dxr, w.at<int32_t>(w.L.inv), w.at<int32_t>(w.L.off) + d->E, nullptr, d->T, d->k, d->H, dx);
  mark(d, BQM_STAGE_COMBINE_DGRAD, 1, s);
  return launch_status("combine dgrad");
}
}  // namespace
}  // namespace bqm

extern "C" bqm_status bqm_moe_dgrad(const bqm_moe_desc *d, const uint16_t *dy, void *ws, size_t ws_bytes, uint16_t *dx,
                                    float *dtopk_w, void *stream) {
  return dgrad_impl(d, nullptr, nullptr, dy, ws, ws_bytes, dx, dtopk_w, stream, "bqm_moe_dgrad");
}

extern "C" bqm_status bqm_moe_dgrad_colwise(const bqm_moe_desc *d, const bqm_qtensor *w_gu_col,
                                            const bqm_qtensor *w_dn_col, const uint16_t *dy, void *ws,
                                            size_t ws_bytes, uint16_t *dx, float *dtopk_w, void *stream) {
  const char *who = "bqm_moe_dgrad_colwise";
  BQM_TRY(check_desc(d, who));
  BQM_REQUIRE(w_gu_col && w_dn_col, BQM_ERR_INVALID_ARG, "%s: columnwise copies are NULL", who);
  BQM_REQUIRE(d->w_gu.fmt == BQM_FMT_NVFP4 && w_gu_col->fmt == BQM_FMT_NVFP4 && w_dn_col->fmt == BQM_FMT_NVFP4,
              BQM_ERR_UNSUPPORTED, "%s: NVFP4 weights only", who);
  BQM_REQUIRE(w_gu_col->scale_mode == BQM_SCALE_PER_TENSOR && w_dn_col->scale_mode == BQM_SCALE_PER_TENSOR,
              BQM_ERR_INVALID_ARG, "%s: columnwise copies need per-tensor scales", who);
  BQM_REQUIRE(w_gu_col->n_mat == d->E && w_gu_col->rows == d->H && w_gu_col->cols == 2 * d->I, BQM_ERR_SHAPE,
              "%s: w_gu_col must be [E, H, 2I]", who);
  BQM_REQUIRE(w_dn_col->n_mat == d->E && w_dn_col->rows == d->I && w_dn_col->cols == d->H, BQM_ERR_SHAPE,
              "%s: w_dn_col must be [E, I, H]", who);
  BQM_REQUIRE(w_gu_col->codes && w_gu_col->scales && w_gu_col->s_dec && w_dn_col->codes && w_dn_col->scales &&
                  w_dn_col->s_dec,
              BQM_ERR_INVALID_ARG, "%s: NULL pointer in a columnwise copy", who);
  BQM_REQUIRE(aligned16(w_gu_col->codes) && aligned16(w_dn_col->codes), BQM_ERR_ALIGN,
              "%s: codes not 16-byte aligned", who);
  return dgrad_impl(d, w_gu_col, w_dn_col, dy, ws, ws_bytes, dx, dtopk_w, stream, who);
}

extern "C" bqm_status bqm_lora_grad(const bqm_moe_desc *d, const uint16_t *x, const uint16_t *dy, void *ws,
                                    size_t ws_bytes, float *dA_gu, float *dB_gu, float *dA_dn, float *dB_dn,
                                    void *stream) {
  BQM_TRY(check_desc(d, "bqm_lora_grad"));
  BQM_REQUIRE(d->r > 0, BQM_ERR_INVALID_ARG, "bqm_lora_grad: r must be > 0");
  Ws w;
  BQM_TRY(check_ws(d, ws, ws_bytes, "bqm_lora_grad", w));
  BQM_REQUIRE(dA_gu && dB_gu && dA_dn && dB_dn, BQM_ERR_INVALID_ARG, "bqm_lora_grad: NULL output");
  BQM_REQUIRE(aligned16(dA_gu) && aligned16(dB_gu) && aligned16(dA_dn) && aligned16(dB_dn), BQM_ERR_ALIGN,
              "bqm_lora_grad: output not 16-byte aligned");
  if (d->T > 0) {
    BQM_REQUIRE(x && dy, BQM_ERR_INVALID_ARG, "bqm_lora_grad: x and dy are required");
    BQM_REQUIRE(aligned16(x) && aligned16(dy), BQM_ERR_ALIGN, "bqm_lora_grad: x/dy not 16-byte aligned");
  }
  hipStream_t s = as_stream(stream);
  const int H = (int)d->H, I = (int)d->I, r = d->r;
  WgradParams p{};
  p.perm = w.at<int32_t>(w.L.perm);
  p.offsets = w.at<int32_t>(w.L.off);
  p.tw = w.at<float>(w.L.tw);
  p.k = d->k;
  p.E = d->E;
  const int split = lora_split(d->E);
  const int64_t R = d->T * d->k;
  p.chunk = wgrad_chunk(R);
  int32_t *chunk_off = w.at<int32_t>(w.L.wchunk);
  p.chunk_off = chunk_off;
  p.slot_off = chunk_off + d->E + 1;
  p.part = w.at<float>(w.L.wpart);
  const int32_t *multi = chunk_off + 2 * (d->E + 1);
  wgrad_chunks<<<1, 1024, 0, s>>>(p.offsets, d->E, p.chunk, chunk_off, chunk_off + d->E + 1,
                                  chunk_off + 2 * (d->E + 1));
  BQM_TRY(launch_status("lora grad chunks"));
  // bounds: sum over e of max(1, ceil(n_e / chunk)) <= E + R / chunk chunks, and at most
  // R / chunk experts have more than one
  const unsigned n_chunks = (unsigned)(d->E + R / p.chunk);
  const unsigned n_multi = (unsigned)std::max<int64_t>(1, std::min<int64_t>(d->E, R / p.chunk));
  // shared: C is the one [M, N] gradient of a shared A, summed over the experts in
  // `split` parts (partials in the workspace, then added in part order)
  auto go = [&](int M, int N, const uint16_t *P, int64_t pld, int pg, int sp, const uint16_t *Q, int64_t qld, int qg,
                const float *cs, float *C, bool shared, const char *what) {
    p.M = M;
    p.N = N;
    p.P = P;
    p.p_ld = pld;
    p.p_gather = pg;
    p.scale_p = sp;
    p.Q = Q;
    p.q_ld = qld;
    p.q_gather = qg;
    p.c_scale = cs;
    p.split = shared ? split : 0;
    p.C = shared ? w.at<float>(w.L.part) : C;
    dim3 grid((unsigned)(cdiv(M, WB) * cdiv(N, WB)), shared ? (unsigned)split : n_chunks);
    if (shared) lora_wgrad<true><<<grid, NTHR, 0, s>>>(p);
    else lora_wgrad<false><<<grid, NTHR, 0, s>>>(p);
    BQM_TRY(launch_status(what));
    if (!shared) {
      const int64_t n4 = (int64_t)M * N / 4;
      wgrad_sum_chunks<<<dim3((unsigned)std::min<int64_t>(cdiv(n4, NTHR), 64), n_multi), NTHR, 0, s>>>(
          reinterpret_cast<const float4 *>(p.part), p.chunk_off, p.slot_off, multi, cs, n4,
          reinterpret_cast<float4 *>(C));
      BQM_TRY(launch_status(what));
    }
    if (shared) {
      const int64_t n4 = (int64_t)M * N / 4;
      sum_parts<<<(unsigned)cdiv(n4, NTHR), NTHR, 0, s>>>(reinterpret_cast<const float4 *>(p.C), split, n4,
                                                          reinterpret_cast<float4 *>(C));
      BQM_TRY(launch_status(what));
    }
    return BQM_OK;
  };
  const bool sh = d->lora_shared_a != 0;
  const uint16_t *dh = w.at<uint16_t>(w.L.dh), *ugu = w.at<uint16_t>(w.L.ugu), *vgu = w.at<uint16_t>(w.L.vgu);
  const uint16_t *udn = w.at<uint16_t>(w.L.udn), *vdn = w.at<uint16_t>(w.L.vdn), *a = w.at<uint16_t>(w.L.a);
  // dB_gu [2I, r] = dh^T U_gu' ; dA_gu [r, H] = V_gu'^T X ; U' and V' already carry the LoRA scale
  mark(d, BQM_STAGE_LORA_GRAD, 0, s);
  // (U, V divided by s_dec where that folds: the expert's factor is restored on the output)
  const float *fu_gu = lora_folds_s_dec(d, true) ? d->w_gu.s_dec : nullptr;
  const float *fv_gu = lora_folds_s_dec(d, false) ? d->w_gu.s_dec : nullptr;
  const float *fu_dn = lora_folds_s_dec(d, true) ? d->w_dn.s_dec : nullptr;
  const float *fv_dn = lora_folds_s_dec(d, false) ? d->w_dn.s_dec : nullptr;
  BQM_TRY(go(2 * I, r, dh, 2 * I, 0, 0, ugu, 2 * r, 0, fu_gu, dB_gu, false, "lora dB_gu"));
  BQM_TRY(go(r, H, vgu, 2 * r, 0, 0, x, H, 1, fv_gu, dA_gu, sh, "lora dA_gu"));
  // dB_dn [H, r] = (w dY)^T U_dn' ; dA_dn [r, I] = (w V_dn')^T a
  BQM_TRY(go(H, r, dy, H, 1, 1, udn, 2 * r, 0, fu_dn, dB_dn, false, "lora dB_dn"));
  BQM_TRY(go(r, I, vdn, 2 * r, 0, 1, a, I, 0, fv_dn, dA_dn, sh, "lora dA_dn"));
  mark(d, BQM_STAGE_LORA_GRAD, 1, s);
  return BQM_OK;
}
