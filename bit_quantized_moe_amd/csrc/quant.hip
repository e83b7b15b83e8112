// NVFP4 (Four-Over-Six) and NF4 quantizers and dequantizers for gfx950.
//
// NVFP4: one E4M3 scale per 16 consecutive elements along the last axis and
// one FP32 scale per 2-D matrix (weights) or per row (token activations); each
// block tries the scale t/6 and t/4 and keeps the one whose FP32 squared error,
// measured against the target scaled down once by the inverse of
// amax / (6 * M), is lower (4-bitter page, section "Four-Over-Six for RL
// Weights and Activations"; GLM page, section "Why can't we just transpose the
// one copy?").  NF4: blocksize 64, FP32 absmax (nf4moe page, section "The fix:
// dequant-on-forward for routed experts").
//
// Every rounding is a single IEEE round-to-nearest-even operation (this file is
// compiled with -ffp-contract=off and correctly rounded FP32 division), so codes
// and scales are deterministic bit patterns.
//
// Memory layout: one thread owns one 16-element block (32 bytes of bf16 in,
// 8 bytes of codes and 1 scale byte out); consecutive threads own consecutive
// blocks, so a wave reads 2 KB and writes 512 B of codes contiguously.  The
// per-tensor amax is a separate pass (one atomicMax per workgroup into the
// matrix's slot) before the quantize pass.
#include "common.h"
#include "internal.h"
#include "nf4_levels.inc"

#include <algorithm>
#include <mutex>

namespace bqm {
namespace {

constexpr int kThreads = 256;

// Streaming (non-temporal) accesses: every byte these kernels read or write is touched
// once, so the loads and stores carry the non-temporal hint (measured: per-tensor
// quantize 8.4 -> 7.9 ms, NF4 quantize 5.0 -> 4.6 ms over the two GLM stacks).
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
  const nt_u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st_nt(uint4 *p, uint4 v) {
  const nt_u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<nt_u32x4 *>(p));
}
__device__ __forceinline__ void st_nt(uint2 *p, uint2 v) {
  const nt_u32x2 x = {v.x, v.y};
  __builtin_nontemporal_store(x, reinterpret_cast<nt_u32x2 *>(p));
}

// fl(t / 6) without a division: q = fl(t * fl(1/6)), the remainder t - 6 q exact in one
// fma, then one fma correction.  Checked exhaustively against the correctly rounded
// quotient: equal for every finite float t >= 2^-119; below that both are far under the
// smallest E4M3 step (2^-9), so the block scale is code 0 either way.
__device__ __forceinline__ float div6(float t) {
  const float r6 = 0x1.555556p-3f;  // fl(1/6)
  const float q = t * r6;
  const float r = __builtin_fmaf(-q, 6.0f, t);
  return __builtin_fmaf(r, r6, q);
}

// E4M3FN codes of two non-negative finite floats, each rounded to nearest even and
// saturated at 448, in one hardware conversion.  Clamping to 448 first is the same
// saturation: every value in [448, 464) rounds to 448, and E4M3FN has nothing above.
__device__ __forceinline__ void e4m3_pair(float a, float b, uint32_t &ca, uint32_t &cb) {
  const uint32_t p = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(a, 448.0f), fminf(b, 448.0f), 0, false);
  ca = p & 0xFFu;
  cb = (p >> 8) & 0xFFu;
}

// One scale candidate: E2M1 codes of y * r (the hardware conversion rounds to
// nearest, ties to even, saturating at 6, and keeps the sign) and the squared
// error of the decoded values against y, summed in element order 0..15 in FP32.
// Signs cancel in the error: |y| - |q| sb = +-(y - q sb).
typedef __attribute__((ext_vector_type(2))) float f32x2;

__device__ __forceinline__ float candidate(const float (&y)[16], float sb, float r, uint32_t &c_lo,
                                           uint32_t &c_hi) {
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const float v0 = y[2 * p] * r, v1 = y[2 * p + 1] * r;
    switch (p & 3) {
      case 0: c[p >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[p >> 2], v0, v1, 1.0f, 0); break;
      case 1: c[p >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[p >> 2], v0, v1, 1.0f, 1); break;
      case 2: c[p >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[p >> 2], v0, v1, 1.0f, 2); break;
      default: c[p >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[p >> 2], v0, v1, 1.0f, 3); break;
    }
  }
  float err = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    f32x2 q;
    switch (p & 3) {
      case 0: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 0); break;
      case 1: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 1); break;
      case 2: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 2); break;
      default: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 3); break;
    }
    // q*sb is exact (<= 6 significant bits), so the fused form rounds y - q*sb once, as
    // the separate product and difference do
    const float d0 = __builtin_fmaf(-q.x, sb, y[2 * p]);
    err = err + d0 * d0;
    const float d1 = __builtin_fmaf(-q.y, sb, y[2 * p + 1]);
    err = err + d1 * d1;
  }
  c_lo = c[0];
  c_hi = c[1];
  return err;
}

// The strict FP32 form of a candidate's error (the reference the 4-bitter page's fast
// path is measured against): each candidate value is scaled back up to the original
// domain, fl(fl(q * sb) * s_dec) (q * sb exact), and compared with the original x:
// sum of fl(d * d), d = fl(x - that), in element order in FP32.  The codes are the same
// as candidate()'s.
__device__ __forceinline__ float strict_error(const float (&x)[16], float sb, float s_dec, uint32_t c_lo,
                                              uint32_t c_hi) {
  const uint32_t c[2] = {c_lo, c_hi};
  float err = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    f32x2 q;
    switch (p & 3) {
      case 0: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 0); break;
      case 1: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 1); break;
      case 2: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 2); break;
      default: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[p >> 2], 1.0f, 3); break;
    }
    const float d0 = x[2 * p] - (q.x * sb) * s_dec;
    err = err + d0 * d0;
    const float d1 = x[2 * p + 1] - (q.y * sb) * s_dec;
    err = err + d1 * d1;
  }
  return err;
}

// 4/6 modes: off (scale t/6 only), the scaled-domain error (target scaled down once),
// and the strict FP32 reference error
constexpr int kFosOff = 0, kFosScaled = 1, kFosStrict = 2;

// Quantize one block of 16 bf16 values held as 8 words; returns the E4M3 code.
// rcp[c] = fl(1 / e4m3(c)) (0 for c = 0).
template <int kMode>
__device__ __forceinline__ uint32_t quant_block16(const uint32_t (&w)[8], float s_enc, float s_dec, const float *rcp,
                                                  uint32_t &lo, uint32_t &hi) {
  float y[16];
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = bf16_lo(w[i]) * s_enc;
    y[2 * i + 1] = bf16_hi(w[i]) * s_enc;
    t = fmaxf(t, fmaxf(fabsf(y[2 * i]), fabsf(y[2 * i + 1])));
  }
  uint32_t sb6, sb4;
  e4m3_pair(div6(t), t * 0.25f, sb6, sb4);  // t * 0.25 == t/4 exactly rounded
  const float f6 = __builtin_amdgcn_cvt_f32_fp8(sb6, 0);
  float e6 = candidate(y, f6, rcp[sb6], lo, hi);
  uint32_t sb = sb6;
  if (kMode != kFosOff) {
    if (sb4 != sb6) {
      uint32_t l4, h4;
      const float f4 = __builtin_amdgcn_cvt_f32_fp8(sb4, 0);
      float e4 = candidate(y, f4, rcp[sb4], l4, h4);
      if (kMode == kFosStrict) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x[2 * i] = bf16_lo(w[i]);
          x[2 * i + 1] = bf16_hi(w[i]);
        }
        e6 = strict_error(x, f6, s_dec, lo, hi);
        e4 = strict_error(x, f4, s_dec, l4, h4);
      }
      if (e4 < e6) {
        sb = sb4;
        lo = l4;
        hi = h4;
      }
    }
  }
  return sb;
}

// Fills rcp[0..127) with fl(1 / e4m3(c)) (rcp[0] = 0); the block synchronizes.
__device__ __forceinline__ void fill_rcp(float *rcp) {
  if (threadIdx.x < 127) {
    const float v = e4m3_to_f32(threadIdx.x);
    rcp[threadIdx.x] = threadIdx.x ? 1.0f / v : 0.0f;
  }
  __syncthreads();
}

__device__ __forceinline__ void load_block16(const uint4 *p, uint32_t (&w)[8]) {
  const uint4 a = ld_nt(p), b = ld_nt(p + 1);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

__device__ __forceinline__ uint32_t absmax_bits_u32(uint32_t w) {
  uint32_t a = w & 0x7FFFu, b = (w >> 16) & 0x7FFFu;
  return a > b ? a : b;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t t = __shfl_xor(v, o, 64);
    v = v > t ? v : t;
  }
  return v;
}

// Block-wide max of non-negative values; every thread gets the result.
__device__ __forceinline__ uint32_t block_max_u(uint32_t v, uint32_t *red) {
  v = wave_max_u(v);
  int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  uint32_t m = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = m > red[i] ? m : red[i];
  __syncthreads();
  return m;
}

// Decode scale from amax: s_dec = fl(A / fl(6M)), s_enc = fl(1 / s_dec).
__device__ __forceinline__ void global_scale(float amax, float denom, float &s_dec, float &s_enc) {
  s_dec = amax > 0.0f ? amax / denom : 1.0f;
  s_enc = 1.0f / s_dec;
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// Per-tensor quantizer in two launches over the whole stack: the amax pass
// (every 16-byte vector read once, a block max, one atomicMax per workgroup
// into the matrix's slot) and the quantize pass, which reads the final amax.
// The second read of the input is inherent to a per-tensor scale; callers
// that already hold the scales pass them in and skip the first launch.
constexpr int64_t kAmaxVec = 16384;     // 128K elements per amax chunk
constexpr int64_t kQuantBlocks = 2048;  // 32K elements per quantize chunk

__global__ void __launch_bounds__(kThreads) clear_u32(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) p[i] = 0u;
}

// grid = n_mat * P workgroups
__global__ void __launch_bounds__(kThreads) nvfp4_amax(const uint4 *__restrict__ x, int64_t vec_per_mat, int64_t P,
                                                       uint32_t *__restrict__ amax) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x / P, c = blockIdx.x % P;
  const uint4 *xm = x + m * vec_per_mat;
  const int64_t b = c * kAmaxVec, e = b + kAmaxVec < vec_per_mat ? b + kAmaxVec : vec_per_mat;
  uint32_t mx = 0u;
  for (int64_t j = b + threadIdx.x; j < e; j += kThreads) {
    const uint4 v = ld_nt(&xm[j]);
    uint32_t a0 = absmax_bits_u32(v.x), a1 = absmax_bits_u32(v.y);
    uint32_t a2 = absmax_bits_u32(v.z), a3 = absmax_bits_u32(v.w);
    a0 = a0 > a1 ? a0 : a1;
    a2 = a2 > a3 ? a2 : a3;
    a0 = a0 > a2 ? a0 : a2;
    mx = mx > a0 ? mx : a0;
  }
  mx = block_max_u(mx, red);
  if (threadIdx.x == 0) atomicMax(&amax[m], mx);
}

// grid = n_mat * G workgroups; s_dec from amax (bf16 magnitude bits) or s_dec_in
template <int kMode>
__global__ void __launch_bounds__(kThreads) nvfp4_quant_tensor(
    const uint4 *__restrict__ x, int64_t blocks_per_mat, int64_t G, const uint32_t *__restrict__ amax,
    const float *__restrict__ s_dec_in, float denom, uint2 *__restrict__ codes, uint8_t *__restrict__ scales,
    float *__restrict__ s_dec_out) {
  __shared__ float rcp[128];
  fill_rcp(rcp);
  const int64_t m = blockIdx.x / G, c = blockIdx.x % G;
  float s_dec, s_enc;
  if (s_dec_in) {
    s_dec = s_dec_in[m];
    s_enc = 1.0f / s_dec;
  } else {
    global_scale(__uint_as_float(amax[m] << 16), denom, s_dec, s_enc);
  }
  if (c == 0 && threadIdx.x == 0) s_dec_out[m] = s_dec;
  const uint4 *xm = x + m * blocks_per_mat * 2;
  uint2 *cm = codes + m * blocks_per_mat;
  uint8_t *sm = scales + m * blocks_per_mat;
  const int64_t b = c * kQuantBlocks, e = b + kQuantBlocks < blocks_per_mat ? b + kQuantBlocks : blocks_per_mat;
  for (int64_t blk = b + threadIdx.x; blk < e; blk += kThreads) {
    uint32_t w[8];
    load_block16(xm + 2 * blk, w);
    uint32_t lo, hi;
    const uint32_t sb = quant_block16<kMode>(w, s_enc, s_dec, rcp, lo, hi);
    st_nt(&cm[blk], make_uint2(lo, hi));
    __builtin_nontemporal_store((uint8_t)sb, &sm[blk]);
  }
}

// bf16 pair P (elements 2P, 2P+1) of a code word times its block scale: exact
template <int P>
__device__ __forceinline__ uint32_t nvfp4_val_sb(uint32_t c, float sb) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, P);
  return pack_bf16_rne(v.x * sb, v.y * sb);
}

// block `idx` (row-major over the rows) of the per-row quantizer: codes, scale and,
// with kExp, the bf16 values times the block scale
template <int kMode, bool kExp>
__device__ __forceinline__ void quant_row_block(const uint32_t (&w)[8], int64_t idx, float s_enc, float s_dec,
                                                const float *rcp, uint2 *__restrict__ codes,
                                                uint8_t *__restrict__ scales, uint4 *__restrict__ expanded) {
  uint32_t lo, hi;
  const uint32_t sb = quant_block16<kMode>(w, s_enc, s_dec, rcp, lo, hi);
  codes[idx] = make_uint2(lo, hi);
  scales[idx] = (uint8_t)sb;
  if constexpr (kExp) {
    const float sbf = __builtin_amdgcn_cvt_f32_fp8(sb, 0);
    uint4 *y = expanded + 2 * idx;
    y[0] = make_uint4(nvfp4_val_sb<0>(lo, sbf), nvfp4_val_sb<1>(lo, sbf), nvfp4_val_sb<2>(lo, sbf),
                      nvfp4_val_sb<3>(lo, sbf));
    y[1] = make_uint4(nvfp4_val_sb<0>(hi, sbf), nvfp4_val_sb<1>(hi, sbf), nvfp4_val_sb<2>(hi, sbf),
                      nvfp4_val_sb<3>(hi, sbf));
  }
}

constexpr int kRowKeep = 4;  // blocks per lane the per-row quantizer keeps in registers

// Per-row quantizer: one wave per row (the per-token activation scale, computed
// across the row in the same kernel).  rows_total = n_mat * rows.  kExp: the same
// pass also writes each block's values times its block scale as bf16 (exact), the
// rows the W4A4 GEMMs multiply (their per-row s_dec goes on the accumulator).
template <int kMode, bool kExp = false>
__global__ void __launch_bounds__(kThreads) nvfp4_quant_rows(
    const uint4 *__restrict__ x, int64_t rows_total, int64_t blocks_per_row,
    const float *__restrict__ s_dec_in, float denom, uint2 *__restrict__ codes,
    uint8_t *__restrict__ scales, float *__restrict__ s_dec_out, uint4 *__restrict__ expanded = nullptr) {
  __shared__ float rcp[128];
  fill_rcp(rcp);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows_total) return;
  const uint4 *xr = x + row * blocks_per_row * 2;
  float s_dec, s_enc;
  // Rows of at most 64 kRowKeep blocks stay in registers between the row maximum and
  // the quantization (each lane holds its blocks lane, lane + 64, ...): one read of
  // the row, one memory round trip per row instead of two.
  if (!s_dec_in && blocks_per_row <= 64 * kRowKeep) {
    uint32_t w[kRowKeep][8];
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < kRowKeep; ++j) {
      const int64_t blk = lane + 64 * j;
      if (blk < blocks_per_row) {
        load_block16(xr + 2 * blk, w[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t a = absmax_bits_u32(w[j][i]);
          mx = mx > a ? mx : a;
        }
      }
    }
    mx = wave_max_u(mx);
    global_scale(__uint_as_float(mx << 16), denom, s_dec, s_enc);
    if (lane == 0) s_dec_out[row] = s_dec;
#pragma unroll
    for (int j = 0; j < kRowKeep; ++j) {
      const int64_t blk = lane + 64 * j;
      if (blk < blocks_per_row) quant_row_block<kMode, kExp>(w[j], row * blocks_per_row + blk, s_enc, s_dec, rcp,
                                                             codes, scales, expanded);
    }
    return;
  }
  if (s_dec_in) {
    s_dec = s_dec_in[row];
    s_enc = 1.0f / s_dec;
  } else {
    uint32_t mx = 0u;
    for (int64_t i = lane; i < blocks_per_row * 2; i += 64) {
      uint4 v = xr[i];
      uint32_t a = absmax_bits_u32(v.x), c = absmax_bits_u32(v.y);
      uint32_t d = absmax_bits_u32(v.z), f = absmax_bits_u32(v.w);
      a = a > c ? a : c;
      d = d > f ? d : f;
      a = a > d ? a : d;
      mx = mx > a ? mx : a;
    }
    mx = wave_max_u(mx);
    global_scale(__uint_as_float(mx << 16), denom, s_dec, s_enc);
  }
  if (lane == 0) s_dec_out[row] = s_dec;
  for (int64_t blk = lane; blk < blocks_per_row; blk += 64) {
    uint32_t w[8];
    load_block16(xr + 2 * blk, w);
    quant_row_block<kMode, kExp>(w, row * blocks_per_row + blk, s_enc, s_dec, rcp, codes, scales, expanded);
  }
}

// ---------------------------------------------------------------------------
// Dequantizers and the NF4 quantizer: one lane per 8 consecutive elements (one
// 32-bit word of codes, 16 bytes of bf16), so every load and store instruction
// of a wave covers contiguous memory; a workgroup takes kDqUnits consecutive
// 8-element units.
// ---------------------------------------------------------------------------
constexpr int kDqIter = 4;
constexpr int64_t kDqUnits = (int64_t)kDqIter * kThreads;

// Segment (a run of seg_units units sharing one decode scale) of unit u, for the
// units of one workgroup: seg0 is the segment of its first unit, `first` that
// segment's first unit, so u - first < kDqUnits + seg_units.
__device__ __forceinline__ int64_t seg_of(int64_t u, int64_t seg0, int64_t first, int64_t seg_units) {
  const uint32_t off = (uint32_t)(u - first);
  if (seg_units >= kDqUnits) return seg0 + (off >= (uint32_t)seg_units ? 1 : 0);
  return seg0 + off / (uint32_t)seg_units;
}

// byte P of a code word: elements 2P (low nibble) and 2P+1, decoded with their sign
// (a zero magnitude with the sign bit set gives -0) and scaled: fl(fl(v * sb) * sd)
// with v * sb exact
template <int P>
__device__ __forceinline__ uint32_t nvfp4_dq_pair(uint32_t c, float sb, float sd) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, P);
  return pack_bf16_rne((v.x * sb) * sd, (v.y * sb) * sd);
}

// NVFP4 dequantize: bf16(fl(fl(val * sb) * s_dec)).  seg_units: units per s_dec
// (a whole matrix, or one row in per-row mode).  Without kSdec the output is val * sb
// alone, exact in bf16 (at most 6 significant bits): the scaled-domain values that a
// GEMM multiplies, with s_dec applied to its accumulator.
template <bool kSdec>
__global__ void __launch_bounds__(kThreads) nvfp4_dequant(const uint32_t *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales,
                                                          const float *__restrict__ s_dec, int64_t nunits,
                                                          int64_t seg_units, uint4 *__restrict__ y) {
  const int64_t base = (int64_t)blockIdx.x * kDqUnits;
  const int64_t seg0 = base / seg_units, first = seg0 * seg_units;
  uint32_t c[kDqIter];
  uint32_t sbc[kDqIter];
  float sd[kDqIter];
#pragma unroll
  for (int it = 0; it < kDqIter; ++it) {
    const int64_t u0 = base + it * kThreads + threadIdx.x;
    const int64_t u = u0 < nunits ? u0 : nunits - 1;
    c[it] = codes[u];
    sbc[it] = scales[u >> 1];
    sd[it] = kSdec ? s_dec[seg_of(u, seg0, first, seg_units)] : 1.0f;
  }
#pragma unroll
  for (int it = 0; it < kDqIter; ++it) {
    const int64_t u = base + it * kThreads + threadIdx.x;
    if (u < nunits) {
      const float sb = __builtin_amdgcn_cvt_f32_fp8(sbc[it], 0);
      st_nt(&y[u], make_uint4(nvfp4_dq_pair<0>(c[it], sb, sd[it]), nvfp4_dq_pair<1>(c[it], sb, sd[it]),
                              nvfp4_dq_pair<2>(c[it], sb, sd[it]), nvfp4_dq_pair<3>(c[it], sb, sd[it])));
    }
  }
}

__constant__ float c_nf4_levels[16] = BQM_NF4_LEVELS;
__constant__ float c_nf4_mids[15] = BQM_NF4_MIDPOINTS;

// NF4 code of xn = #{j : xn > mid_j} from one table entry: bucket b = trunc(64 xn + 64)
// clamped to [0, 127] covers xn in about [b/64 - 1, (b+1)/64 - 1]; entry b holds the
// number of midpoints below that range (widened by kNf4Margin, far more than the
// rounding of the bucket arithmetic) and the one midpoint inside it, or +inf.  The
// midpoints are at least 0.08 apart, so no widened range holds two.
constexpr float kNf4Margin = 1e-5f;

__device__ __forceinline__ void fill_nf4_table(uint2 *tbl) {
  if (threadIdx.x < 128) {
    const int b = threadIdx.x;
    const float lo = b == 0 ? -INFINITY : (float)(b - 64) / 64.0f - kNf4Margin;
    const float hi = b == 127 ? INFINITY : (float)(b - 63) / 64.0f + kNf4Margin;
    uint32_t below = 0;
    float inside = INFINITY;
    for (int j = 0; j < 15; ++j) {
      const float m = c_nf4_mids[j];
      if (m < lo)
        ++below;
      else if (m <= hi)
        inside = m;
    }
    tbl[b] = make_uint2(below, __float_as_uint(inside));
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t nf4_code(float xn, const uint2 *tbl) {
  int b = (int)__builtin_fmaf(xn, 64.0f, 64.0f);
  b = b < 0 ? 0 : (b > 127 ? 127 : b);
  const uint2 t = tbl[b];
  return t.x + (xn > __uint_as_float(t.y) ? 1u : 0u);
}

// NF4 quantize: 8 lanes per 64-block (absmax reduced across them), each lane
// codes its 8 elements into one word.
__global__ void __launch_bounds__(kThreads) nf4_quant(const uint4 *__restrict__ x, int64_t nunits,
                                                      uint32_t *__restrict__ codes, float *__restrict__ absmax) {
  __shared__ uint2 tbl[128];
  fill_nf4_table(tbl);
  const int64_t base = (int64_t)blockIdx.x * kDqUnits;
  uint4 v[kDqIter];
#pragma unroll
  for (int it = 0; it < kDqIter; ++it) {
    const int64_t u0 = base + it * kThreads + threadIdx.x;
    v[it] = ld_nt(&x[u0 < nunits ? u0 : nunits - 1]);
  }
#pragma unroll
  for (int it = 0; it < kDqIter; ++it) {
    const int64_t u = base + it * kThreads + threadIdx.x;
    const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
    uint32_t mx = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m = absmax_bits_u32(w[i]);
      mx = mx > m ? mx : m;
    }
    // nunits is a multiple of 8, so an 8-lane group is entirely in range or entirely out
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const uint32_t t = __shfl_xor(mx, o, 64);
      mx = mx > t ? mx : t;
    }
    const float a = __uint_as_float(mx << 16);
    const float r = a > 0.0f ? 1.0f / a : 0.0f;
    uint32_t code = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xv = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
      code |= nf4_code(xv * r, tbl) << (4 * i);
    }
    if (u < nunits) {
      __builtin_nontemporal_store(code, &codes[u]);
      if ((threadIdx.x & 7) == 0) absmax[u >> 3] = a;
    }
  }
}

// Nested absmax of one NF4 block: fl(fl(e4m3(q) * s2) + offset) (this file is
// compiled without contraction, so the two roundings stay separate)
__device__ __forceinline__ float nested_absmax(uint32_t q, const float *sdm, uint32_t blk) {
  return __builtin_amdgcn_cvt_f32_fp8(q, 0) * sdm[1 + (blk >> 8)] + sdm[0];
}

// NF4 dequantize: bf16(fl(level[code] * absmax)); kNested: absmax' from the nested
// code (scales uint8 [blocks], sd per matrix [offset, s2 of each 256-block group],
// nb blocks and G groups per matrix)
template <bool kNested>
__global__ void __launch_bounds__(kThreads) nf4_dequant(const uint32_t *__restrict__ codes,
                                                        const void *__restrict__ scales, const float *__restrict__ sd,
                                                        uint32_t nb, uint32_t G, int64_t nunits,
                                                        uint4 *__restrict__ y) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = c_nf4_levels[threadIdx.x];
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kDqUnits;
  uint32_t c[kDqIter];
  float a[kDqIter];
#pragma unroll
  for (int it = 0; it < kDqIter; ++it) {
    const int64_t u0 = base + it * kThreads + threadIdx.x;
    const int64_t u = u0 < nunits ? u0 : nunits - 1;
    c[it] = codes[u];
    if constexpr (kNested) {
      const uint32_t bg = (uint32_t)(u >> 3), m = bg / nb;
      a[it] = nested_absmax(reinterpret_cast<const uint8_t *>(scales)[bg], sd + (int64_t)m * (1 + G), bg - m * nb);
    } else {
      a[it] = reinterpret_cast<const float *>(scales)[u >> 3];
    }
  }
#pragma unroll
  for (int it = 0; it < kDqIter; ++it) {
    const int64_t u = base + it * kThreads + threadIdx.x;
    if (u < nunits) {
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        o[p] = pack_bf16_rne(lv[(c[it] >> (8 * p)) & 0xFu] * a[it], lv[(c[it] >> (8 * p + 4)) & 0xFu] * a[it]);
      st_nt(&y[u], make_uint4(o[0], o[1], o[2], o[3]));
    }
  }
}

// Nested absmax, pass 1: one workgroup of 1024 threads per matrix of nb blocks, and
// offset = fl32(fl64(sum) / nb) to sd[m (1 + G)], where fl64(sum) is the exact sum of
// the matrix's FP32 absmax rounded once to the nearest double (ties to even), so the
// result depends on neither the order of the additions nor the number of threads.
// The exact sum is an integer in units of 2^-149 (the least FP32 subnormal): each
// value is its 24-bit significand shifted to its exponent, split over two 32-bit
// limbs, and every thread adds its strided share into its own 64-bit limb counters
// in LDS (no carries needed below 2^31 values).  The threads' counters are then
// added in a tree (integer sums: exact in any order), and thread 0 propagates the
// carries and rounds the top 53 bits.
constexpr int64_t kNestGroup = 256;
constexpr int kNestSumThreads = 1024;
// 320 bits of two's complement: FP32 magnitudes up to 2^128 from 2^-149, times up to
// 2^31 values, and the sign
constexpr int kSumLimbs = 10;

// the exact sum held in limb counters (limb j weighs 2^(32 j - 149)), rounded to the
// nearest double, ties to even
__device__ double limbs_to_f64(const int64_t (&acc)[kSumLimbs]) {
  uint32_t l[kSumLimbs];
  int64_t c = 0;
#pragma unroll
  for (int j = 0; j < kSumLimbs; ++j) {
    const int64_t v = acc[j] + c;
    l[j] = (uint32_t)((uint64_t)v & 0xffffffffu);
    c = v >> 32;  // arithmetic: the carry or borrow into the next limb
  }
  const bool neg = c < 0;
  if (neg) {  // magnitude of the two's complement value
    uint64_t cy = 1;
#pragma unroll
    for (int j = 0; j < kSumLimbs; ++j) {
      const uint64_t v = (uint64_t)(~l[j]) + cy;
      l[j] = (uint32_t)v;
      cy = v >> 32;
    }
  }
  int h = kSumLimbs - 1;
  while (h >= 0 && l[h] == 0) --h;
  if (h < 0) return 0.0;
  // bits [32 (h - 3), 32 (h + 1)) of the magnitude as a 128-bit window hi:lo
  uint64_t hi = ((uint64_t)l[h] << 32) | (h >= 1 ? l[h - 1] : 0u);
  uint64_t lo = ((uint64_t)(h >= 2 ? l[h - 2] : 0u) << 32) | (h >= 3 ? l[h - 3] : 0u);
  bool sticky = false;
  for (int j = 0; j < h - 3; ++j) sticky |= l[j] != 0;
  const int lz = __clzll(hi);  // < 32: limb h is not zero
  if (lz) {
    hi = (hi << lz) | (lo >> (64 - lz));
    lo <<= lz;
  }
  int top = 32 * h + 31 - lz;  // the leading bit, in units of 2^-149
  uint64_t mant = hi >> 11;    // 53 bits
  const bool half = (hi >> 10) & 1u;
  sticky |= (hi & 0x3ffu) != 0 || lo != 0;
  if (half && (sticky || (mant & 1u))) {
    ++mant;
    if (mant >> 53) {
      mant >>= 1;
      ++top;
    }
  }
  const double r = ldexp((double)mant, top - 52 - 149);
  return neg ? -r : r;
}

__global__ void __launch_bounds__(kNestSumThreads) nf4_nest_offset(const float *__restrict__ absmax, int64_t nb,
                                                                   int64_t G, float *__restrict__ sd) {
  __shared__ unsigned long long acc[kSumLimbs][kNestSumThreads];
  const int t = threadIdx.x;
  const int64_t m = blockIdx.x;
  const float *a = absmax + m * nb;
#pragma unroll
  for (int j = 0; j < kSumLimbs; ++j) acc[j][t] = 0ull;
  for (int64_t i = t; i < nb; i += kNestSumThreads) {
    const uint32_t u = __float_as_uint(a[i]);
    const uint32_t ex = (u >> 23) & 0xffu, fr = u & 0x7fffffu;
    const uint64_t sig = ex ? (fr | 0x800000u) : fr;
    if (!sig) continue;
    const int b = ex ? (int)ex - 1 : 0;  // the significand's lowest bit, in units of 2^-149
    const uint64_t sh = sig << (b & 31);
    const int li = b >> 5;               // at most 8 (finite values: b <= 253)
    uint64_t l0 = sh & 0xffffffffu, l1 = sh >> 32;
    if (u >> 31) {  // negative values (not written by the quantizer) subtract, modulo 2^64
      l0 = 0ull - l0;
      l1 = 0ull - l1;
    }
    atomicAdd(&acc[li][t], (unsigned long long)l0);  // this thread's own counters
    atomicAdd(&acc[li + 1][t], (unsigned long long)l1);
  }
  __syncthreads();
  for (int w = kNestSumThreads / 2; w > 0; w >>= 1) {
    if (t < w) {
#pragma unroll
      for (int j = 0; j < kSumLimbs; ++j) acc[j][t] += acc[j][t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    int64_t s[kSumLimbs];
#pragma unroll
    for (int j = 0; j < kSumLimbs; ++j) s[j] = (int64_t)acc[j][0];
    sd[m * (1 + G)] = (float)(limbs_to_f64(s) / (double)nb);
  }
}

// Pass 2: one wave per group of 256 blocks (all matrices' groups in one grid),
// four blocks per lane: d = fl(a - offset), t = max |d| over the group,
// s2 = fl(t / 448), code = e4m3(|fl(d / s2)|) with the sign bit for d < 0.
__global__ void __launch_bounds__(kThreads) nf4_nest_groups(const float *__restrict__ absmax, int64_t nb, int64_t G,
                                                            int64_t ngroups, uint8_t *__restrict__ qcodes,
                                                            float *__restrict__ sd) {
  const int64_t gg = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (gg >= ngroups) return;
  const int64_t m = gg / G, g = gg - m * G;
  const int lane = threadIdx.x & 63;
  const float *a = absmax + m * nb;
  float *sm = sd + m * (1 + G);
  const float off = sm[0];
  float d[4];
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t bl = g * kNestGroup + 64 * j + lane;
    d[j] = bl < nb ? a[bl] - off : 0.0f;
    t = fmaxf(t, fabsf(d[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) t = fmaxf(t, __shfl_xor(t, o, 64));
  const float s2 = t / 448.0f;
  if (lane == 0) sm[1 + g] = s2;
  uint8_t *qm = qcodes + m * nb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t bl = g * kNestGroup + 64 * j + lane;
    if (bl < nb) {
      uint32_t q = 0, unused;
      if (s2 > 0.0f) {
        const float yv = d[j] / s2;
        e4m3_pair(fabsf(yv), 0.0f, q, unused);
        q |= yv < 0.0f ? 0x80u : 0u;
      }
      qm[bl] = (uint8_t)q;
    }
  }
}

// workgroups for n elements in units of 8, kDqUnits units each
int dq_grid(int64_t n) { return (int)((n / 8 + kDqUnits - 1) / kDqUnits); }

int grid_for(int64_t work_items, int per_block = kThreads, int cap = 65536) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

bqm_status check_qtensor(const bqm_qtensor *q, const char *who, bool need_sdec) {
  BQM_REQUIRE(q, BQM_ERR_INVALID_ARG, "%s: qtensor is NULL", who);
  BQM_REQUIRE(q->fmt == BQM_FMT_NVFP4 || q->fmt == BQM_FMT_NF4, BQM_ERR_INVALID_ARG,
              "%s: unknown format %d", who, q->fmt);
  BQM_REQUIRE(q->n_mat >= 0 && q->rows >= 0 && q->cols >= 0, BQM_ERR_INVALID_ARG,
              "%s: negative size", who);
  BQM_REQUIRE(q->nested == 0 || (q->fmt == BQM_FMT_NF4 && q->nested == 1), BQM_ERR_INVALID_ARG,
              "%s: nested must be 0, or 1 for NF4", who);
  int64_t blk = q->fmt == BQM_FMT_NVFP4 ? 16 : 64;
  BQM_REQUIRE(q->cols % blk == 0, BQM_ERR_SHAPE, "%s: cols=%lld is not a multiple of %lld", who,
              (long long)q->cols, (long long)blk);
  int64_t n = q->n_mat * q->rows * q->cols;
  if (n == 0) return BQM_OK;
  BQM_REQUIRE(q->codes && q->scales, BQM_ERR_INVALID_ARG, "%s: codes/scales pointer is NULL", who);
  BQM_REQUIRE(aligned16(q->codes) && aligned16(q->scales), BQM_ERR_ALIGN,
              "%s: codes/scales not 16-byte aligned", who);
  if (q->fmt == BQM_FMT_NVFP4) {
    BQM_REQUIRE(q->scale_mode == BQM_SCALE_PER_TENSOR || q->scale_mode == BQM_SCALE_PER_ROW,
                BQM_ERR_INVALID_ARG, "%s: bad scale_mode %d", who, q->scale_mode);
    if (need_sdec) {
      BQM_REQUIRE(q->s_dec, BQM_ERR_INVALID_ARG, "%s: s_dec pointer is NULL", who);
      BQM_REQUIRE(aligned16(q->s_dec), BQM_ERR_ALIGN, "%s: s_dec not 16-byte aligned", who);
    }
  } else if (q->nested) {
    BQM_REQUIRE(q->s_dec, BQM_ERR_INVALID_ARG, "%s: nested NF4 needs s_dec", who);
    BQM_REQUIRE(aligned16(q->s_dec), BQM_ERR_ALIGN, "%s: s_dec not 16-byte aligned", who);
    BQM_REQUIRE(q->n_mat * q->rows * q->cols / 64 < ((int64_t)1 << 31), BQM_ERR_SHAPE,
                "%s: nested NF4 stack too large", who);
  }
  return BQM_OK;
}


}  // namespace
}  // namespace bqm

using namespace bqm;

extern "C" size_t bqm_quantize_nvfp4_workspace_size(int64_t n_mat, int64_t rows, int64_t cols,
                                                    int32_t scale_mode) {
  (void)rows;
  (void)cols;
  if (scale_mode == BQM_SCALE_PER_ROW || n_mat <= 0) return 0;
  return (size_t)n_mat * sizeof(uint32_t);
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the running amax of each matrix lives in a file-scope
// device array (one copy per GPU, kept until the process ends) instead of a caller
// workspace.  Host code never passes the array's name to a kernel (in host code it
// is only a stand-in for the symbol): the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress and kept.
static constexpr int64_t kScratchMats = 65536;  // matrices per call: 256 KiB per GPU
static __device__ __align__(256) uint32_t scratch[kScratchMats];

namespace bqm {
namespace {

// Checks of the quantizer arguments shared by both entry points (host only, nothing
// launched).  Returns the number of matrices whose running amax the call needs
// (0: per-row mode or caller scales).
bqm_status check_quantize_nvfp4(const uint16_t *x, int32_t four_over_six, const float *s_dec_in,
                                const bqm_qtensor *out, const char *who, int64_t &amax_slots) {
  amax_slots = 0;
  bqm_status st = check_qtensor(out, who, true);
  if (st != BQM_OK) return st;
  BQM_REQUIRE(out->fmt == BQM_FMT_NVFP4, BQM_ERR_INVALID_ARG, "%s: out->fmt must be BQM_FMT_NVFP4", who);
  const int64_t n_mat = out->n_mat, per_mat = out->rows * out->cols;
  if (n_mat * per_mat == 0) return BQM_OK;
  BQM_REQUIRE(x, BQM_ERR_INVALID_ARG, "%s: x is NULL", who);
  BQM_REQUIRE(aligned16(x), BQM_ERR_ALIGN, "%s: x not 16-byte aligned", who);
  BQM_REQUIRE(!s_dec_in || aligned16(s_dec_in), BQM_ERR_ALIGN, "%s: s_dec_in not 16-byte aligned", who);
  BQM_REQUIRE(four_over_six >= kFosOff && four_over_six <= kFosStrict, BQM_ERR_INVALID_ARG,
              "%s: four_over_six must be 0, 1 or 2", who);
  if (out->scale_mode == BQM_SCALE_PER_TENSOR) {
    const int64_t P = cdiv(per_mat / 8, kAmaxVec), G = cdiv(per_mat / 16, kQuantBlocks);
    BQM_REQUIRE(n_mat * std::max(P, G) < ((int64_t)1 << 31), BQM_ERR_SHAPE, "%s: tensor too large", who);
    if (!s_dec_in) amax_slots = n_mat;
  }
  return BQM_OK;
}

// The launches of a checked call.  amax: n_mat running-amax slots when amax_slots > 0.
bqm_status quantize_nvfp4_launch(const uint16_t *x, int32_t four_over_six, const float *s_dec_in, bqm_qtensor *out,
                                 uint32_t *amax, hipStream_t s) {
  const int64_t n_mat = out->n_mat, rows = out->rows, cols = out->cols;
  const int64_t per_mat = rows * cols;
  out->four_over_six = four_over_six;
  if (n_mat * per_mat == 0) return BQM_OK;
  const float denom = four_over_six ? 6.0f * 256.0f : 6.0f * 448.0f;
  const uint4 *xv = reinterpret_cast<const uint4 *>(x);
  uint2 *cv = reinterpret_cast<uint2 *>(out->codes);
  uint8_t *sv = reinterpret_cast<uint8_t *>(out->scales);
  if (out->scale_mode == BQM_SCALE_PER_ROW) {
    const int64_t rows_total = n_mat * rows;
    const int64_t bpr = cols / 16;
    int grid = (int)cdiv(rows_total, kThreads / 64);
    if (four_over_six == kFosStrict)
      nvfp4_quant_rows<kFosStrict><<<grid, kThreads, 0, s>>>(xv, rows_total, bpr, s_dec_in, denom, cv, sv,
                                                             out->s_dec);
    else if (four_over_six)
      nvfp4_quant_rows<kFosScaled><<<grid, kThreads, 0, s>>>(xv, rows_total, bpr, s_dec_in, denom, cv, sv,
                                                             out->s_dec);
    else
      nvfp4_quant_rows<kFosOff><<<grid, kThreads, 0, s>>>(xv, rows_total, bpr, s_dec_in, denom, cv, sv,
                                                          out->s_dec);
    return launch_status("nvfp4_quant_rows");
  }
  const int64_t blocks_per_mat = per_mat / 16;
  const int64_t P = cdiv(per_mat / 8, kAmaxVec), G = cdiv(blocks_per_mat, kQuantBlocks);
  bqm_status st = BQM_OK;
  if (!s_dec_in) {
    // a fill kernel, not a memset, so that the call can be captured in a graph
    clear_u32<<<(int)std::min<int64_t>(cdiv(n_mat, kThreads), 1024), kThreads, 0, s>>>(amax, n_mat);
    st = launch_status("clear_u32");
    if (st != BQM_OK) return st;
    nvfp4_amax<<<(int)(n_mat * P), kThreads, 0, s>>>(xv, per_mat / 8, P, amax);
    st = launch_status("nvfp4_amax");
    if (st != BQM_OK) return st;
  }
  if (four_over_six == kFosStrict)
    nvfp4_quant_tensor<kFosStrict><<<(int)(n_mat * G), kThreads, 0, s>>>(xv, blocks_per_mat, G, amax, s_dec_in, denom,
                                                                         cv, sv, out->s_dec);
  else if (four_over_six)
    nvfp4_quant_tensor<kFosScaled><<<(int)(n_mat * G), kThreads, 0, s>>>(xv, blocks_per_mat, G, amax, s_dec_in, denom,
                                                                         cv, sv, out->s_dec);
  else
    nvfp4_quant_tensor<kFosOff><<<(int)(n_mat * G), kThreads, 0, s>>>(xv, blocks_per_mat, G, amax, s_dec_in, denom,
                                                                      cv, sv, out->s_dec);
  return launch_status("nvfp4_quant_tensor");
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t *g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's `scratch` (the current device, which must be the
// stream's device).
bqm_status scratch_for(hipStream_t s, const char *who, uint32_t **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BQM_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (s) {
    int sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return fail(BQM_ERR_HIP, "%s: hipStreamGetDevice: %s", who, hipGetErrorString(e));
    BQM_REQUIRE(sdev == dev, BQM_ERR_INVALID_ARG, "%s: the stream belongs to device %d, device %d is current", who,
                sdev, dev);
  }
  BQM_REQUIRE(dev >= 0 && dev < kMaxDevices, BQM_ERR_UNSUPPORTED, "%s: device index %d (at most %d devices)", who,
              dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(BQM_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = reinterpret_cast<uint32_t *>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return BQM_OK;
}

}  // namespace
}  // namespace bqm

extern "C" bqm_status bqm_quantize_nvfp4(const uint16_t *x, int32_t four_over_six,
                                         const float *s_dec_in, bqm_qtensor *out, void *ws,
                                         size_t ws_bytes, void *stream) {
  const char *who = "bqm_quantize_nvfp4";
  int64_t slots = 0;
  bqm_status st = check_quantize_nvfp4(x, four_over_six, s_dec_in, out, who, slots);
  if (st != BQM_OK) return st;
  uint32_t *amax = nullptr;
  if (slots > 0) {
    const size_t need = bqm_quantize_nvfp4_workspace_size(out->n_mat, out->rows, out->cols, 0);
    BQM_REQUIRE(ws && ws_bytes >= need, BQM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                ws_bytes);
    BQM_REQUIRE(aligned16(ws), BQM_ERR_ALIGN, "%s: ws not 16-byte aligned", who);
    amax = reinterpret_cast<uint32_t *>(ws);
  }
  return quantize_nvfp4_launch(x, four_over_six, s_dec_in, out, amax, as_stream(stream));
}

extern "C" bqm_status bqm_quantize_nvfp4_noalloc(const uint16_t *x, int32_t four_over_six, const float *s_dec_in,
                                                 bqm_qtensor *out, void *stream) {
  const char *who = "bqm_quantize_nvfp4_noalloc";
  int64_t slots = 0;
  bqm_status st = check_quantize_nvfp4(x, four_over_six, s_dec_in, out, who, slots);
  if (st != BQM_OK) return st;
  BQM_REQUIRE(slots <= kScratchMats, BQM_ERR_WORKSPACE,
              "%s: %lld matrices need a running amax each; the static scratch holds %lld (pass s_dec_in, or use "
              "bqm_quantize_nvfp4 with a workspace)",
              who, (long long)slots, (long long)kScratchMats);
  hipStream_t s = as_stream(stream);
  uint32_t *amax = nullptr;
  if (slots > 0) {
    st = scratch_for(s, who, &amax);
    if (st != BQM_OK) return st;
  }
  return quantize_nvfp4_launch(x, four_over_six, s_dec_in, out, amax, s);
}

extern "C" bqm_status bqm_quantize_nf4(const uint16_t *x, bqm_qtensor *out, void *stream) {
  bqm_status st = check_qtensor(out, "bqm_quantize_nf4", false);
  if (st != BQM_OK) return st;
  BQM_REQUIRE(out->fmt == BQM_FMT_NF4 && !out->nested, BQM_ERR_INVALID_ARG,
              "bqm_quantize_nf4: out must be plain NF4 (FP32 absmax; bqm_nf4_nest makes the nested form)");
  const int64_t n = out->n_mat * out->rows * out->cols;
  if (n == 0) return BQM_OK;
  BQM_REQUIRE(x, BQM_ERR_INVALID_ARG, "bqm_quantize_nf4: x is NULL");
  BQM_REQUIRE(aligned16(x), BQM_ERR_ALIGN, "bqm_quantize_nf4: x not 16-byte aligned");
  BQM_REQUIRE(n / 8 / kDqUnits < INT32_MAX, BQM_ERR_SHAPE, "bqm_quantize_nf4: tensor too large");
  nf4_quant<<<dq_grid(n), kThreads, 0, as_stream(stream)>>>(
      reinterpret_cast<const uint4 *>(x), n / 8, reinterpret_cast<uint32_t *>(out->codes),
      reinterpret_cast<float *>(out->scales));
  return launch_status("nf4_quant");
}

extern "C" bqm_status bqm_dequantize(const bqm_qtensor *q, uint16_t *y, void *stream) {
  bqm_status st = check_qtensor(q, "bqm_dequantize", true);
  if (st != BQM_OK) return st;
  const int64_t n = q->n_mat * q->rows * q->cols;
  if (n == 0) return BQM_OK;
  BQM_REQUIRE(y, BQM_ERR_INVALID_ARG, "bqm_dequantize: y is NULL");
  BQM_REQUIRE(aligned16(y), BQM_ERR_ALIGN, "bqm_dequantize: y not 16-byte aligned");
  BQM_REQUIRE(n / 8 / kDqUnits < INT32_MAX, BQM_ERR_SHAPE, "bqm_dequantize: tensor too large");
  hipStream_t s = as_stream(stream);
  if (q->fmt == BQM_FMT_NVFP4) {
    const int64_t seg_units = q->scale_mode == BQM_SCALE_PER_ROW ? q->cols / 8 : q->rows * q->cols / 8;
    BQM_REQUIRE(seg_units < (int64_t)1 << 31, BQM_ERR_SHAPE, "bqm_dequantize: matrix too large");
    nvfp4_dequant<true><<<dq_grid(n), kThreads, 0, s>>>(
        reinterpret_cast<const uint32_t *>(q->codes), reinterpret_cast<const uint8_t *>(q->scales), q->s_dec,
        n / 8, seg_units, reinterpret_cast<uint4 *>(y));
    return launch_status("nvfp4_dequant");
  }
  const int64_t nb = q->rows * q->cols / 64;
  if (q->nested)
    nf4_dequant<true><<<dq_grid(n), kThreads, 0, s>>>(reinterpret_cast<const uint32_t *>(q->codes), q->scales,
                                                      q->s_dec, (uint32_t)nb, (uint32_t)cdiv(nb, kNestGroup), n / 8,
                                                      reinterpret_cast<uint4 *>(y));
  else
    nf4_dequant<false><<<dq_grid(n), kThreads, 0, s>>>(reinterpret_cast<const uint32_t *>(q->codes), q->scales,
                                                       nullptr, 0, 0, n / 8, reinterpret_cast<uint4 *>(y));
  return launch_status("nf4_dequant");
}

extern "C" bqm_status bqm_nf4_nest(const bqm_qtensor *plain, bqm_qtensor *nested, void *stream) {
  bqm_status st = check_qtensor(plain, "bqm_nf4_nest", false);
  if (st != BQM_OK) return st;
  st = check_qtensor(nested, "bqm_nf4_nest", false);
  if (st != BQM_OK) return st;
  BQM_REQUIRE(plain->fmt == BQM_FMT_NF4 && !plain->nested, BQM_ERR_INVALID_ARG,
              "bqm_nf4_nest: plain must be NF4 with FP32 absmax");
  BQM_REQUIRE(nested->fmt == BQM_FMT_NF4 && nested->nested == 1, BQM_ERR_INVALID_ARG,
              "bqm_nf4_nest: nested must be NF4 with nested = 1");
  BQM_REQUIRE(plain->n_mat == nested->n_mat && plain->rows == nested->rows && plain->cols == nested->cols,
              BQM_ERR_SHAPE, "bqm_nf4_nest: shapes differ");
  const int64_t n = plain->n_mat * plain->rows * plain->cols;
  if (n == 0) return BQM_OK;
  BQM_REQUIRE(plain->n_mat < ((int64_t)1 << 31), BQM_ERR_SHAPE, "bqm_nf4_nest: too many matrices");
  hipStream_t s = as_stream(stream);
  if (nested->codes != plain->codes &&
      hipMemcpyAsync(nested->codes, plain->codes, (size_t)(n / 2), hipMemcpyDeviceToDevice, s) != hipSuccess)
    return launch_status("bqm_nf4_nest: copy of the codes");
  const int64_t nb = plain->rows * plain->cols / 64, G = cdiv(nb, kNestGroup);
  const float *am = reinterpret_cast<const float *>(plain->scales);
  nf4_nest_offset<<<(unsigned)plain->n_mat, kNestSumThreads, 0, s>>>(am, nb, G, nested->s_dec);
  st = launch_status("nf4_nest_offset");
  if (st != BQM_OK) return st;
  const int64_t ngroups = plain->n_mat * G;
  nf4_nest_groups<<<(unsigned)cdiv(ngroups, kThreads / 64), kThreads, 0, s>>>(
      am, nb, G, ngroups, reinterpret_cast<uint8_t *>(nested->scales), nested->s_dec);
  return launch_status("nf4_nest_groups");
}

namespace bqm {
// Per-token NVFP4 with Four-Over-Six of n_rows rows (cols % 16 == 0, 16-byte aligned
// pointers): codes, scales and per-row s_dec, and in the same pass the bf16 rows of
// val * sb (no s_dec), exact.
bqm_status nvfp4_quantize_rows_expand(const uint16_t *x, int64_t n_rows, int64_t cols, uint8_t *codes,
                                      uint8_t *scales, float *s_dec, uint16_t *expanded, hipStream_t s) {
  if (n_rows * cols == 0) return BQM_OK;
  const int grid = (int)cdiv(n_rows, kThreads / 64);
  nvfp4_quant_rows<kFosScaled, true><<<grid, kThreads, 0, s>>>(
      reinterpret_cast<const uint4 *>(x), n_rows, cols / 16, nullptr, 6.0f * 256.0f, reinterpret_cast<uint2 *>(codes),
      scales, s_dec, reinterpret_cast<uint4 *>(expanded));
  return launch_status("nvfp4_quant_rows (expanded)");
}
}  // namespace bqm
