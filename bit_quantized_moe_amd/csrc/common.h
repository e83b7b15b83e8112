// Private helpers shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bqm.h"

namespace bqm {

// Sets the thread-local message returned by bqm_last_error and returns `s`.
bqm_status fail(bqm_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
bqm_status ok();
// Turns the last launch error (if any) into BQM_ERR_HIP.
bqm_status launch_status(const char *what);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// device-side number-format helpers (bit-exact; compiled with -ffp-contract=off)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bqm_bf16x2 __attribute__((ext_vector_type(2)));
typedef float bqm_f32x2 __attribute__((ext_vector_type(2)));

// two floats -> bf16 pair (a in the low half), round to nearest even (one
// v_cvt_pk_bf16_f32; the same bits as f32_to_bf16 for finite inputs)
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const bqm_f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bqm_bf16x2));
}

// E4M3FN code (0..126) -> float
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return c < 8u ? (float)c * 0x1p-9f : __uint_as_float((c + 960u) << 20);
}

// E2M1 magnitude code (0..7) -> float32 bits of its value
__device__ __forceinline__ uint32_t e2m1_mag_bits(uint32_t m) {
  return m >= 2u ? (m + 252u) << 22 : (m == 1u ? 0x3F000000u : 0u);
}

}  // namespace bqm

#define BQM_REQUIRE(cond, status, ...)                \
  do {                                                \
    if (!(cond)) return ::bqm::fail((status), __VA_ARGS__); \
  } while (0)
