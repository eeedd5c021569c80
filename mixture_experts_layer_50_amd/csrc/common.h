// Internal helpers shared by the HIP sources of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16 with the gfx950 conversion instruction (v_cvt_pk_bf16_f32:
// round to nearest, ties to even; a NaN stays a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two values packed as bf16 (a in the low half).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Element type traits for the two layer dtypes.
template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elt<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f2bf(v); }
};

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------- host side
// Thread-local error text and status helpers (abi.hip).
void set_error(const char* fmt, ...);
moe_status_t check_launch(const char* what);

// Kernel timer hooks (abi.hip).  prof_begin returns a token passed to prof_end.
int prof_begin(const char* name, hipStream_t s);
void prof_end(int token, hipStream_t s);

struct ProfScope {
  int tok;
  hipStream_t s;
  ProfScope(const char* name, hipStream_t st) : tok(prof_begin(name, st)), s(st) {}
  ~ProfScope() { prof_end(tok, s); }
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace moe
