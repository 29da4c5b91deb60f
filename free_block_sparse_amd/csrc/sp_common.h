// Shared device/host helpers of libsparsepr (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparsepr.h"

namespace sp {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr uint64_t kGolden64 = 0x9E3779B97F4A7C15ull;

// ---------------------------------------------------------------- conversions
__host__ __device__ inline float bf16_to_f32(bf16_t h) {
  union { uint32_t u; float f; } c;
  c.u = static_cast<uint32_t>(h) << 16;
  return c.f;
}

// round-to-nearest-even; NaN stays NaN
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  if ((c.u & 0x7f800000u) == 0x7f800000u && (c.u & 0x007fffffu)) return 0x7fc0;
  uint32_t lsb = (c.u >> 16) & 1u;
  c.u += 0x7fffu + lsb;
  return static_cast<bf16_t>(c.u >> 16);
}

// Two fp32 values rounded to nearest-even bf16 and packed (the first in the
// low half): one v_cvt_pk_bf16_f32 on gfx950, the same rounding as f32_to_bf16.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<double> {
  __device__ static inline double load(const double* p) { return *p; }
  __device__ static inline void store(double* p, double v) { *p = v; }
};
template <> struct Elem<float> {
  __device__ static inline float load(const float* p) { return *p; }
  __device__ static inline void store(float* p, float v) { *p = v; }
};
template <> struct Elem<_Float16> {
  __device__ static inline float load(const _Float16* p) { return (float)*p; }
  __device__ static inline void store(_Float16* p, float v) { *p = (_Float16)v; }
};
template <> struct Elem<bf16_t> {
  __device__ static inline float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static inline void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// A [B, H, N, d] tensor seen per (b*H + h) slice.
struct View4 {
  const void* p;
  long long sb, sh, sn;
  int H;
  __device__ inline long long row_off(int bh, long long n) const {
    int b = bh / H, h = bh - (bh / H) * H;
    return (long long)b * sb + (long long)h * sh + n * sn;
  }
};

struct MutView4 {
  void* p;
  long long sb, sh, sn;
  int H;
  __device__ inline long long row_off(int bh, long long n) const {
    int b = bh / H, h = bh - (bh / H) * H;
    return (long long)b * sb + (long long)h * sh + n * sn;
  }
};

__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Workgroup i of a one-dimensional grid of W workgroups, seen as block blk of
// slice `slice` (nb blocks per slice, W = nb * slices).  The hardware hands
// consecutive workgroups of a grid to the eight XCDs in turn, so the slices
// are laid out as eight contiguous runs, one per XCD: every block of a slice
// then runs on one XCD and the slice's shared operands stay in that XCD's L2.
// A bijection for any W and nb; only the placement depends on the dispatch
// order.
constexpr int kXcds = 8;
__device__ inline void xcd_slice(int i, int W, int nb, int& slice, int& blk) {
  const int x = i % kXcds, k = i / kXcds;
  const int q = W / kXcds, r = W % kXcds;
  const int t = x * q + (x < r ? x : r) + k;
  slice = t / nb;
  blk = t - slice * nb;
}

// Orderable unsigned image of a double: a < b  <=>  ord(a) < ord(b) (NaN excluded).
__host__ __device__ inline uint64_t ord_f64(double x) {
  union { double d; uint64_t u; } c;
  c.d = x;
  return (c.u & 0x8000000000000000ull) ? ~c.u : (c.u | 0x8000000000000000ull);
}

}  // namespace sp
