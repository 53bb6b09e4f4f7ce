// Shared device helpers for the gfx950 kernels of libminih3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace minih3 {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (gfx950 converts with v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Storage-type traits: load / store one element as fp32.
template <typename T> struct Act;
template <> struct Act<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};

// Sum over the 64 lanes, result in every lane: within each 16-lane row by
// DPP moves (quad xor 1, quad xor 2, half-row mirror, row mirror), then two
// lane exchanges across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Sum over the N lanes of a row (N = 16 or 32, aligned groups), result in
// every lane of the row: DPP within 16 lanes, then one lane exchange across
// the two 16-lane halves.
template <int N>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(N == 16 || N == 32, "row width");
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  if (N == 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// Per-head RMSNorm and rotary turn of one lane's CPL channels of a head row
// of CPL * LPR = 128 channels spread over LPR aligned lanes: v is scaled by
// 1 / sqrt(mean(v^2) + eps) and the weights g, then channel pair p (2p,
// 2p + 1) is turned by the angle whose cosine and sine are cs[p], sn[p]
// (1 and 0 for a pair that is not rotated). The fused multiply-adds are
// explicit so that every kernel that calls this rounds alike. The
// reciprocal square root is the hardware instruction on an argument held at
// or above the smallest normal float (it is at least eps), which gives the
// library rsqrtf's bits without its range scaling.
template <int CPL, int LPR>
__device__ __forceinline__ void qk_norm_rotate(float* v, const float* g, const float* cs, const float* sn,
                                               float eps) {
  static_assert(CPL * LPR == 128, "head width");
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) sq = __builtin_fmaf(v[e], v[e], sq);
  const float r = __builtin_amdgcn_rsqf(fmaxf(row_sum<LPR>(sq) * (1.f / 128) + eps, 0x1p-126f));
#pragma unroll
  for (int p = 0; p < CPL / 2; ++p) {
    const float a = v[2 * p] * r * g[2 * p], b = v[2 * p + 1] * r * g[2 * p + 1];
    v[2 * p] = __builtin_fmaf(a, cs[p], -(b * sn[p]));
    v[2 * p + 1] = __builtin_fmaf(a, sn[p], b * cs[p]);
  }
}

// AdaLN table row of a packed row: tag * num_tvals + tidx, or -1 for a
// padding row. Out-of-range values are clamped so that the table is never
// read out of bounds (the layout is validated separately on request).
__device__ __forceinline__ int table_row_of(int tag, int tidx, int num_tags, int num_tvals) {
  if (tag < 0 || tag >= num_tags) return -1;
  tidx = tidx < 0 ? 0 : (tidx >= num_tvals ? num_tvals - 1 : tidx);
  return tag * num_tvals + tidx;
}

}  // namespace minih3
