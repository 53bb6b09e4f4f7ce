// Per-row AdaLN modulation: y = LN(x) * (1 + scale) + shift, with the
// modulation vectors selected by the row's modality tag and timestep index.
// Page "MiniMaxH3Transformer3DModel": the per-row tag selects the AdaLN
// modulation parameters (class description); norm_eps is the eps of the
// pre-attention and pre-feed-forward norms (Parameters). The LayerNorm
// carries no affine part of its own; padding rows get zero shift/scale.
//
// HBM-bound: one workgroup per row, the row held in registers between the
// mean, variance and output passes, 16-byte coalesced loads and stores,
// fp32 statistics. The input may be the fp32 residual stream of a bf16
// block (the library keeps the residual in fp32 between the two gated
// residual adds and between blocks).
#include "common.h"
#include "kernels.h"
#include "rotq.h"

namespace minih3 {

template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = r;
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* v) {
    floatx4 r = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r[i];
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i];
    *reinterpret_cast<floatx4*>(p) = r;
  }
};

// VN input values of type TI (VN = the output vector width)
template <typename TI, int VN>
__device__ __forceinline__ void load_in(const TI* p, float* v) {
  if constexpr (sizeof(TI) == 4) {
#pragma unroll
    for (int i = 0; i < VN; i += 4) Vec<float>::load(reinterpret_cast<const float*>(p) + i, v + i);
  } else {
    static_assert(VN == Vec<bf16_t>::N, "bf16 input feeds a bf16 output");
    Vec<bf16_t>::load(reinterpret_cast<const bf16_t*>(p), v);
  }
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();  // red[] reuse across calls
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) s += red[w];
  return s;
}

template <typename TI, typename T, int NT, int MAXV>
__global__ void __launch_bounds__(NT) k_adaln(const TI* x, T* y,  // x and y may alias: a row is read whole first
                                              const float* __restrict__ table, const int32_t* __restrict__ tags,
                                              const int32_t* __restrict__ tidx, int S, int D, int which, float eps,
                                              int num_tags, int num_tvals) {
  constexpr int VN = Vec<T>::N;
  __shared__ float red[NT / 64];
  const long row = blockIdx.x;
  const int s = (int)(row % S);
  const int nv = D / VN;
  const TI* xr = x + row * D;
  T* yr = y + row * D;

  float v[MAXV][VN];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    int c = threadIdx.x + i * NT;
    if (c < nv) {
      load_in<TI, VN>(xr + c * VN, v[i]);
#pragma unroll
      for (int e = 0; e < VN; ++e) sum += v[i][e];
    }
  }
  const float mean = block_sum<NT>(sum, red) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    int c = threadIdx.x + i * NT;
    if (c < nv) {
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        float d = v[i][e] - mean;
        sq += d * d;
      }
    }
  }
  const float var = block_sum<NT>(sq, red) / (float)D;
  const float rstd = rsqrtf(var + eps);

  const int tr = table_row_of(tags[s], tidx[s], num_tags, num_tvals);
  const float* shift = tr >= 0 ? table + ((long)tr * 6 + 3 * which + 0) * D : nullptr;
  const float* scale = tr >= 0 ? table + ((long)tr * 6 + 3 * which + 1) * D : nullptr;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    int c = threadIdx.x + i * NT;
    if (c < nv) {
      float o[VN];
      if (tr >= 0) {
#pragma unroll
        for (int e = 0; e < VN; e += 4) {
          floatx4 sh = *reinterpret_cast<const floatx4*>(shift + c * VN + e);
          floatx4 sc = *reinterpret_cast<const floatx4*>(scale + c * VN + e);
#pragma unroll
          for (int u = 0; u < 4; ++u) o[e + u] = (v[i][e + u] - mean) * rstd * (1.f + sc[u]) + sh[u];
        }
      } else {
#pragma unroll
        for (int e = 0; e < VN; ++e) o[e] = (v[i][e] - mean) * rstd;
      }
      Vec<T>::store(yr + c * VN, o);
    }
  }
}

// AdaLN whose output row goes straight to rotated W8A8 codes: the modulated
// row is rounded to bf16 (the value the bf16 kernel stores), then rotated and
// quantized by rotate_quantize_row. Chunk c = t + 256 i of 8 values is block
// 16 i + t / 16, lane t % 16 of that function's layout, so the registers
// pass over as they are; codes and scale equal those of k_adaln (bf16)
// followed by k_rot_quant bit for bit.
template <typename TI, int MAXV>
__global__ void __launch_bounds__(256) k_adaln_rq(const TI* x, int8_t* __restrict__ q, float* __restrict__ qscale,
                                                  const float* __restrict__ table, const int32_t* __restrict__ tags,
                                                  const int32_t* __restrict__ tidx, int S, int D, int which,
                                                  float eps, int num_tags, int num_tvals) {
  constexpr int NT = 256, VN = 8;
  __shared__ float red[NT / 64];
  __shared__ float red_q[4];
  const long row = blockIdx.x;
  const int s = (int)(row % S);
  const int nv = D / VN;
  const TI* xr = x + row * D;
  float v[MAXV][VN];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    int c = threadIdx.x + i * NT;
#pragma unroll
    for (int e = 0; e < VN; ++e) v[i][e] = 0.f;
    if (c < nv) {
      load_in<TI, VN>(xr + c * VN, v[i]);
#pragma unroll
      for (int e = 0; e < VN; ++e) sum += v[i][e];
    }
  }
  const float mean = block_sum<NT>(sum, red) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    int c = threadIdx.x + i * NT;
    if (c < nv) {
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        float d = v[i][e] - mean;
        sq += d * d;
      }
    }
  }
  const float var = block_sum<NT>(sq, red) / (float)D;
  const float rstd = rsqrtf(var + eps);
  const int tr = table_row_of(tags[s], tidx[s], num_tags, num_tvals);
  const float* shift = tr >= 0 ? table + ((long)tr * 6 + 3 * which + 0) * D : nullptr;
  const float* scale = tr >= 0 ? table + ((long)tr * 6 + 3 * which + 1) * D : nullptr;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    int c = threadIdx.x + i * NT;
    if (c < nv) {
      float o[VN];
      if (tr >= 0) {
#pragma unroll
        for (int e = 0; e < VN; e += 4) {
          floatx4 sh = *reinterpret_cast<const floatx4*>(shift + c * VN + e);
          floatx4 sc = *reinterpret_cast<const floatx4*>(scale + c * VN + e);
#pragma unroll
          for (int u = 0; u < 4; ++u) o[e + u] = (v[i][e + u] - mean) * rstd * (1.f + sc[u]) + sh[u];
        }
      } else {
#pragma unroll
        for (int e = 0; e < VN; ++e) o[e] = (v[i][e] - mean) * rstd;
      }
#pragma unroll
      for (int e = 0; e < VN; e += 2) {  // the stored bf16 values
        const uint32_t pk = pack_bf16x2(o[e], o[e + 1]);
        v[i][e] = __uint_as_float(pk << 16);
        v[i][e + 1] = __uint_as_float(pk & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) v[i][e] = 0.f;
    }
  }
  rotate_quantize_row<MAXV>(v, D / 128, q + row * D, qscale + row, red_q);
}

template <typename TI>
hipError_t launch_adaln_rq_t(const TI* x, int8_t* q, float* qscale, const float* table, const int32_t* tags,
                             const int32_t* tidx, int B, int S, int D, int which, float eps, int num_tags,
                             int num_tvals, hipStream_t st) {
  if (D % 128 != 0 || D > 8 * 1024) return hipErrorInvalidValue;
  const int nv = D / 8;
  dim3 grid((unsigned)((long)B * S));
  if (nv <= 256)
    k_adaln_rq<TI, 1><<<grid, 256, 0, st>>>(x, q, qscale, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  else if (nv <= 512)
    k_adaln_rq<TI, 2><<<grid, 256, 0, st>>>(x, q, qscale, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  else if (nv <= 768)
    k_adaln_rq<TI, 3><<<grid, 256, 0, st>>>(x, q, qscale, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  else
    k_adaln_rq<TI, 4><<<grid, 256, 0, st>>>(x, q, qscale, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  return hipGetLastError();
}

hipError_t launch_adaln_rq(const void* x, bool x_f32, int8_t* q, float* qscale, const float* table,
                           const int32_t* tags, const int32_t* tidx, int B, int S, int D, int which, float eps,
                           int num_tags, int num_tvals, hipStream_t st) {
  if (x_f32)
    return launch_adaln_rq_t<float>(static_cast<const float*>(x), q, qscale, table, tags, tidx, B, S, D, which, eps,
                                    num_tags, num_tvals, st);
  return launch_adaln_rq_t<bf16_t>(static_cast<const bf16_t*>(x), q, qscale, table, tags, tidx, B, S, D, which, eps,
                                   num_tags, num_tvals, st);
}

template <typename TI, typename T>
hipError_t launch_adaln_t(const TI* x, T* y, const float* table, const int32_t* tags, const int32_t* tidx, int B,
                          int S, int D, int which, float eps, int num_tags, int num_tvals, hipStream_t st) {
  constexpr int NT = 256;
  const int nv = D / Vec<T>::N;
  dim3 grid((unsigned)((long)B * S));
  if (nv <= NT * 1)
    k_adaln<TI, T, NT, 1><<<grid, NT, 0, st>>>(x, y, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  else if (nv <= NT * 2)
    k_adaln<TI, T, NT, 2><<<grid, NT, 0, st>>>(x, y, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  else if (nv <= NT * 3)
    k_adaln<TI, T, NT, 3><<<grid, NT, 0, st>>>(x, y, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  else if (nv <= NT * 4)
    k_adaln<TI, T, NT, 4><<<grid, NT, 0, st>>>(x, y, table, tags, tidx, S, D, which, eps, num_tags, num_tvals);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
hipError_t launch_adaln(const void* x, bool x_f32, T* y, const float* table, const int32_t* tags,
                        const int32_t* tidx, int B, int S, int D, int which, float eps, int num_tags, int num_tvals,
                        hipStream_t st) {
  if (x_f32)
    return launch_adaln_t<float, T>(static_cast<const float*>(x), y, table, tags, tidx, B, S, D, which, eps,
                                    num_tags, num_tvals, st);
  return launch_adaln_t<T, T>(static_cast<const T*>(x), y, table, tags, tidx, B, S, D, which, eps, num_tags,
                              num_tvals, st);
}

template hipError_t launch_adaln<bf16_t>(const void*, bool, bf16_t*, const float*, const int32_t*, const int32_t*,
                                         int, int, int, int, float, int, int, hipStream_t);
template hipError_t launch_adaln<float>(const void*, bool, float*, const float*, const int32_t*, const int32_t*, int,
                                        int, int, int, float, int, int, hipStream_t);

// fp32 -> act copy (taps of the fp32 residual stream)
template <typename T>
__global__ void __launch_bounds__(256) k_cast_f32(const float* __restrict__ x, T* __restrict__ y, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) Act<T>::st(y + i, x[i]);
}

template <typename T>
hipError_t launch_cast_f32(const float* x, T* y, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_cast_f32<T><<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(x, y, n);
  return hipGetLastError();
}
template hipError_t launch_cast_f32<bf16_t>(const float*, bf16_t*, long, hipStream_t);
template hipError_t launch_cast_f32<float>(const float*, float*, long, hipStream_t);

}  // namespace minih3
