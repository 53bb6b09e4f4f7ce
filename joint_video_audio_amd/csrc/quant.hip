// Rotated W8A8 INT8: rotation and quantization of rows.
// Page "HyperFlow H3 Flash Brings MiniMax H3 Video to One GPU", How it got
// smaller and faster: rotated W8A8 INT8 quantization of the linear layers.
// The rotation is the normalised Hadamard transform of every 128-wide block
// of a row (the same for activations and weight rows, so products are
// unchanged); quantization is symmetric int8 per row: code = rint(v * (127 /
// amax)), scale = amax / 127, an all-zero row gives codes 0 and scale 0.
//
// The codes are integers decided by floating point, so the arithmetic order
// is fixed: the butterflies run in stages h = 1, 2, 4, ..., 64, each mapping
// (v_i, v_{i+h}) (bit h of i clear) to (v_i + v_{i+h}, v_i - v_{i+h}) in
// fp32, then one multiplication by fp32(1 / sqrt(128)); the reciprocal
// 127 / amax and the scale amax / 127 are correctly rounded fp32 divisions.
//
// One workgroup of 256 threads per row (HBM-bound: read the row once, write
// one byte per element): thread t holds 8 consecutive values of block
// 16 p + (t / 16) in pass p, the first three stages are in-lane and the
// other four exchange values between lanes 1, 2, 4 and 8 apart inside a
// 16-lane group; the row's absolute maximum is a workgroup reduction.
#include "common.h"
#include "kernels.h"

namespace minih3 {

namespace {

template <typename T>
__device__ __forceinline__ void load8v(const T* p, float* v);
template <>
__device__ __forceinline__ void load8v<bf16_t>(const bf16_t* p, float* v) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8v<float>(const float* p, float* v) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

template <typename T, int MAXP>
__global__ void __launch_bounds__(256) k_rot_quant(const T* __restrict__ x, int K, int8_t* __restrict__ q,
                                                   float* __restrict__ scale) {
  __shared__ float red[4];
  const int t = threadIdx.x, sub = t & 15, grp = t >> 4;
  const long row = blockIdx.x;
  const int nb = K / 128;
  const T* xr = x + row * K;
  float v[MAXP][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int b = 16 * p + grp;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[p][j] = 0.f;
    if (b < nb) {  // uniform over a 16-lane group
      load8v<T>(xr + 128 * b + 8 * sub, v[p]);
#pragma unroll
      for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j & h)) {
            const float a = v[p][j], c = v[p][j + h];
            v[p][j] = a + c;
            v[p][j + h] = a - c;
          }
    }
  }
  // Lane-crossing stages h = 8, 16, 32, 64: the partner lane is d = h / 8
  // away; the lane whose bit d is clear holds v_i and keeps v_i + partner,
  // the other holds v_{i+h} and keeps partner - v_{i+h}. Every lane of the
  // wave joins the exchange (lanes of a missing block exchange among
  // themselves and are never stored).
#pragma unroll
  for (int d = 1; d < 16; d *= 2) {
    const bool hi = sub & d;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float o = __shfl_xor(v[p][j], d, 64);
        v[p][j] = hi ? o - v[p][j] : v[p][j] + o;
      }
  }
  const float kNorm = __uint_as_float(0x3db504f3u);  // fp32(1 / sqrt(128))
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (16 * p + grp < nb) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[p][j] = v[p][j] * kNorm;
        amax = fmaxf(amax, fabsf(v[p][j]));
      }
    }
  }
  amax = fmaxf(amax, dpp_mov<0xB1>(amax));
  amax = fmaxf(amax, dpp_mov<0x4E>(amax));
  amax = fmaxf(amax, dpp_mov<0x141>(amax));
  amax = fmaxf(amax, dpp_mov<0x140>(amax));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool zero = !(amax > 0.f);
  const float inv = zero ? 0.f : 127.f / amax;
  int8_t* qr = q + row * K;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int b = 16 * p + grp;
    if (b < nb) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float c = rintf(v[p][j] * inv);
        c = fminf(fmaxf(c, -127.f), 127.f);
        w[j >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (j & 3));
      }
      *reinterpret_cast<u32x2*>(qr + 128 * b + 8 * sub) = u32x2{w[0], w[1]};
    }
  }
  if (t == 0) scale[row] = zero ? 0.f : amax / 127.f;
}

template <typename T, int MAXP>
static void rq_launch(const T* x, int M, int K, int8_t* q, float* s, hipStream_t st) {
  k_rot_quant<T, MAXP><<<dim3((unsigned)M), 256, 0, st>>>(x, K, q, s);
}

}  // namespace

template <typename T>
hipError_t launch_rot_quant(const T* x, int M, int K, int8_t* q, float* scale, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (K % 128 != 0 || K > 16384) return hipErrorInvalidValue;
  const int passes = (K / 128 + 15) / 16;
  switch (passes) {
    case 1: rq_launch<T, 1>(x, M, K, q, scale, st); break;
    case 2: rq_launch<T, 2>(x, M, K, q, scale, st); break;
    case 3: rq_launch<T, 3>(x, M, K, q, scale, st); break;
    case 4: rq_launch<T, 4>(x, M, K, q, scale, st); break;
    case 5: rq_launch<T, 5>(x, M, K, q, scale, st); break;
    case 6: rq_launch<T, 6>(x, M, K, q, scale, st); break;
    case 7: rq_launch<T, 7>(x, M, K, q, scale, st); break;
    case 8: rq_launch<T, 8>(x, M, K, q, scale, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_rot_quant<bf16_t>(const bf16_t*, int, int, int8_t*, float*, hipStream_t);
template hipError_t launch_rot_quant<float>(const float*, int, int, int8_t*, float*, hipStream_t);

}  // namespace minih3
