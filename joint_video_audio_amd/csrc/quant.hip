// Rotated W8A8 INT8: rotation and quantization of rows stored in memory.
// Page "HyperFlow H3 Flash Brings MiniMax H3 Video to One GPU", How it got
// smaller and faster: rotated W8A8 INT8 quantization of the linear layers.
// The arithmetic (normalised Hadamard transform of every 128-wide block,
// symmetric per-row int8) is rotate_quantize_row (rotq.h), shared with the
// AdaLN kernel that quantizes its own output rows.
//
// One workgroup of 256 threads per row (HBM-bound: read the row once, write
// one byte per element): thread t loads 8 consecutive values of block
// 16 p + (t / 16) in pass p.
#include "common.h"
#include "kernels.h"
#include "rotq.h"

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
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int b = 16 * p + grp;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[p][j] = 0.f;
    if (b < nb) load8v<T>(xr + 128 * b + 8 * sub, v[p]);  // uniform over a 16-lane group
  }
  rotate_quantize_row<MAXP>(v, nb, q + row * K, scale + row, red);
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
