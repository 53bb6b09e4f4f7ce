// Rotation and int8 quantization of one row held in registers by a
// workgroup of 256 threads (rotated W8A8). Page "HyperFlow H3 Flash Brings
// MiniMax H3 Video to One GPU", How it got smaller and faster: rotated W8A8
// INT8 quantization of the linear layers. The rotation is the normalised
// Hadamard transform of every 128-wide block of the row; quantization is
// symmetric per row: code = rint(v * (127 / amax)) in [-127, 127], scale =
// amax / 127; an all-zero row gives codes 0 and scale 0.
//
// Layout: thread t holds the 8 consecutive values 8 (t % 16) .. + 7 of block
// 16 p + t / 16 in v[p] (zeros where the block is past the row's nb blocks).
// The codes are integers decided by floating point, so the order is fixed:
// butterfly stages h = 1, 2, 4 (in the lane), 8, 16, 32, 64 (lanes 1, 2, 4, 8
// apart), each (v_i, v_{i+h}) -> (v_i + v_{i+h}, v_i - v_{i+h}) in fp32,
// then one multiplication by fp32(1 / sqrt(128)); 127 / amax and amax / 127
// are correctly rounded fp32 divisions. red: 4 floats of shared memory used
// by nothing else while this runs.
#pragma once
#include "common.h"

namespace minih3 {

template <int MAXP>
__device__ __forceinline__ void rotate_quantize_row(float (&v)[MAXP][8], int nb, int8_t* qr, float* scale_out,
                                                    float* red) {
  const int t = threadIdx.x, sub = t & 15, grp = t >> 4;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (16 * p + grp < nb) {  // uniform over a 16-lane group
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
  float amax = 0.f;
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
  if (t == 0) *scale_out = zero ? 0.f : amax / 127.f;
}

}  // namespace minih3
