// Per-head query/key RMSNorm followed by the 3-D rotary embedding, and the
// transpose of the values into the key-contiguous layout the attention
// kernel reads.
//
// Page "MiniMaxH3Transformer3DModel", Parameters: qk_norm_eps is the eps of
// the per-head query/key norms; rope_freq_dim rotary frequencies per axis,
// the t, h and w axes share one inv_freq buffer of that length, and
// 2 * 3 * rope_freq_dim of the head channels are rotated; rope_theta is the
// base of the frequency schedule. Reading of what the page leaves open: the
// norm weight has head_dim entries shared by all heads; axis a owns channels
// [2fd*a, 2fd*(a+1)) and its pair j is channels (2j, 2j+1), turned by
// pos[a] * theta^(-j/fd); the remaining channels pass through.
//
// One workgroup handles 64 rows of one head. In the q/k pass lane l of a
// wave owns channel pair l of a row, so the RMS is one wave reduction and
// the rotation is lane-local. HBM-bound.
#include "common.h"
#include "kernels.h"

namespace minih3 {

struct RopeFreqs {
  float inv_freq[64];
};

template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float& a, float& b) {
    uint32_t r = *reinterpret_cast<const uint32_t*>(p);
    a = __uint_as_float(r << 16);
    b = __uint_as_float(r & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(bf16_t* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
  }
};
template <> struct Pair<float> {
  static __device__ __forceinline__ void load(const float* p, float& a, float& b) {
    float2 r = *reinterpret_cast<const float2*>(p);
    a = r.x;
    b = r.y;
  }
  static __device__ __forceinline__ void store(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
};

template <typename T>
__global__ void __launch_bounds__(256) k_qk_norm_rope(const T* __restrict__ qkv, const float* __restrict__ gq,
                                                      const float* __restrict__ gk, const int32_t* __restrict__ pos,
                                                      T* __restrict__ qo, T* __restrict__ ko, T* __restrict__ vto,
                                                      int S, int H, int stride, int fd, float eps, RopeFreqs fr) {
  constexpr int HD = 128;
  constexpr int VN = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int CPR = HD / VN;              // chunks per row of one head
  constexpr int PITCH = 64 + VN;            // LDS row pitch (elements) of the transposed tile
  __shared__ T vs[HD * PITCH];

  const int s0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int W = H * HD;
  const long head_base = ((long)b * H + h) * stride;  // row offset of (b, h) in [B, H, stride, hd]

  // ---- q and k: RMSNorm + RoPE, lane owns channels (2*lane, 2*lane+1)
  const float gq0 = gq[2 * lane], gq1 = gq[2 * lane + 1];
  const float gk0 = gk[2 * lane], gk1 = gk[2 * lane + 1];
  const int axis = fd > 0 ? lane / fd : 3;
  const bool rot = lane < 3 * fd;
  const float invf = rot ? fr.inv_freq[lane - axis * fd] : 0.f;
  for (int r = wid; r < 64; r += 4) {
    const int s = s0 + r;
    float q0 = 0.f, q1 = 0.f, k0 = 0.f, k1 = 0.f;
    if (s < S) {
      const T* src = qkv + ((long)b * S + s) * (3L * W) + h * HD + 2 * lane;
      Pair<T>::load(src, q0, q1);
      Pair<T>::load(src + W, k0, k1);
      const float rq = rsqrtf(wave_sum(q0 * q0 + q1 * q1) * (1.f / HD) + eps);
      const float rk = rsqrtf(wave_sum(k0 * k0 + k1 * k1) * (1.f / HD) + eps);
      q0 *= rq * gq0;
      q1 *= rq * gq1;
      k0 *= rk * gk0;
      k1 *= rk * gk1;
      if (rot) {
        const float ang = (float)pos[3L * s + axis] * invf;
        float sn, cs;
        sincosf(ang, &sn, &cs);
        float a = q0 * cs - q1 * sn, c = q0 * sn + q1 * cs;
        q0 = a;
        q1 = c;
        a = k0 * cs - k1 * sn;
        c = k0 * sn + k1 * cs;
        k0 = a;
        k1 = c;
      }
    }
    if (s < stride) {
      Pair<T>::store(qo + (head_base + s) * HD + 2 * lane, q0, q1);
      Pair<T>::store(ko + (head_base + s) * HD + 2 * lane, k0, k1);
    }
  }

  // ---- v: [64 rows][128] -> [128][64 rows] through LDS
  for (int c = threadIdx.x; c < 64 * CPR; c += 256) {
    const int r = c / CPR, d0 = (c % CPR) * VN;
    const int s = s0 + r;
    T tmp[VN];
    if (s < S) {
      const T* src = qkv + ((long)b * S + s) * (3L * W) + 2 * W + h * HD + d0;
      *reinterpret_cast<u32x4*>(tmp) = *reinterpret_cast<const u32x4*>(src);
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) tmp[e] = T(0);
    }
#pragma unroll
    for (int e = 0; e < VN; ++e) vs[(d0 + e) * PITCH + r] = tmp[e];
  }
  __syncthreads();
  const int n_cols = stride - s0 < 64 ? stride - s0 : 64;
  for (int c = threadIdx.x; c < HD * (64 / VN); c += 256) {
    const int d = c / (64 / VN), r0 = (c % (64 / VN)) * VN;
    if (r0 < n_cols) {
      T* dst = vto + (((long)b * H + h) * HD + d) * stride + s0 + r0;
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&vs[d * PITCH + r0]);
    }
  }
}

template <typename T>
hipError_t launch_qk_norm_rope(const T* qkv, const float* gq, const float* gk, const int32_t* pos, T* qo, T* ko,
                               T* vto, int B, int S, int H, int stride, int fd, float theta, float eps,
                               hipStream_t st) {
  if (fd < 0 || 6 * fd > 128 || stride % 64 != 0 || stride < S) return hipErrorInvalidValue;
  RopeFreqs fr;
  for (int j = 0; j < 64; ++j) fr.inv_freq[j] = j < fd ? (float)pow((double)theta, -(double)j / fd) : 0.f;
  dim3 grid((unsigned)(stride / 64), (unsigned)H, (unsigned)B);
  k_qk_norm_rope<T><<<grid, 256, 0, st>>>(qkv, gq, gk, pos, qo, ko, vto, S, H, stride, fd, eps, fr);
  return hipGetLastError();
}

template hipError_t launch_qk_norm_rope<bf16_t>(const bf16_t*, const float*, const float*, const int32_t*, bf16_t*,
                                                bf16_t*, bf16_t*, int, int, int, int, int, float, float,
                                                hipStream_t);
template hipError_t launch_qk_norm_rope<float>(const float*, const float*, const float*, const int32_t*, float*,
                                               float*, float*, int, int, int, int, int, float, float, hipStream_t);

}  // namespace minih3
