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
// One workgroup handles 64 rows of HG heads (2 when the head count is even,
// else 1). In the q/k pass a lane owns 16 bytes of a row (8 bf16 channels),
// so a row's RMS is a reduction over 16 lanes done with DPP moves and the
// rotation pairs stay inside the lane; a row's sines and cosines are taken
// once for the HG heads.
// On request (bf16) the pass also records, per head and document, the
// largest |k| of the stored keys, which the attention kernel bounds its
// scores with. HBM-bound.
#include "common.h"
#include "kernels.h"

namespace minih3 {

struct RopeFreqs {
  float inv_freq[64];
};

// 16 bytes of one row: CPL channels as fp32; stored() is the value a channel
// has once written back in T.
template <typename T> struct Chunk;
template <> struct Chunk<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
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
  static __device__ __forceinline__ float stored(float x) {
    return __uint_as_float(pack_bf16x2(x, 0.f) << 16);
  }
};
template <> struct Chunk<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const floatx4 r = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r[i];
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<floatx4*>(p) = floatx4{v[0], v[1], v[2], v[3]};
  }
  static __device__ __forceinline__ float stored(float x) { return x; }
};

template <typename T, int HG>
__global__ void __launch_bounds__(256) k_qk_norm_rope(const T* __restrict__ qkv, const float* __restrict__ gq,
                                                      const float* __restrict__ gk, const int32_t* __restrict__ pos,
                                                      T* __restrict__ qo, T* __restrict__ ko, T* __restrict__ vto,
                                                      const uint64_t* __restrict__ masks, float* __restrict__ kmax,
                                                      int S, int H, int stride, int fd, float eps, RopeFreqs fr) {
  constexpr int HD = 128;
  constexpr int VN = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int CPR = HD / VN;              // chunks per row of one head
  constexpr int PITCH = 64 + VN;            // LDS row pitch (elements) of the transposed tile
  __shared__ T vs[HD * PITCH];
  __shared__ float red[4][HG][2];

  const int s0 = blockIdx.x * 64, h0 = blockIdx.y * HG, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int W = H * HD;

  // ---- q and k: RMSNorm + RoPE. Lane l owns the CPL channels of chunk
  // l % LPR of row l / LPR of the wave's group of RPW rows, so one 16-byte
  // load per tensor, sums over the LPR lanes of a row, and rotation pairs
  // inside the lane; a row's sines and cosines serve the HG heads.
  constexpr int CPL = 16 / sizeof(T), LPR = HD / CPL, RPW = 64 / LPR, PPL = CPL / 2;
  const int sub = lane / LPR, cl = lane % LPR;
  float gqv[CPL], gkv[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    gqv[e] = gq[cl * CPL + e];
    gkv[e] = gk[cl * CPL + e];
  }
  int ax[PPL];
  float invf[PPL];
  bool rot[PPL];
#pragma unroll
  for (int p = 0; p < PPL; ++p) {
    const int j = cl * PPL + p;  // rotation pair (channels 2j, 2j+1)
    ax[p] = fd > 0 ? j / fd : 3;
    rot[p] = j < 3 * fd;
    invf[p] = rot[p] ? fr.inv_freq[j - ax[p] * fd] : 0.f;
  }
  // key norms (bf16 path): largest |k| per head and document over this tile's
  // rows, taken from the stored values; padding rows are document 1
  const bool norms = kmax && s0 < S;  // the tile masks cover rows below S only
  const uint64_t mpad = norms ? masks[2 * blockIdx.x + 1] : 0ull;
  float mx[HG][2];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) mx[hh][0] = mx[hh][1] = 0.f;
  for (int r0 = wid * RPW; r0 < 64; r0 += 4 * RPW) {
    const int r = r0 + sub, s = s0 + r;
    const bool live = s < S;
    float sn[PPL], cs[PPL];
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      sn[p] = 0.f;
      cs[p] = 1.f;
      if (live && rot[p]) sincosf((float)pos[3L * s + ax[p]] * invf[p], &sn[p], &cs[p]);
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const int h = h0 + hh;
      const long head_base = ((long)b * H + h) * stride;  // row offset of (b, h) in [B, H, stride, hd]
      float q[CPL], k[CPL];
      if (live) {
        const T* src = qkv + ((long)b * S + s) * (3L * W) + h * HD + cl * CPL;
        Chunk<T>::load(src, q);
        Chunk<T>::load(src + W, k);
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) q[e] = k[e] = 0.f;
      }
      qk_norm_rotate<CPL, LPR>(q, gqv, cs, sn, eps);
      qk_norm_rotate<CPL, LPR>(k, gkv, cs, sn, eps);
      if (!live) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) q[e] = k[e] = 0.f;
      }
      if (norms) {
        float n2 = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const float a = Chunk<T>::stored(k[e]);
          n2 = __builtin_fmaf(a, a, n2);
        }
        n2 = row_sum<LPR>(n2);
        const int d = (int)((mpad >> r) & 1ull);
        if (live) mx[hh][d] = fmaxf(mx[hh][d], n2);
      }
      if (s < stride) {
        Chunk<T>::store(qo + (head_base + s) * HD + cl * CPL, q);
        Chunk<T>::store(ko + (head_base + s) * HD + cl * CPL, k);
      }
    }
  }
  if (norms) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) mx[hh][d] = fmaxf(mx[hh][d], __shfl_xor(mx[hh][d], o, 64));
    if (lane == 0)
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        red[wid][hh][0] = mx[hh][0];
        red[wid][hh][1] = mx[hh][1];
      }
    __syncthreads();
    if (threadIdx.x < 2 * HG) {
      const int hh = threadIdx.x >> 1, d = threadIdx.x & 1;
      const float m = sqrtf(fmaxf(fmaxf(red[0][hh][d], red[1][hh][d]), fmaxf(red[2][hh][d], red[3][hh][d])));
      // non-negative floats order as ints
      atomicMax(reinterpret_cast<int*>(kmax + 2 * ((long)b * H + h0 + hh) + d), __float_as_int(m));
    }
  }

  // ---- v: [64 rows][128] -> [128][64 rows] through LDS, head by head
  const int n_cols = stride - s0 < 64 ? stride - s0 : 64;
  for (int hh = 0; hh < HG; ++hh) {
    const int h = h0 + hh;
    if (hh > 0) __syncthreads();  // the previous head's columns are out of LDS
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
    for (int c = threadIdx.x; c < HD * (64 / VN); c += 256) {
      const int d = c / (64 / VN), r0 = (c % (64 / VN)) * VN;
      if (r0 < n_cols) {
        T* dst = vto + (((long)b * H + h) * HD + d) * stride + s0 + r0;
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&vs[d * PITCH + r0]);
      }
    }
  }
}

template <typename T, int HG>
static void launch_heads(dim3 grid, const T* qkv, const float* gq, const float* gk, const int32_t* pos, T* qo, T* ko,
                         T* vto, const uint64_t* masks, float* kmax, int S, int H, int stride, int fd, float eps,
                         const RopeFreqs& fr, hipStream_t st) {
  grid.y = (unsigned)(H / HG);
  k_qk_norm_rope<T, HG><<<grid, 256, 0, st>>>(qkv, gq, gk, pos, qo, ko, vto, masks, kmax, S, H, stride, fd, eps, fr);
}

template <typename T>
hipError_t launch_qk_norm_rope(const T* qkv, const float* gq, const float* gk, const int32_t* pos, T* qo, T* ko,
                               T* vto, int B, int S, int H, int stride, int fd, float theta, float eps,
                               hipStream_t st, const uint64_t* masks, float* kmax) {
  if (fd < 0 || 6 * fd > 128 || stride % 64 != 0 || stride < S) return hipErrorInvalidValue;
  if (kmax && (!masks || sizeof(T) != 2)) return hipErrorInvalidValue;
  RopeFreqs fr;
  for (int j = 0; j < 64; ++j) fr.inv_freq[j] = j < fd ? (float)pow((double)theta, -(double)j / fd) : 0.f;
  const dim3 grid((unsigned)(stride / 64), 1u, (unsigned)B);
  if (H % 2 == 0)
    launch_heads<T, 2>(grid, qkv, gq, gk, pos, qo, ko, vto, masks, kmax, S, H, stride, fd, eps, fr, st);
  else
    launch_heads<T, 1>(grid, qkv, gq, gk, pos, qo, ko, vto, masks, kmax, S, H, stride, fd, eps, fr, st);
  return hipGetLastError();
}

// table[s * np + j] = (cos, sin) of pos[s][j / fd] * inv_freq[j mod fd], the
// turn of rotation pair j (< np = 3 fd) of row s, computed as above: the
// projection epilogue that normalizes and rotates q and k in place of
// k_qk_norm_rope reads it.
__global__ void __launch_bounds__(256) k_rope_table(const int32_t* __restrict__ pos, float2* __restrict__ table,
                                                    int S, int fd, RopeFreqs fr) {
  const int np = 3 * fd;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)S * np) return;
  const int s = (int)(i / np), j = (int)(i - (long)s * np), ax = j / fd;
  float sn, cs;
  sincosf((float)pos[3L * s + ax] * fr.inv_freq[j - ax * fd], &sn, &cs);
  table[i] = make_float2(cs, sn);
}

// Rows [S, stride) of q and k and columns [S, stride) of v^T set to zero,
// one workgroup per (batch item, head).
__global__ void __launch_bounds__(256) k_qk_tail_zero(bf16_t* __restrict__ qo, bf16_t* __restrict__ ko,
                                                      bf16_t* __restrict__ vto, int S, int stride) {
  const long bh = blockIdx.x;
  const int n = (stride - S) * 128;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int s = S + i / 128, c = i % 128;
    qo[(bh * stride + s) * 128 + c] = bf16_t(0);
    ko[(bh * stride + s) * 128 + c] = bf16_t(0);
    vto[(bh * 128 + c) * stride + s] = bf16_t(0);
  }
}

hipError_t launch_rope_table(const int32_t* pos, float* table, int S, int fd, float theta, hipStream_t st) {
  if (fd <= 0 || 6 * fd > 128 || S <= 0) return hipErrorInvalidValue;
  RopeFreqs fr;
  for (int j = 0; j < 64; ++j) fr.inv_freq[j] = j < fd ? (float)pow((double)theta, -(double)j / fd) : 0.f;
  const long n = (long)S * 3 * fd;
  k_rope_table<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(pos, reinterpret_cast<float2*>(table), S, fd, fr);
  return hipGetLastError();
}

hipError_t launch_qk_tail_zero(bf16_t* qo, bf16_t* ko, bf16_t* vto, int BH, int S, int stride, hipStream_t st) {
  if (stride < S) return hipErrorInvalidValue;
  if (stride == S) return hipSuccess;
  k_qk_tail_zero<<<dim3((unsigned)BH), 256, 0, st>>>(qo, ko, vto, S, stride);
  return hipGetLastError();
}

template hipError_t launch_qk_norm_rope<bf16_t>(const bf16_t*, const float*, const float*, const int32_t*, bf16_t*,
                                                bf16_t*, bf16_t*, int, int, int, int, int, float, float,
                                                hipStream_t, const uint64_t*, float*);
template hipError_t launch_qk_norm_rope<float>(const float*, const float*, const float*, const int32_t*, float*,
                                               float*, float*, int, int, int, int, int, float, float, hipStream_t,
                                               const uint64_t*, float*);

}  // namespace minih3
