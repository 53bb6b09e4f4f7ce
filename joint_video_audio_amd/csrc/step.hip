// Pieces of a denoising step around the blocks: the unmerged LoRA linear
// layer and the flow-matching Euler update.
// Page "HyperFlow for MiniMax-H3", header table (a PEFT LoRA of rank 256 and
// alpha 256 on the attention and feed-forward layers; a fixed sigma grid with
// video shift 12 and audio shift 3); page "MiniMaxH3Transformer3DModel",
// `forward` (a scale applied to the LoRA layers; the model returns
// velocities).
//
// Unmerged LoRA, y = x W^T + s (x A^T) B^T with s = scale * alpha / rank, is
// one contraction over the concatenated inner dimension:
// y = [x | s t] [W | B]^T with t = x A^T. The projection kernel runs it as
// is (K + rank columns): [W | B] is packed once per layer by k_concat_rows,
// and the kernel reads its A operand from x and s t in place (no per-call
// copy). The low-rank part adds about 2 rank / K of the layer's work.
#include "common.h"
#include "kernels.h"

namespace minih3 {

namespace {

// out[m] = [x[m, 0:K] | s * t[m, 0:R]] (rows of K + R values); one 16-byte
// piece per thread. s == 1 copies t bit for bit.
template <typename T>
__global__ void __launch_bounds__(256) k_concat_rows(const T* __restrict__ x, const T* __restrict__ t, float s,
                                                     T* __restrict__ out, long M, int K, int R) {
  constexpr int V = 16 / sizeof(T);
  const int pk = K / V, pr = R / V, pw = pk + pr;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * pw) return;
  const long m = i / pw;
  const int p = (int)(i - m * pw);
  u32x4 v;
  if (p < pk) {
    v = *reinterpret_cast<const u32x4*>(x + m * K + (long)p * V);
  } else {
    v = *reinterpret_cast<const u32x4*>(t + m * R + (long)(p - pk) * V);
    if (s != 1.f) {
      float f[V];
#pragma unroll
      for (int j = 0; j < V; ++j) f[j] = Act<T>::ld(reinterpret_cast<const T*>(&v) + j) * s;
#pragma unroll
      for (int j = 0; j < V; ++j) Act<T>::st(reinterpret_cast<T*>(&v) + j, f[j]);
    }
  }
  *reinterpret_cast<u32x4*>(out + m * (K + R) + (long)p * V) = v;
}

// x_next[b, i] = x[b, i] + (sigma_next[v] - sigma_now[v]) * vel[b, i] with
// v = tidx[idx[i]] (the row's timestep value), C values per row; one thread
// per value.
__global__ void __launch_bounds__(256) k_euler(const float* x, const float* __restrict__ vel, float* x_next, long n,
                                               int C, int nrows, const int32_t* __restrict__ idx,
                                               const int32_t* __restrict__ tidx, int S,
                                               const float* __restrict__ sig_now,
                                               const float* __restrict__ sig_next, int ntv) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int i = (int)((e / C) % nrows);
  int r = idx[i];
  r = r < 0 ? 0 : (r >= S ? S - 1 : r);
  int v = tidx[r];
  v = v < 0 ? 0 : (v >= ntv ? ntv - 1 : v);
  const float d = sig_next[v] - sig_now[v];
  x_next[e] = x[e] + d * vel[e];
}

}  // namespace

template <typename T>
hipError_t launch_concat_rows(const T* x, const T* t, float s, T* out, long M, int K, int R, hipStream_t st) {
  constexpr int V = 16 / sizeof(T);
  if (M <= 0) return hipSuccess;
  if (K % V != 0 || R % V != 0) return hipErrorInvalidValue;
  const long n = M * (K / V + R / V);
  k_concat_rows<T><<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(x, t, s, out, M, K, R);
  return hipGetLastError();
}

hipError_t launch_euler(const float* x, const float* vel, float* x_next, int B, int nrows, int C,
                        const int32_t* idx, const int32_t* tidx, int S, const float* sig_now, const float* sig_next,
                        int ntv, hipStream_t st) {
  const long n = (long)B * nrows * C;
  if (n <= 0) return hipSuccess;
  k_euler<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(x, vel, x_next, n, C, nrows, idx, tidx, S, sig_now,
                                                             sig_next, ntv);
  return hipGetLastError();
}

template hipError_t launch_concat_rows<bf16_t>(const bf16_t*, const bf16_t*, float, bf16_t*, long, int, int,
                                               hipStream_t);
template hipError_t launch_concat_rows<float>(const float*, const float*, float, float*, long, int, int, hipStream_t);

}  // namespace minih3
