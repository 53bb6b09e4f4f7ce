// The model's edges around the block stack: the input projections that build
// the packed sequence and the output heads that read it back.
// Page "MiniMaxH3Transformer3DModel": Parameters in_channels and patch_size
// (video rows arrive patchified, in_channels * prod(patch_size) wide),
// audio_in_channels, final_norm_eps (norm_out); the mixed-precision note
// (the two input patch projections and the two output heads are float32);
// `forward`: video / audio rows in the order of video_indices /
// audio_indices, and the velocities returned in those orders.
//
// All four projections are fp32 contractions on v_mfma_f32_16x16x4_f32
// (fp32 storage of weights and latents; the hidden states are the
// activation type):
//  * k_edge_in: packed row idx[r] = W h_r + b. A workgroup computes 64 rows x
//    256 features (four waves of 64 x 64), stages the tile in LDS and stores
//    each row's 256 features as one contiguous run at its packed position.
//  * k_edge_rows: text rows copied to their packed positions; padding rows
//    zeroed.
//  * k_edge_fold: norm_out folded into the head: W' = W diag(gamma),
//    s = W' 1, c = W beta + b, so head(LN(x)) = (W' x - mu s) / sigma + c.
//  * k_edge_out: both heads on gathered rows in one launch. A wave owns 16
//    rows and all output channels of its head over the full hidden width;
//    the four waves of a workgroup share 64-column chunks of W' in a
//    double-buffered LDS ring, with the next chunk's weights and activations
//    in flight while one is used.
//    Row sums of x - x_0 (x_0 the row's first value) and of its square ride
//    along, so the LayerNorm statistics come from the same pass.
#include "common.h"
#include "kernels.h"

namespace minih3 {

namespace {

// Eight consecutive activations as fp32.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

__device__ __forceinline__ int clamp_row(int r, int S) { return r < 0 ? 0 : (r >= S ? S - 1 : r); }

// x[b, idx[r]] = W h[b, r] + bias for r < nrows; h [B, nrows, C] fp32,
// W [D, C] fp32 (C % 16 == 0), x [B, S, D]. Grid (D / 256, ceil(nrows / 64), B).
template <typename T>
__global__ void __launch_bounds__(256) k_edge_in(const float* __restrict__ h, int nrows, int C,
                                                 const float* __restrict__ W, const float* __restrict__ bias,
                                                 const int32_t* __restrict__ idx, int S, int D, T* __restrict__ x) {
  constexpr int kCols = 256, kPad = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T tile[64][kCols + kPad];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int f0 = blockIdx.x * kCols, m0 = blockIdx.y * 64;
  const float* hb = h + (long)blockIdx.z * nrows * C;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Lane (r16, q) holds W[f + r16][k + 4q + t] and h[m + r16][k + 4q + t];
  // MFMA t contracts k slot q of both, so four MFMAs cover 16 columns.
  for (int k = 0; k < C; k += 16) {
    floatx4 wv[4], hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wv[i] = *reinterpret_cast<const floatx4*>(W + (long)(f0 + 64 * wid + 16 * i + r16) * C + k + 4 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 16 * j + r16;
      hv[j] = m < nrows ? *reinterpret_cast<const floatx4*>(hb + (long)m * C + k + 4 * q) : floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[i][t], hv[j][t], acc[i][j], 0, 0, 0);
  }

  // Lane (r16, q) holds features 64 wid + 16 i + 4q .. +3 of tile row 16 j + r16.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = 64 * wid + 16 * i + 4 * q;
    const floatx4 bv = *reinterpret_cast<const floatx4*>(bias + f0 + f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4 v = acc[i][j] + bv;
      T* dst = &tile[16 * j + r16][f];
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
        *reinterpret_cast<floatx4*>(dst) = v;
      }
    }
  }
  __syncthreads();
  // Each row's 256 features go out as one contiguous run of 16-byte pieces.
  constexpr int kPieces = kCols * (int)sizeof(T) / 16;
  T* xb = x + (long)blockIdx.z * S * D;
  for (int e = threadIdx.x; e < 64 * kPieces; e += 256) {
    const int rr = e / kPieces, pc = e % kPieces;
    const int m = m0 + rr;
    if (m >= nrows) continue;
    const int row = clamp_row(idx[m], S);
    *reinterpret_cast<u32x4*>(xb + (long)row * D + f0 + pc * (16 / sizeof(T))) =
        *reinterpret_cast<const u32x4*>(&tile[rr][pc * (16 / sizeof(T))]);
  }
}

// Text rows to their packed positions (grid (n_text, B)) and padding rows
// zeroed (grid (S, B), rows with tag -1 only); one workgroup a row.
template <typename T>
__global__ void __launch_bounds__(256) k_edge_rows(const T* __restrict__ text, const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ tags, int ntext, int S, int D,
                                                   T* __restrict__ x, int zero_pads) {
  const int r = blockIdx.x;
  T* xb = x + (long)blockIdx.y * S * D;
  const int pieces = D * (int)sizeof(T) / 16;
  if (zero_pads) {
    if (tags[r] != -1) return;
    for (int p = threadIdx.x; p < pieces; p += 256)
      *reinterpret_cast<u32x4*>(xb + (long)r * D + p * (16 / sizeof(T))) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int row = clamp_row(idx[r], S);
  const T* src = text + ((long)blockIdx.y * ntext + r) * D;
  for (int p = threadIdx.x; p < pieces; p += 256)
    *reinterpret_cast<u32x4*>(xb + (long)row * D + p * (16 / sizeof(T))) =
        *reinterpret_cast<const u32x4*>(src + p * (16 / sizeof(T)));
}

// Head c (one workgroup each): W'[c] = W[c] * gamma, s[c] = sum W'[c],
// cv[c] = W[c] . beta + b[c].
__global__ void __launch_bounds__(256) k_edge_fold(const float* __restrict__ W, const float* __restrict__ b,
                                                   const float* __restrict__ gamma, const float* __restrict__ beta,
                                                   int D, float* __restrict__ Wf, float* __restrict__ s,
                                                   float* __restrict__ cv) {
  __shared__ float red[2][4];
  const int c = blockIdx.x;
  float s1 = 0.f, s2 = 0.f;
  for (int n = threadIdx.x; n < D; n += 256) {
    const float w = W[(long)c * D + n];
    const float wf = w * gamma[n];
    Wf[(long)c * D + n] = wf;
    s1 += wf;
    s2 += w * beta[n];
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wid] = s1;
    red[1][wid] = s2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    s[c] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    cv[c] = red[1][0] + red[1][1] + red[1][2] + red[1][3] + (b ? b[c] : 0.f);
  }
}

// y[b, r, :] = (W' x_r - mu_r s) / sigma_r + cv with x_r = x[b, idx[r]],
// mu_r, sigma_r its LayerNorm mean and deviation (eps inside), for r < nrows,
// for two heads in one launch: workgroups [0, blocks0) serve head 0, the
// rest head 1, so the small audio head runs beside the video one. NB = the
// larger head's C / 16; a head with fewer output blocks skips the others.
// D % 64 == 0. Grid (blocks0 + blocks1, B), blocks_h = ceil(nrows_h / 64).
template <typename T, int NB>
__global__ void __launch_bounds__(256) k_edge_out(const T* __restrict__ x, EdgeHeads hd, int blocks0, int S, int D,
                                                  float eps) {
  constexpr int Cmax = 16 * NB, KC = 64, kLd = KC + 4;  // 64-column chunks of W', rows padded by 16 bytes
  constexpr int kLoads = (Cmax * KC / 4 + 255) / 256;  // float4 loads per thread per chunk (at most)
  __shared__ __attribute__((aligned(16))) float wl[2][Cmax][kLd];
  const int h = blockIdx.x < blocks0 ? 0 : 1;
  const int blk = h ? blockIdx.x - blocks0 : blockIdx.x;
  const int32_t* __restrict__ idx = hd.idx[h];
  const int nrows = hd.nrows[h], C = hd.C[h], nbh = C / 16;
  const float* __restrict__ Wf = hd.Wf[h];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int m = blk * 64 + 16 * wid + r16;  // the lane's row
  const bool live = m < nrows;
  const int row = clamp_row(idx[live ? m : nrows - 1], S);
  const T* xr = x + ((long)blockIdx.y * S + row) * D;
  float x0;
  {
    float t[8];
    load8<T>(xr, t);
    x0 = t[0];
  }

  floatx4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float s1 = 0.f, s2 = 0.f;
  floatx4 stage[kLoads];
  const int nld = C * KC / 4;  // float4 pieces of a chunk of this head
  auto fetch = [&](int kc) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int e = threadIdx.x + 256 * l;
      if (e < nld) {
        const int c = e / (KC / 4), k4 = e % (KC / 4);
        stage[l] = *reinterpret_cast<const floatx4*>(Wf + (long)c * D + kc * KC + 4 * k4);
      }
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const int e = threadIdx.x + 256 * l;
      if (e < nld) {
        const int c = e / (KC / 4), k4 = e % (KC / 4);
        *reinterpret_cast<floatx4*>(&wl[buf][c][4 * k4]) = stage[l];
      }
    }
  };
  // The lane's 16 activations of a chunk: columns 32 st + 8q .. +7, st = 0, 1.
  float xa[2][8];
  auto fetch_x = [&](int kc) {
#pragma unroll
    for (int st = 0; st < 2; ++st) load8<T>(xr + kc * KC + 32 * st + 8 * q, xa[st]);
  };
  const int nk = D / KC;
  fetch(0);
  fetch_x(0);
  put(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    float xv[2][8];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int t = 0; t < 8; ++t) xv[st][t] = xa[st][t];
    if (kc + 1 < nk) {  // next chunk's weights and activations in flight during this one
      fetch(kc + 1);
      fetch_x(kc + 1);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // Lane (r16, q) holds x_r[32 st + 8q + t] - x_0 and W'[16 i + r16][same
      // column]; MFMA t contracts k slot q of both (eight MFMAs a block).
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        xv[st][t] = live ? xv[st][t] - x0 : 0.f;
        s1 += xv[st][t];
        s2 += xv[st][t] * xv[st][t];
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i >= nbh) break;  // uniform: the head's output blocks
        const float* wrow = &wl[buf][16 * i + r16][32 * st + 8 * q];
        const floatx4 wa = *reinterpret_cast<const floatx4*>(wrow);
        const floatx4 wb = *reinterpret_cast<const floatx4*>(wrow + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[t], xv[st][t], acc[i], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[t], xv[st][4 + t], acc[i], 0, 0, 0);
      }
    }
    if (kc + 1 < nk) put(buf ^ 1);
    __syncthreads();
  }

  // The four lanes of a row (q = 0..3) hold disjoint columns of it.
  s1 += __shfl_xor(s1, 16, 64);
  s1 += __shfl_xor(s1, 32, 64);
  s2 += __shfl_xor(s2, 16, 64);
  s2 += __shfl_xor(s2, 32, 64);
  const float mu = s1 / (float)D;  // mean of x - x_0
  const float var = fmaxf(s2 / (float)D - mu * mu, 0.f);
  const float rs = rsqrtf(var + eps);
  if (!live) return;
  // Lane (r16, q) holds output channels 16 i + 4q .. +3 of its row.
  float* yr = hd.y[h] + ((long)blockIdx.y * nrows + m) * C;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (i >= nbh) break;
    const int c = 16 * i + 4 * q;
    const floatx4 sv = *reinterpret_cast<const floatx4*>(hd.s[h] + c);
    const floatx4 cvv = *reinterpret_cast<const floatx4*>(hd.cv[h] + c);
    floatx4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = (acc[i][t] - mu * sv[t]) * rs + cvv[t];
    *reinterpret_cast<floatx4*>(yr + c) = o;
  }
}

}  // namespace

template <typename T>
hipError_t launch_edge_in(const float* h, int nrows, int C, const float* W, const float* bias, const int32_t* idx,
                          int B, int S, int D, T* x, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  if (C % 16 != 0 || D % 256 != 0) return hipErrorInvalidValue;
  k_edge_in<T><<<dim3((unsigned)(D / 256), (unsigned)((nrows + 63) / 64), (unsigned)B), 256, 0, st>>>(
      h, nrows, C, W, bias, idx, S, D, x);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_edge_rows(const T* text, const int32_t* idx, int ntext, const int32_t* tags, int B, int S, int D,
                            T* x, hipStream_t st) {
  if (ntext > 0) {
    k_edge_rows<T><<<dim3((unsigned)ntext, (unsigned)B), 256, 0, st>>>(text, idx, tags, ntext, S, D, x, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  k_edge_rows<T><<<dim3((unsigned)S, (unsigned)B), 256, 0, st>>>(text, idx, tags, ntext, S, D, x, 1);
  return hipGetLastError();
}

hipError_t launch_edge_fold(const float* W, const float* b, const float* gamma, const float* beta, int C, int D,
                            float* Wf, float* s, float* cv, hipStream_t st) {
  if (C <= 0) return hipSuccess;
  k_edge_fold<<<dim3((unsigned)C), 256, 0, st>>>(W, b, gamma, beta, D, Wf, s, cv);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_edge_out(const T* x, const EdgeHeads& hd, int B, int S, int D, float eps, hipStream_t st) {
  if (D % 64 != 0) return hipErrorInvalidValue;
  const int b0 = (hd.nrows[0] + 63) / 64, b1 = (hd.nrows[1] + 63) / 64;
  if (b0 + b1 == 0) return hipSuccess;
  if (hd.nrows[1] > 0 && hd.C[1] > hd.C[0]) return hipErrorInvalidValue;  // head 0 is the wider one
  dim3 g((unsigned)(b0 + b1), (unsigned)B);
  switch (hd.C[0]) {
    case 16: k_edge_out<T, 1><<<g, 256, 0, st>>>(x, hd, b0, S, D, eps); break;
    case 32: k_edge_out<T, 2><<<g, 256, 0, st>>>(x, hd, b0, S, D, eps); break;
    case 48: k_edge_out<T, 3><<<g, 256, 0, st>>>(x, hd, b0, S, D, eps); break;
    case 64: k_edge_out<T, 4><<<g, 256, 0, st>>>(x, hd, b0, S, D, eps); break;
    case 96: k_edge_out<T, 6><<<g, 256, 0, st>>>(x, hd, b0, S, D, eps); break;
    case 128: k_edge_out<T, 8><<<g, 256, 0, st>>>(x, hd, b0, S, D, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_edge_in<bf16_t>(const float*, int, int, const float*, const float*, const int32_t*, int,
                                           int, int, bf16_t*, hipStream_t);
template hipError_t launch_edge_in<float>(const float*, int, int, const float*, const float*, const int32_t*, int,
                                          int, int, float*, hipStream_t);
template hipError_t launch_edge_rows<bf16_t>(const bf16_t*, const int32_t*, int, const int32_t*, int, int, int,
                                             bf16_t*, hipStream_t);
template hipError_t launch_edge_rows<float>(const float*, const int32_t*, int, const int32_t*, int, int, int, float*,
                                            hipStream_t);
template hipError_t launch_edge_out<bf16_t>(const bf16_t*, const EdgeHeads&, int, int, int, float, hipStream_t);
template hipError_t launch_edge_out<float>(const float*, const EdgeHeads&, int, int, int, float, hipStream_t);

}  // namespace minih3
