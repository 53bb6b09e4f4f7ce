// Projections of the block: C[M, N] = A[M, K] . W[N, K]^T, fp32 accumulate.
//
// The page "MiniMaxH3Transformer3DModel" fixes the widths (Parameters):
// hidden_size 5376 for the residual, num_attention_heads * attention_head_dim
// = 7168 for the attention projections, ffn_dim 14336 for each half of the
// SwiGLU feed-forward. No biases (not mentioned on the page).
//
// Fused epilogues:
//   kEpiStore      : C = acc
//   kEpiGatedResid : C = resid + gate[row] * acc   (gate from the AdaLN table;
//                    a padding row keeps resid unchanged)
//   kEpiSwiGLU     : W rows [0,F) gate, [F,2F) up; C[:, f] = silu(g_f) * u_f
//
// bf16 kernel (gfx950): 256x256 output tile per workgroup of 8 waves (two per
// SIMD), each wave 128x64 as 4x2 v_mfma_f32_32x32x16_bf16 tiles; K step 64 staged in
// LDS (2 stages, 128 KiB). Rows are 128 bytes; the 16-byte chunk c of row r
// sits at c ^ ((r >> 1) & 7), so the 16 lanes a ds_read_b128 serves together
// (16 consecutive rows, one chunk) hit 16 different bank groups of the 64
// banks, and so do tile stores (2 rows x 8 chunks); global loads of step k+1 are in
// flight while step k is multiplied. Tiles are ordered so that the
// workgroups an XCD runs together share A and W panels in its L2.
#include "common.h"
#include "kernels.h"

namespace minih3 {

// ---------------------------------------------------------------- epilogue

template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* v) {
  u32x2 r;
  r[0] = pack_bf16x2(v[0], v[1]);
  r[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(p) = r;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<floatx4*>(p) = floatx4{v[0], v[1], v[2], v[3]};
}
template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v);
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float* v) {
  u32x2 r = *reinterpret_cast<const u32x2*>(p);
  v[0] = __uint_as_float(r[0] << 16);
  v[1] = __uint_as_float(r[0] & 0xffff0000u);
  v[2] = __uint_as_float(r[1] << 16);
  v[3] = __uint_as_float(r[1] & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  floatx4 r = *reinterpret_cast<const floatx4*>(p);
  v[0] = r[0];
  v[1] = r[1];
  v[2] = r[2];
  v[3] = r[3];
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

// Gated residual for 4 consecutive output columns n..n+3 of row m.
template <typename T>
__device__ __forceinline__ void epi_gated(T* C, int ldc, int m, int n, const float* acc, const EpiArgs& ea) {
  const T* resid = reinterpret_cast<const T*>(ea.resid);
  float r[4];
  load4<T>(resid + (long)m * ldc + n, r);
  const int s = m % ea.S;
  const int tr = table_row_of(ea.tags[s], ea.tidx[s], ea.num_tags, ea.num_tvals);
  if (tr >= 0) {
    floatx4 g = *reinterpret_cast<const floatx4*>(ea.table + ((long)tr * 6 + ea.gate_slot) * ldc + n);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] += g[j] * acc[j];
  }
  store4<T>(C + (long)m * ldc + n, r);
}

// ---------------------------------------------------------------- bf16 MFMA kernel

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kStageBytes = (BM + BN) * BK * 2;  // 64 KiB

// WGM x WGN waves; each wave owns a (256/WGM) x (256/WGN) block of the tile.
template <int EPI, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
    k_gemm_bf16(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, bf16_t* __restrict__ C, int M, int N,
                int K, EpiArgs ea) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int MI = WTM / 32, NI = WTN / 32;    // 32x32 MFMA blocks per wave
  constexpr int LPT = BM * 8 / NT;               // 16-byte chunks per thread per operand and K step
  constexpr int RSTEP = NT / 8;                  // row step between a thread's chunks
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid % WGM, wn = wid / WGM;

  // ---- tile order: XCD-contiguous ranges, then groups of 8 M-tiles
  const int MT = (M + BM - 1) / BM, NTL = N / BN;
  const int T = MT * NTL;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int q8 = T >> 3, r8 = T & 7;
  const int pid = xcd * q8 + (xcd < r8 ? xcd : r8) + loc;
  constexpr int GROUP_M = 8;
  const int npg = GROUP_M * NTL;
  const int g = pid / npg;
  const int first_m = g * GROUP_M;
  const int gsz = MT - first_m < GROUP_M ? MT - first_m : GROUP_M;
  const int tm = first_m + (pid % npg) % gsz;
  const int tn = (pid % npg) / gsz;
  const int m0 = tm * BM;

  // ---- global -> LDS mapping: thread owns chunk column (tid & 7) of rows (tid >> 3) + RSTEP i
  const int ck = tid & 7;
  const int r0 = tid >> 3;
  const int swz = ck ^ ((r0 >> 1) & 7);  // rows r0 + RSTEP i share (row >> 1) & 7
  const bf16_t* a_src[LPT];
  const bf16_t* w_src[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int row = r0 + RSTEP * i;
    int am = m0 + row;
    am = am < M ? am : M - 1;
    a_src[i] = A + (long)am * K + ck * 8;
    int wr;
    if (EPI == kEpiSwiGLU) {
      // wave block of WTN rows: first half gate rows, second half the matching up rows
      const int wblk = row / WTN, sel = (row % WTN) / (WTN / 2), o = row % (WTN / 2);
      wr = sel * ea.ffn_dim + 128 * tn + (WTN / 2) * wblk + o;
    } else {
      wr = tn * BN + row;
    }
    w_src[i] = W + (long)wr * K + ck * 8;
  }
  const int st_off = r0 * 128 + (swz << 4);  // + i * RSTEP * 128

  floatx16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4 ra[LPT], rw[LPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + kt * BK);
      rw[i] = *reinterpret_cast<const u32x4*>(w_src[i] + kt * BK);
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* As = lds + stage * kStageBytes;
    uint8_t* Ws = As + BM * BK * 2;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      *reinterpret_cast<u32x4*>(As + st_off + i * RSTEP * 128) = ra[i];
      *reinterpret_cast<u32x4*>(Ws + st_off + i * RSTEP * 128) = rw[i];
    }
  };

  // fragment read offsets: row (lane & 31) of a 32-row block, chunk 2kk + (lane >> 5)
  const int fr_row = lane & 31, fr_hi = lane >> 5, fr_sw = (fr_row >> 1) & 7;

  const int KT = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* As = lds + stage * kStageBytes;
    const uint8_t* Ws = As + BM * BK * 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = ((2 * kk + fr_hi) ^ fr_sw) << 4;
      bf16x8 wf[NI], af[MI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        wf[ni] = *reinterpret_cast<const bf16x8*>(Ws + (wn * WTN + ni * 32 + fr_row) * 128 + chunk);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(As + (wm * WTM + mi * 32 + fr_row) * 128 + chunk);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ni], af[mi], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds row m = ... + (lane & 31), columns 8i + 4*(lane>>5) + j
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = m0 + wm * WTM + mi * 32 + fr_row;
    if (m >= M) continue;
    if (EPI == kEpiSwiGLU) {
      const int F = ea.ffn_dim;
#pragma unroll
      for (int ni = 0; ni < NI / 2; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = silu(acc[mi][ni][4 * i + j]) * acc[mi][ni + NI / 2][4 * i + j];
          const int f = 128 * tn + (WTN / 2) * wn + ni * 32 + 8 * i + 4 * fr_hi;
          store4<bf16_t>(C + (long)m * F + f, v);
        }
    } else {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = tn * BN + wn * WTN + ni * 32 + 8 * i + 4 * fr_hi;
          float v[4] = {acc[mi][ni][4 * i], acc[mi][ni][4 * i + 1], acc[mi][ni][4 * i + 2], acc[mi][ni][4 * i + 3]};
          if (EPI == kEpiGatedResid)
            epi_gated<bf16_t>(C, N, m, n, v, ea);
          else
            store4<bf16_t>(C + (long)m * N + n, v);
        }
    }
  }
}

// ---------------------------------------------------------------- fp32 kernel
// Plain LDS-tiled FMA kernel for fp32 storage (small workloads, parity).
// 64x64 output tile, 256 threads with 4x4 outputs each, K step 16.

template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_f32(const float* __restrict__ A, const float* __restrict__ W,
                                                  float* __restrict__ C, int M, int N, int K, EpiArgs ea) {
  constexpr int TM = 64, TN = 64, TK = 16;
  constexpr int NB = EPI == kEpiSwiGLU ? 2 : 1;
  __shared__ float As[TK][TM + 4];
  __shared__ float Ws[NB][TK][TN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int ldc = EPI == kEpiSwiGLU ? ea.ffn_dim : N;
  float acc[NB][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int e = tid; e < TM * TK; e += 256) {
      const int r = e / TK, c = e % TK;
      const int m = m0 + r < M ? m0 + r : M - 1;
      As[c][r] = A[(long)m * K + k0 + c];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int wr = (EPI == kEpiSwiGLU ? b * ea.ffn_dim : 0) + n0 + r;
        Ws[b][c][r] = W[(long)wr * K + k0 + c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < TK; ++c) {
      float a[4], w[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[c][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[b][j] = Ws[b][c][tx * 4 + j];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] += a[i] * w[b][j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    const int n = n0 + tx * 4;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = EPI == kEpiSwiGLU ? silu(acc[0][i][j]) * acc[NB - 1][i][j] : acc[0][i][j];
    if (EPI == kEpiGatedResid)
      epi_gated<float>(C, ldc, m, n, v, ea);
    else
      store4<float>(C + (long)m * ldc + n, v);
  }
}

// ---------------------------------------------------------------- launchers

#ifndef MINIH3_GEMM_WAVES
#define MINIH3_GEMM_WAVES 8
#endif
constexpr int kGemmWGM = 2, kGemmWGN = MINIH3_GEMM_WAVES / 2;

template <>
hipError_t launch_gemm<bf16_t>(int epi, const bf16_t* A, const bf16_t* W, bf16_t* C, int M, int N, int K,
                               const EpiArgs& ea, hipStream_t st) {
  if (M <= 0 || N % BN != 0 || K % BK != 0) return hipErrorInvalidValue;
  if (epi == kEpiSwiGLU && (N != 2 * ea.ffn_dim || ea.ffn_dim % 128 != 0)) return hipErrorInvalidValue;
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  dim3 grid((unsigned)tiles);
  constexpr int NT = 64 * kGemmWGM * kGemmWGN;
  switch (epi) {
    case kEpiStore: k_gemm_bf16<kEpiStore, kGemmWGM, kGemmWGN><<<grid, NT, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiGatedResid:
      k_gemm_bf16<kEpiGatedResid, kGemmWGM, kGemmWGN><<<grid, NT, 0, st>>>(A, W, C, M, N, K, ea);
      break;
    case kEpiSwiGLU: k_gemm_bf16<kEpiSwiGLU, kGemmWGM, kGemmWGN><<<grid, NT, 0, st>>>(A, W, C, M, N, K, ea); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <>
hipError_t launch_gemm<float>(int epi, const float* A, const float* W, float* C, int M, int N, int K,
                              const EpiArgs& ea, hipStream_t st) {
  if (M <= 0 || N % 64 != 0 || K % 16 != 0) return hipErrorInvalidValue;
  const int ncols = epi == kEpiSwiGLU ? ea.ffn_dim : N;
  if (epi == kEpiSwiGLU && (N != 2 * ea.ffn_dim || ea.ffn_dim % 64 != 0)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(ncols / 64), (unsigned)((M + 63) / 64));
  switch (epi) {
    case kEpiStore: k_gemm_f32<kEpiStore><<<grid, 256, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiGatedResid: k_gemm_f32<kEpiGatedResid><<<grid, 256, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiSwiGLU: k_gemm_f32<kEpiSwiGLU><<<grid, 256, 0, st>>>(A, W, C, M, N, K, ea); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace minih3
