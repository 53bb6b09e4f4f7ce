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
// SIMD), each wave 128x64 as 4x2 v_mfma_f32_32x32x16_bf16 tiles. K steps of 32
// go through a ring of 4 LDS stages (128 KiB) filled by direct global->LDS
// loads (global_load_lds_dwordx4) three steps ahead, so no registers stage
// the operands and the load latency hides behind three steps of MFMA work;
// one barrier per step. Tiles are ordered so that the workgroups an XCD runs
// together share A and W panels in its L2.
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

constexpr int BM = 256, BN = 256;
#ifndef MINIH3_GEMM_BK
#define MINIH3_GEMM_BK 64
#endif
#ifndef MINIH3_GEMM_STAGES
#define MINIH3_GEMM_STAGES 2
#endif
constexpr int BK = MINIH3_GEMM_BK;                  // K step (32 or 64)
constexpr int kStages = MINIH3_GEMM_STAGES;         // LDS ring depth; loads run kStages-1 steps ahead
constexpr int kRowBytes = BK * 2;                   // one tile row per stage
constexpr int kCPR = kRowBytes / 16;                // 16-byte chunks per row
constexpr int kOpBytes = BM * kRowBytes;            // one operand tile per stage
constexpr int kStageBytes = 2 * kOpBytes;           // A + W
static_assert(kStages * kStageBytes <= 160 * 1024, "LDS");

// Logical chunk c of tile row r sits at chunk c ^ swz(r): the 16 lanes a
// ds_read_b128 serves together read 16 consecutive rows at one chunk, and
// (r * kCPR + physical chunk) mod 16 -- the 16-byte bank group -- is then
// different for all 16.
__device__ __forceinline__ int gemm_swz(int r) { return (r / (16 / kCPR)) % kCPR; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// WGM x WGN waves (two per SIMD); each wave owns a (256/WGM) x (256/WGN)
// block of the 256x256 tile.
template <int EPI, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
    k_gemm_bf16(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, bf16_t* __restrict__ C, int M, int N,
                int K, EpiArgs ea) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int MI = WTM / 32, NI = WTN / 32;    // 32x32 MFMA blocks per wave
  constexpr int INSTS = 2 * kOpBytes / 1024;     // 1 KiB LDS-DMA wave instructions per stage (A then W)
  constexpr int IPW = INSTS / NW;                // ... per wave
  static_assert(INSTS % NW == 0, "DMA split");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStageBytes];

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

  // ---- LDS-DMA sources. A DMA wave instruction fills 1 KiB of a stage =
  // 1024 / kRowBytes rows; lane L writes row (1024 / kRowBytes) u + L / kCPR,
  // physical chunk L % kCPR, i.e. logical chunk (L % kCPR) ^ swz(row).
  const bf16_t* src[IPW];
  int dst_off[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int u = wid * IPW + j;                 // instruction index in the stage
    const bool is_w = u >= INSTS / 2;
    const int ub = is_w ? u - INSTS / 2 : u;
    const int row = (1024 / kRowBytes) * ub + lane / kCPR;
    const int c = (lane % kCPR) ^ gemm_swz(row);
    if (is_w) {
      int wr;
      if (EPI == kEpiSwiGLU) {
        // wave block of WTN rows: first half gate rows, second half the matching up rows
        const int wblk = row / WTN, sel = (row % WTN) / (WTN / 2), o = row % (WTN / 2);
        wr = sel * ea.ffn_dim + 128 * tn + (WTN / 2) * wblk + o;
      } else {
        wr = tn * BN + row;
      }
      src[j] = W + (long)wr * K + c * 8;
    } else {
      int am = m0 + row;
      am = am < M ? am : M - 1;
      src[j] = A + (long)am * K + c * 8;
    }
    dst_off[j] = (is_w ? kOpBytes : 0) + ub * 1024;
  }
  auto issue = [&](int kt) {
    uint8_t* stage = lds + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + kt * BK), (lds_ptr_t)(stage + dst_off[j]), 16, 0, 0);
  };

  floatx16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment read offsets: row (lane & 31) of a 32-row block, chunk 2kk + (lane >> 5)
  const int fr_row = lane & 31, fr_hi = lane >> 5, fr_sw = gemm_swz(fr_row);
  auto compute = [&](int kt) {
    const uint8_t* As = lds + (kt % kStages) * kStageBytes;
    const uint8_t* Ws = As + kOpBytes;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = ((2 * kk + fr_hi) ^ fr_sw) << 4;
      bf16x8 wf[NI], af[MI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        wf[ni] = *reinterpret_cast<const bf16x8*>(Ws + (wn * WTN + ni * 32 + fr_row) * kRowBytes + chunk);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(As + (wm * WTM + mi * 32 + fr_row) * kRowBytes + chunk);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ni], af[mi], acc[mi][ni], 0, 0, 0);
    }
  };

  // ---- pipeline: stages kt+1 .. kt+3 in flight while kt is multiplied.
  // Before the barrier of step kt a wave waits until its own DMA of stage kt
  // has landed (at most the later stages' IPW-instruction groups outstanding);
  // the barrier then publishes stage kt to every wave and guarantees that
  // all waves are done with the stage the next DMA overwrites.
  const int KT = K / BK;
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < KT) issue(p);
  for (int kt = 0; kt < KT; ++kt) {
    const int later = KT - 1 - kt;  // stages issued after kt (at most kStages - 2)
    if (kStages >= 4 && later >= 2)
      wait_vmcnt<(kStages >= 4 ? 2 : 0) * IPW>();
    else if (kStages >= 3 && later >= 1)
      wait_vmcnt<(kStages >= 3 ? 1 : 0) * IPW>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + kStages - 1 < KT) issue(kt + kStages - 1);
    compute(kt);
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
  if (M <= 0 || N % BN != 0 || K % 64 != 0) return hipErrorInvalidValue;
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
