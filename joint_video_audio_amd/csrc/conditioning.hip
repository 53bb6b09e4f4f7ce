// Timestep conditioning: the AdaLN tables of a block from the distinct
// timestep values of the packed sequence.
// Page "MiniMaxH3Transformer3DModel": Parameters freq_dim (sinusoidal
// timestep embedding, timesteps unscaled in [0, 1]), time_embed_hidden_dim
// and time_embed_dim (the timestep MLP, whose output feeds every AdaLN
// projection); the mixed-precision note (timestep MLP in float32, block
// stack in bfloat16); the class description (the row's modality tag selects
// its AdaLN modulation). Page "HyperFlow for MiniMax-H3", How it works: a
// second embedder for the step endpoint r, blended with a fixed gate.
//
// The conditioning batch holds one row per timestep value (a few dozen at
// most), so every contraction here is skinny: M <= 64 rows per launch
// column against thousands of weight rows. Weights stream from HBM once;
// the few input rows stay in L2.
//  * k_sinusoid: the sinusoidal embedding of the timesteps, once.
//  * k_skinny_f32: fp32 y = in(x) . W^T on v_mfma_f32_16x16x4_f32. A wave
//    owns 16 weight rows and up to 64 input rows over one K range; split-K
//    partial sums are added in a fixed order by k_rows_finish, which also
//    applies the bias, the SiLU and the two-time blend.
//  * k_adaln_proj: the bf16 table projection on v_mfma_f32_16x16x32_bf16;
//    a wave owns 64 weight rows and keeps four k-steps of weight and
//    activation fragments in flight.
#include "common.h"
#include "kernels.h"

namespace minih3 {

namespace {

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + expf(-v)); }

// Four consecutive inputs (row m, columns k..k+3) of the skinny product.
template <int IN>
__device__ __forceinline__ floatx4 skinny_in(const float* x, int m, int K, int k) {
  floatx4 v = *reinterpret_cast<const floatx4*>(x + (long)m * K + k);
  if constexpr (IN == kInSilu) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = silu_f(v[j]);
  }
  return v;
}

// fp32 fragment order of a [Mpad, K] matrix (Mpad, K multiples of 16): the
// 16-byte unit (mb * (K / 16) + st) * 64 + lane, lane = (r16, q), holds
// columns 16 st + 4q .. +3 of row 16 mb + r16 -- the B operand of
// v_mfma_f32_16x16x4_f32 for the four MFMAs of step st, and the layout in
// which the accumulators of a 16 x 16 output block leave the MFMA. A wave
// moves a 16 x 16 block as one contiguous 1 KB.

// s = [cos(t_m f_c), sin(t_m f_c)] over F columns, f_c = period^(-c / (F/2)),
// in fragment order with Mpad rows (zero past M); one thread a unit.
__global__ void __launch_bounds__(256) k_sinusoid(const float* __restrict__ t, float* __restrict__ s, int M, int Mpad,
                                                  int F, float log2_period) {
  const long u = (long)blockIdx.x * 256 + threadIdx.x;
  if (u >= (long)Mpad * F / 4) return;
  const int lane = (int)(u & 63);
  const long blk = u >> 6;
  const int KS = F / 16;
  const int mb = (int)(blk / KS), st = (int)(blk - (long)mb * KS);
  const int m = 16 * mb + (lane & 15), c0 = 16 * st + 4 * (lane >> 4);
  const int half = F >> 1;
  const bool is_sin = c0 >= half;  // four columns never straddle the halves (F/2 % 16 == 0)
  const int j0 = is_sin ? c0 - half : c0;
  floatx4 v = {0.f, 0.f, 0.f, 0.f};
  if (m < M) {
    const float tm = t[m];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float f = exp2f(-log2_period * (float)(j0 + j) / (float)half);
      float sv, cv;
      sincosf(tm * f, &sv, &cv);
      v[j] = is_sin ? sv : cv;
    }
  }
  *reinterpret_cast<floatx4*>(s + u * 4) = v;
}

// y[m, n] = sum_k in(x)[m, k] W[n, k] over k in this split's range.
// Grid: (ceil(N/64), splits, ceil(M / (16 MB))), 4 waves of 16 weight rows.
// XF: x is in fragment order with Mpad rows (plain input), else row-major.
// One split: act(y + bias) goes, with OF, to out in fragment order (Mpad
// rows, zero past M), else to out row (n / ng) * M + m at column n % ng;
// several splits: the raw partial sum goes to part[split][m][n].
template <int IN, int XF, int OF, int MB>
__global__ void __launch_bounds__(256) k_skinny_f32(const float* __restrict__ x, const float* __restrict__ w,
                                                    const float* __restrict__ bias, float* __restrict__ out,
                                                    int M, int N, int K, int kchunk, int ng, int act) {
  const int lane = threadIdx.x & 63;
  const int nb = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (nb * 16 >= N) return;  // whole wave; no barrier follows
  const int r16 = lane & 15, q = lane >> 4;
  const int k_beg = blockIdx.y * kchunk;
  const int k_end = min(K, k_beg + kchunk);
  const int m0 = blockIdx.z * 16 * MB;
  const float* wr = w + (long)(nb * 16 + r16) * K + 4 * q;

  constexpr int PF = 4;
  const int steps = (k_end - k_beg) / 16;
  floatx4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 wv[PF], xv[PF][MB];
  // Operands of 16-column step s: lane (r16, q) holds W[n0 + r16][k + 4q + j]
  // and in(x)[m0 + 16 mb + r16][k + 4q + j], k = k_beg + 16 s; MFMA j
  // contracts k slot q of both, so four MFMAs cover the step. Steps past the
  // end re-read the last one (and are not accumulated), so every iteration
  // issues the same loads and the in-order load counter stays exact.
  auto load = [&](int slot, int s) {
    const int k = k_beg + 16 * min(s, steps - 1) + 4 * q;
    wv[slot] = *reinterpret_cast<const floatx4*>(wr - 4 * q + k);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (XF) {
        const long unit = ((long)(m0 / 16 + mb) * (K / 16) + (k - 4 * q) / 16) * 64 + lane;
        xv[slot][mb] = *reinterpret_cast<const floatx4*>(x + unit * 4);
      } else {
        const int m = m0 + 16 * mb + r16;
        xv[slot][mb] = m < M ? skinny_in<IN>(x, m, K, k) : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
#pragma unroll
  for (int s = 0; s < PF - 1; ++s) load(s, s);
  for (int kt = 0; kt < steps; kt += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      load((s + PF - 1) % PF, kt + s + PF - 1);
      if (kt + s < steps) {  // consecutive MFMAs go to different accumulators
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[s][j], xv[s][mb][j], acc[mb], 0, 0, 0);
      }
    }
  }

  // Lane (r16, q) holds y[m0 + 16 mb + r16][n0 + 4q .. n0 + 4q + 3].
  const int n = nb * 16 + 4 * q;
  const bool split = gridDim.y > 1;
  floatx4 b = {0.f, 0.f, 0.f, 0.f};
  if (!split && bias) b = *reinterpret_cast<const floatx4*>(bias + n);
  const int g = n / ng, c = n - g * ng;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + 16 * mb + r16;
    if constexpr (OF) {
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      if (m < M) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = act ? silu_f(acc[mb][j] + b[j]) : acc[mb][j] + b[j];
      }
      *reinterpret_cast<floatx4*>(out + (((long)(m0 / 16 + mb) * (N / 16) + nb) * 64 + lane) * 4) = v;
      continue;
    }
    if (m >= M) continue;
    floatx4 v = acc[mb];
    if (split) {
      *reinterpret_cast<floatx4*>(out + ((long)blockIdx.y * M + m) * N + n) = v;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] += b[j];
        if (act) v[j] = silu_f(v[j]);
      }
      *reinterpret_cast<floatx4*>(out + ((long)g * M + m) * ng + c) = v;
    }
  }
}

// out[m, n] = act(sum_s part[s][m][n] + bias[n]); with prev, the blend
// (1 - gate) prev[m, n] + gate * that (prev may be out). Four columns a thread.
__global__ void __launch_bounds__(256) k_rows_finish(const float* __restrict__ part, int splits,
                                                     const float* __restrict__ bias, float* out, int M, int N,
                                                     int act, const float* prev, float gate) {
  const long i4 = (long)blockIdx.x * 256 + threadIdx.x;
  const long total4 = (long)M * N / 4;
  if (i4 >= total4) return;
  const long e = i4 * 4;
  const int n = (int)(e % N);
  floatx4 v = *reinterpret_cast<const floatx4*>(part + e);
  for (int s = 1; s < splits; ++s) v += *reinterpret_cast<const floatx4*>(part + (long)s * M * N + e);
  if (bias) v += *reinterpret_cast<const floatx4*>(bias + n);
  if (act) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = silu_f(v[j]);
  }
  if (prev) v = (1.f - gate) * *reinterpret_cast<const floatx4*>(prev + e) + gate * v;
  *reinterpret_cast<floatx4*>(out + e) = v;
}

// a = bf16(SiLU(e)) for m < M, zero for M <= m < Mpad, stored in MFMA
// fragment order: 16-byte unit ((mb * KT + ks) * 64 + lane), lane = (r16, q),
// holds a[16 mb + r16][32 ks + 8 q .. +7], KT = K / 32; one thread a unit.
__global__ void __launch_bounds__(256) k_silu_bf16(const float* __restrict__ e, bf16_t* __restrict__ a, int M,
                                                   int Mpad, int K) {
  const long u = (long)blockIdx.x * 256 + threadIdx.x;
  const int KT = K / 32;
  if (u >= (long)Mpad * K / 8) return;
  const int lane = (int)(u & 63);
  const long blk = u >> 6;  // mb * KT + ks
  const int mb = (int)(blk / KT), ks = (int)(blk - (long)mb * KT);
  const int m = 16 * mb + (lane & 15), k = 32 * ks + 8 * (lane >> 4);
  u32x4 r = {0u, 0u, 0u, 0u};
  if (m < M) {
    const floatx4 v0 = *reinterpret_cast<const floatx4*>(e + (long)m * K + k);
    const floatx4 v1 = *reinterpret_cast<const floatx4*>(e + (long)m * K + k + 4);
    r[0] = pack_bf16x2(silu_f(v0[0]), silu_f(v0[1]));
    r[1] = pack_bf16x2(silu_f(v0[2]), silu_f(v0[3]));
    r[2] = pack_bf16x2(silu_f(v1[0]), silu_f(v1[1]));
    r[3] = pack_bf16x2(silu_f(v1[2]), silu_f(v1[3]));
  }
  *reinterpret_cast<u32x4*>(a + u * 8) = r;
}

// table[(n / ng) * M + m][n % ng] = sum_k a[m, k] W[n, k] + bias[n] with
// bf16 W and a, fp32 accumulation. One wave per workgroup owns weight rows
// n0 .. n0+63 (four 16-row blocks) and MB 16-row blocks of a from m0.
// a has Mpad rows (a multiple of 16 MB, zero past M) in fragment order, so
// each of its loads is one contiguous 1 KB; K is a multiple of 32.
template <int MB>
__global__ void __launch_bounds__(64) k_adaln_proj(const bf16_t* __restrict__ w, const bf16_t* __restrict__ bias,
                                                   const bf16_t* __restrict__ a, float* __restrict__ table, int M,
                                                   int K, int ng) {
  constexpr int NB = 4, PF = 4;
  const int lane = threadIdx.x;
  const int r16 = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB;
  const int m0 = blockIdx.y * 16 * MB;
  const long kb16 = 16L * K;
  const bf16_t* wp = w + (long)(n0 + r16) * K + 8 * q;
  const bf16_t* ap = a + ((long)(m0 / 16) * (K / 32) * 64 + lane) * 8;  // fragment-major
  const int KT = K / 32;

  floatx4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  u32x4 wf[PF][NB], af[PF][MB];

  // Fragments of k-step s: lane (r16, q) holds W[n0 + 16 i + r16][32 s + 8q .. +7]
  // (A operand) and a[m0 + 16 j + r16][32 s + 8q .. +7] (B operand). Steps
  // past the end re-read the last one (and are not accumulated), so every
  // iteration issues the same loads and the in-order load counter stays exact.
  auto load = [&](int slot, int s) {
    s = min(s, KT - 1);
#pragma unroll
    for (int i = 0; i < NB; ++i) wf[slot][i] = *reinterpret_cast<const u32x4*>(wp + i * kb16 + 32 * s);
#pragma unroll
    for (int j = 0; j < MB; ++j) af[slot][j] = *reinterpret_cast<const u32x4*>(ap + ((long)j * KT + s) * 512);
  };
#pragma unroll
  for (int s = 0; s < PF - 1; ++s) load(s, s);
  for (int kt = 0; kt < KT; kt += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      load((s + PF - 1) % PF, kt + s + PF - 1);
      if (kt + s < KT) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < MB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[s][i]),
                                                                __builtin_bit_cast(bf16x8, af[s][j]), acc[i][j], 0,
                                                                0, 0);
      }
    }
  }

  // Lane (r16, q) holds rows n0 + 16 i + 4q .. +3 for input row m0 + 16 j + r16.
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + 16 * i + 4 * q;
    floatx4 b = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const u32x2 bb = *reinterpret_cast<const u32x2*>(bias + n);
      b = floatx4{__uint_as_float(bb[0] << 16), __uint_as_float(bb[0] & 0xffff0000u), __uint_as_float(bb[1] << 16),
                  __uint_as_float(bb[1] & 0xffff0000u)};
    }
    const int g = n / ng, c = n - g * ng;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int m = m0 + 16 * j + r16;
      if (m < M) *reinterpret_cast<floatx4*>(table + ((long)g * M + m) * ng + c) = acc[i][j] + b;
    }
  }
}

int mblocks(int M) { return M > 32 ? 4 : (M > 16 ? 2 : 1); }

// K range of one split: K / splits rounded up to whole 16-column steps.
int skinny_kchunk(int K, int splits) { return ((K + splits - 1) / splits + 15) / 16 * 16; }

}  // namespace

template <int IN, int XF, int OF>
static void skinny_launch(dim3 grid, int mb, const float* x, const float* w, const float* bias, float* out, int M,
                          int N, int K, int kchunk, int ng, int act, hipStream_t st) {
  if (mb == 4)
    k_skinny_f32<IN, XF, OF, 4><<<grid, 256, 0, st>>>(x, w, bias, out, M, N, K, kchunk, ng, act);
  else if (mb == 2)
    k_skinny_f32<IN, XF, OF, 2><<<grid, 256, 0, st>>>(x, w, bias, out, M, N, K, kchunk, ng, act);
  else
    k_skinny_f32<IN, XF, OF, 1><<<grid, 256, 0, st>>>(x, w, bias, out, M, N, K, kchunk, ng, act);
}

hipError_t launch_skinny_f32(int mode, const float* x, const float* w, const float* bias, float* out, int M, int N,
                             int K, int splits, int ng, int act, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int mb = mblocks(M);
  const int kchunk = skinny_kchunk(K, splits);
  splits = (K + kchunk - 1) / kchunk;
  if (mode == kFragToFrag && splits != 1) return hipErrorInvalidValue;
  dim3 grid((unsigned)((N / 16 + 3) / 4), (unsigned)splits, (unsigned)((M + 16 * mb - 1) / (16 * mb)));
  if (mode == kFragToFrag)
    skinny_launch<kInPlain, 1, 1>(grid, mb, x, w, bias, out, M, N, K, kchunk, ng, act, st);
  else if (mode == kFragToRows)
    skinny_launch<kInPlain, 1, 0>(grid, mb, x, w, bias, out, M, N, K, kchunk, ng, act, st);
  else
    skinny_launch<kInSilu, 0, 0>(grid, mb, x, w, bias, out, M, N, K, kchunk, ng, act, st);
  return hipGetLastError();
}

hipError_t launch_sinusoid(const float* t, float* s, int M, int F, float period, hipStream_t st) {
  const long n = (long)padded_rows(M) * F / 4;
  if (n <= 0) return hipSuccess;
  k_sinusoid<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(t, s, M, padded_rows(M), F, log2f(period));
  return hipGetLastError();
}

int skinny_splits(int K, int splits) {
  const int kchunk = skinny_kchunk(K, splits);
  return (K + kchunk - 1) / kchunk;
}

hipError_t launch_rows_finish(const float* part, int splits, const float* bias, float* out, int M, int N, int act,
                              const float* prev, float gate, hipStream_t st) {
  const long n4 = (long)M * N / 4;
  if (n4 <= 0) return hipSuccess;
  k_rows_finish<<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, st>>>(part, splits, bias, out, M, N, act, prev, gate);
  return hipGetLastError();
}

int padded_rows(int M) { return ((M + 16 * mblocks(M) - 1) / (16 * mblocks(M))) * 16 * mblocks(M); }

hipError_t launch_adaln_proj(const float* emb, const bf16_t* w, const bf16_t* bias, bf16_t* a_scratch, float* table,
                             int M, int N, int K, int ng, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int mb = mblocks(M);
  const int Mpad = padded_rows(M);
  const long n8 = (long)Mpad * K / 8;
  k_silu_bf16<<<dim3((unsigned)((n8 + 255) / 256)), 256, 0, st>>>(emb, a_scratch, M, Mpad, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(N / 64), (unsigned)(Mpad / (16 * mb)));
  if (mb == 4)
    k_adaln_proj<4><<<grid, 64, 0, st>>>(w, bias, a_scratch, table, M, K, ng);
  else if (mb == 2)
    k_adaln_proj<2><<<grid, 64, 0, st>>>(w, bias, a_scratch, table, M, K, ng);
  else
    k_adaln_proj<1><<<grid, 64, 0, st>>>(w, bias, a_scratch, table, M, K, ng);
  return hipGetLastError();
}

}  // namespace minih3
