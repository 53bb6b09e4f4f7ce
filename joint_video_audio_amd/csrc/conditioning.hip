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
//    a wave owns 64 weight rows and streams them through its own LDS ring
//    in long contiguous runs.
#include "common.h"
#include "kernels.h"

namespace minih3 {

namespace {

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + expf(-v)); }

// Operands of up to two independent chains (the base timestep MLP and the
// step-endpoint one) handled by one launch.
template <typename P>
struct Pair {
  P p[2];
};

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
// in fragment order with Mpad rows (zero past M); one thread a unit. Grid
// row y handles the timesteps t[y] into s[y] (base and step endpoint).
__global__ void __launch_bounds__(256) k_sinusoid(Pair<const float*> tp, Pair<float*> sp, int M, int Mpad, int F,
                                                  float log2_period) {
  const float* __restrict__ t = tp.p[blockIdx.y];
  float* __restrict__ s = sp.p[blockIdx.y];
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
// Grid: (ceil(N/64), splits, chains * ceil(M / (16 MB))), 4 waves of 16
// weight rows; grid z picks the chain (its x, W, bias, out) and the row chunk.
// XF: x is in fragment order with Mpad rows (plain input), else row-major.
// One split: act(y + bias) goes, with OF, to out in fragment order (Mpad
// rows, zero past M), else to out row (n / ng) * M + m at column n % ng;
// several splits: the raw partial sum goes to part[split][m][n].
// With k2 > 0 (XF only) the last k2 columns of the input come from x2 in
// its own fragment order ([Mpad, k2]) and x holds the first K - k2 columns.
// scale multiplies the product before the bias and the activation.
template <int IN, int XF, int OF, int MB, int S2>
__global__ void __launch_bounds__(256) k_skinny_f32(Pair<const float*> xp, Pair<const float*> wp,
                                                    Pair<const float*> bp, Pair<float*> op, int mchunks, int M,
                                                    int N, int K, int kchunk, int ng, int act, Pair<const float*> x2p,
                                                    int k2, float scale) {
  const int lane = threadIdx.x & 63;
  const int nb = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (nb * 16 >= N) return;  // whole wave; no barrier follows
  const int chain = blockIdx.z / mchunks;
  const float* __restrict__ x = xp.p[chain];
  const float* __restrict__ x2 = x2p.p[chain];
  const int K1 = K - k2;  // columns held by x
  const float* __restrict__ w = wp.p[chain];
  const float* __restrict__ bias = bp.p[chain];
  float* __restrict__ out = op.p[chain];
  const int r16 = lane & 15, q = lane >> 4;
  const int k_beg = blockIdx.y * kchunk;
  const int k_end = min(K, k_beg + kchunk);
  const int m0 = (blockIdx.z - chain * mchunks) * 16 * MB;
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
        const int ks = k - 4 * q;  // first column of the step
        if (S2 && ks >= K1) {  // S2: the input has a second part (the steps from K1 on)
          const long unit = ((long)(m0 / 16 + mb) * (k2 / 16) + (ks - K1) / 16) * 64 + lane;
          xv[slot][mb] = *reinterpret_cast<const floatx4*>(x2 + unit * 4);
        } else {
          const long unit = ((long)(m0 / 16 + mb) * (K1 / 16) + ks / 16) * 64 + lane;
          xv[slot][mb] = *reinterpret_cast<const floatx4*>(x + unit * 4);
        }
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
        for (int j = 0; j < 4; ++j) {
          const float y = scale * acc[mb][j] + b[j];
          v[j] = act ? silu_f(y) : y;
        }
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
        v[j] = scale * v[j] + b[j];
        if (act) v[j] = silu_f(v[j]);
      }
      *reinterpret_cast<floatx4*>(out + ((long)g * M + m) * ng + c) = v;
    }
  }
}

// y_c[m, n] = act(sum_s part_c[s][m][n] + bias_c[n]) for each chain c; out is
// y_0, or with two chains the blend (1 - gate) y_0 + gate y_1. Four columns
// a thread; the partial sums are added in split order.
__global__ void __launch_bounds__(256) k_rows_finish(Pair<const float*> pp, Pair<const float*> bp, int chains,
                                                     int splits, float* __restrict__ out, int M, int N, int act,
                                                     float gate) {
  const long i4 = (long)blockIdx.x * 256 + threadIdx.x;
  const long total4 = (long)M * N / 4;
  if (i4 >= total4) return;
  const long e = i4 * 4;
  const int n = (int)(e % N);
  floatx4 y[2];
  for (int c = 0; c < chains; ++c) {
    const float* part = pp.p[c];
    floatx4 v = *reinterpret_cast<const floatx4*>(part + e);
    for (int s = 1; s < splits; ++s) v += *reinterpret_cast<const floatx4*>(part + (long)s * M * N + e);
    if (bp.p[c]) v += *reinterpret_cast<const floatx4*>(bp.p[c] + n);
    if (act) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = silu_f(v[j]);
    }
    y[c] = v;
  }
  *reinterpret_cast<floatx4*>(out + e) = chains == 2 ? (1.f - gate) * y[0] + gate * y[1] : y[0];
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS (buffer form): lane
// L of the wave lands at dst + 16 L; voff is the lane's byte offset.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, lds_ptr_t dst) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// table[(n / ng) * M + m][n % ng] = sum_k a[m, k] W[n, k] + bias[n] with
// bf16 W and a, fp32 accumulation. One wave per workgroup owns weight rows
// n0 .. n0+63 (four 16-row blocks) and MB 16-row blocks of a from m0.
//
// The weights are the only large operand. They are streamed through a
// three-stage LDS ring private to the wave (no barriers): a stage is 128
// columns of the 64 rows, moved by 16 buffer-to-LDS instructions that each
// read 4 rows x 256 contiguous bytes, so every row is fetched in long runs.
// Row r of a stage sits at r * 256 bytes with 16-byte chunk c stored at c ^
// (r & 15): the 16 lanes of a fragment read (16 rows, one chunk) hit 16
// different bank groups. a has Mpad rows (a multiple of 16 MB, zero past M)
// in fragment order, so each of its loads is one contiguous 1 KB; it is
// loaded into registers in the same group as the stage's weights, which
// keeps the in-order load counter exact. K is a multiple of 32; columns past
// K are clamped on load and their k-steps skipped.
template <int MB>
__global__ void __launch_bounds__(64) k_adaln_proj(const bf16_t* __restrict__ w, const bf16_t* __restrict__ bias,
                                                   const bf16_t* __restrict__ a, float* __restrict__ table, int M,
                                                   int K, int ng) {
  constexpr int NB = 4, NS = 3, SPS = 4;         // n-blocks, ring stages, k-steps per stage
  constexpr int kStageBytes = 64 * SPS * 64;     // 64 rows x 256 bytes
  constexpr int kOps = 16 + SPS * MB;            // loads issued per stage
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * kStageBytes];
  const int lane = threadIdx.x;
  const int r16 = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB;
  const int m0 = blockIdx.y * 16 * MB;
  const int KT = K / 32, KG = (KT + SPS - 1) / SPS;
  const bf16_t* ap = a + ((long)(m0 / 16) * KT * 64 + lane) * 8;  // fragment order

  floatx4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  u32x4 af[NS][SPS][MB];

  // DMA instruction j of a stage: rows 4j .. 4j+3; lane L takes row
  // 4j + L/16 and logical chunk (L % 16) ^ (row & 15) of the stage's 256 bytes.
  const int drow0 = lane >> 4, dchunk = lane & 15;
  // Stage g: weight columns 128 g .. 128 g + 127 into ring slot `slot`, and
  // the a fragments of k-steps 4 g .. 4 g + 3 (clamped to the last one).
  auto issue = [&](int slot, int g) {
    g = min(g, KG - 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = 4 * j + drow0;
      const int col = min(128 * g + 8 * (dchunk ^ (row & 15)), K - 8);
      dma16(w, (uint32_t)(((long)(n0 + row) * K + col) * 2),
            (lds_ptr_t)(lds + slot * kStageBytes + j * 1024));
    }
#pragma unroll
    for (int ss = 0; ss < SPS; ++ss) {
      const int s = min(SPS * g + ss, KT - 1);
#pragma unroll
      for (int jm = 0; jm < MB; ++jm) af[slot][ss][jm] = *reinterpret_cast<const u32x4*>(ap + ((long)jm * KT + s) * 512);
    }
  };
  auto compute = [&](int slot, int g) {
    const uint8_t* st = lds + slot * kStageBytes;
#pragma unroll
    for (int ss = 0; ss < SPS; ++ss) {
      if (SPS * g + ss >= KT) break;
      u32x4 wf[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int row = 16 * i + r16;
        wf[i] = *reinterpret_cast<const u32x4*>(st + row * 256 + 16 * ((SPS * ss + q) ^ (row & 15)));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int jm = 0; jm < MB; ++jm)
          acc[i][jm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[i]),
                                                               __builtin_bit_cast(bf16x8, af[slot][ss][jm]),
                                                               acc[i][jm], 0, 0, 0);
    }
  };

  issue(0, 0);
  issue(1, 1);
  for (int g0 = 0; g0 < KG; g0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int g = g0 + u;
      // stage g landed once only the group issued after it is outstanding;
      // its slot's previous contents were consumed by the last iteration
      wait_vmcnt<kOps>();
      issue((u + 2) % NS, g + 2);
      if (g < KG) compute(u, g);
    }
  }
  wait_vmcnt<0>();

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
static void skinny_launch(dim3 grid, int mb, const SkinnyArgs& g, int mchunks, int M, int N, int K, int kchunk,
                          int ng, int act, hipStream_t st) {
  const Pair<const float*> xp{{g.x[0], g.x[1]}}, wp{{g.w[0], g.w[1]}}, bp{{g.bias[0], g.bias[1]}};
  const Pair<const float*> x2p{{g.x2[0], g.x2[1]}};
  const Pair<float*> op{{g.out[0], g.out[1]}};
  // the two-part input gets its own instantiation: the test of the part
  // inside the load loop would otherwise sit among the MFMAs of every launch
  if (g.k2 > 0) {
    if (mb == 4)
      k_skinny_f32<IN, XF, OF, 4, 1><<<grid, 256, 0, st>>>(xp, wp, bp, op, mchunks, M, N, K, kchunk, ng, act, x2p,
                                                           g.k2, g.scale);
    else if (mb == 2)
      k_skinny_f32<IN, XF, OF, 2, 1><<<grid, 256, 0, st>>>(xp, wp, bp, op, mchunks, M, N, K, kchunk, ng, act, x2p,
                                                           g.k2, g.scale);
    else
      k_skinny_f32<IN, XF, OF, 1, 1><<<grid, 256, 0, st>>>(xp, wp, bp, op, mchunks, M, N, K, kchunk, ng, act, x2p,
                                                           g.k2, g.scale);
  } else {
    if (mb == 4)
      k_skinny_f32<IN, XF, OF, 4, 0><<<grid, 256, 0, st>>>(xp, wp, bp, op, mchunks, M, N, K, kchunk, ng, act, x2p,
                                                           g.k2, g.scale);
    else if (mb == 2)
      k_skinny_f32<IN, XF, OF, 2, 0><<<grid, 256, 0, st>>>(xp, wp, bp, op, mchunks, M, N, K, kchunk, ng, act, x2p,
                                                           g.k2, g.scale);
    else
      k_skinny_f32<IN, XF, OF, 1, 0><<<grid, 256, 0, st>>>(xp, wp, bp, op, mchunks, M, N, K, kchunk, ng, act, x2p,
                                                           g.k2, g.scale);
  }
}

hipError_t launch_skinny_f32(int mode, const SkinnyArgs& g, int chains, int M, int N, int K, int splits, int ng,
                             int act, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (chains < 1 || chains > 2) return hipErrorInvalidValue;
  const int mb = mblocks(M);
  const int kchunk = skinny_kchunk(K, splits);
  splits = (K + kchunk - 1) / kchunk;
  if (mode == kFragToFrag && splits != 1) return hipErrorInvalidValue;
  if (g.k2 < 0 || g.k2 % 16 != 0 || g.k2 >= K || (g.k2 > 0 && (mode == kRowsSilu || !g.x2[0])) ||
      (g.k2 > 0 && chains == 2 && !g.x2[1]) || (g.scale != 1.f && splits != 1))
    return hipErrorInvalidValue;
  const int mchunks = (M + 16 * mb - 1) / (16 * mb);
  dim3 grid((unsigned)((N / 16 + 3) / 4), (unsigned)splits, (unsigned)(chains * mchunks));
  if (mode == kFragToFrag)
    skinny_launch<kInPlain, 1, 1>(grid, mb, g, mchunks, M, N, K, kchunk, ng, act, st);
  else if (mode == kFragToRows)
    skinny_launch<kInPlain, 1, 0>(grid, mb, g, mchunks, M, N, K, kchunk, ng, act, st);
  else
    skinny_launch<kInSilu, 0, 0>(grid, mb, g, mchunks, M, N, K, kchunk, ng, act, st);
  return hipGetLastError();
}

hipError_t launch_sinusoid(const float* t0, const float* t1, float* s0, float* s1, int M, int F, float period,
                           hipStream_t st) {
  const long n = (long)padded_rows(M) * F / 4;
  if (n <= 0) return hipSuccess;
  const int chains = t1 ? 2 : 1;
  k_sinusoid<<<dim3((unsigned)((n + 255) / 256), (unsigned)chains), 256, 0, st>>>(
      Pair<const float*>{{t0, t1}}, Pair<float*>{{s0, s1}}, M, padded_rows(M), F, log2f(period));
  return hipGetLastError();
}

int skinny_splits(int K, int splits) {
  const int kchunk = skinny_kchunk(K, splits);
  return (K + kchunk - 1) / kchunk;
}

hipError_t launch_rows_finish(const float* part0, const float* part1, int splits, const float* bias0,
                              const float* bias1, float* out, int M, int N, int act, float gate, hipStream_t st) {
  const long n4 = (long)M * N / 4;
  if (n4 <= 0) return hipSuccess;
  k_rows_finish<<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, st>>>(
      Pair<const float*>{{part0, part1}}, Pair<const float*>{{bias0, bias1}}, part1 ? 2 : 1, splits, out, M, N, act,
      gate);
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
