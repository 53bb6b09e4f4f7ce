// Attention over one packed sequence with padding rows in their own
// document.
//
// Page "MiniMaxH3Transformer3DModel", class description: attention is full
// self-attention over the packed sequence (no cross-attention); a layout
// carrying padding rows (tag -1) keeps them in their own attention
// document via a boolean mask, and a padless sequence is one document. The
// batch axis replicates the layout and each item is its own document.
// Scale 1/sqrt(head_dim) unless the caller gives one (the page is silent).
//
// bf16 kernel (gfx950), flash-style with an fp32 online softmax:
//   * workgroup = 4 waves x 64 queries of one head; q stays in registers;
//   * K tiles [64 keys][128] and V^T tiles [128][64 keys] are staged in LDS
//     (2 stages, XOR-swizzled 16-byte chunks), the next tile's global loads
//     in flight while the current one is used;
//   * scores are computed transposed, S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16, so each lane owns one query column: the row
//     max needs one exchange between the two 32-lane halves and the running
//     max / sum / rescale are per-lane scalars. Key rows are fed to the MFMA
//     in an order (bits 2 and 3 of the row swapped) that makes the score
//     registers exactly the B operand of O^T += V^T P^T, so P never leaves
//     registers;
//   * exponentials in base 2 with scale*log2(e) folded into one FMA;
//   * document masks per 64-key tile (non-padding / padding bit masks built
//     once per call): tiles holding no key of a wave's documents are
//     skipped, fully-matching tiles need no per-element mask.
//   * workgroups are ordered so that the workgroups of one head run on the
//     same XCD and share its K/V stream in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace minih3 {

constexpr int kAttnQ = 256;  // queries per workgroup
constexpr int kKV = 64;      // keys per tile

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// key index inside a 32-key block held by accumulator register r of lane half hi
__device__ __forceinline__ int key_of_reg(int r, int hi) {
  const int i = r >> 2, j = r & 3;
  return 16 * (i >> 1) + 8 * hi + 4 * (i & 1) + j;
}

__global__ void __launch_bounds__(256, 1)
    k_attn_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ vt,
                bf16_t* __restrict__ out, const uint64_t* __restrict__ masks, const int32_t* __restrict__ list_real,
                const int32_t* __restrict__ list_pad, const int32_t* __restrict__ meta, int S, int H, int stride,
                float c_log2, int n_qt, int total) {
  constexpr int HD = 128;
  constexpr int KT_BYTES = kKV * HD * 2;     // 16 KiB
  constexpr int STAGE = 2 * KT_BYTES;        // K + V^T
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- workgroup -> (query tile, head, batch); XCD-contiguous order
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int pid = xcd * q8 + (xcd < r8 ? xcd : r8) + loc;
  const int qt = pid % n_qt;
  const int bh = pid / n_qt;  // b * H + h
  const int h = bh % H, b = bh / H;
  const long head_row = (long)bh * stride;  // row offset of (b,h) in [B,H,stride,hd]
  const int ntiles = stride / kKV;
  const int nt_real = (S + kKV - 1) / kKV;

  // ---- documents of this workgroup's and this wave's queries
  const int qw0 = qt * kAttnQ + wid * 64;  // first query of the wave
  bool wq_real = false, wq_pad = false;
  if (qw0 < S) {
    const int t = qw0 / kKV;
    wq_real = masks[2 * t] != 0;
    wq_pad = masks[2 * t + 1] != 0;
  }
  bool g_real = false, g_pad = false;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int qq = qt * kAttnQ + w * 64;
    if (qq < S) {
      g_real |= masks[2 * (qq / kKV)] != 0;
      g_pad |= masks[2 * (qq / kKV) + 1] != 0;
    }
  }
  const int* list = nullptr;
  int n_iter;
  if (g_real && g_pad) {
    n_iter = nt_real;  // every tile
  } else if (g_pad) {
    list = list_pad;
    n_iter = meta[1];
  } else {
    list = list_real;
    n_iter = meta[0];
  }

  // per-lane query documents (1 = padding row) for the two 32-query blocks
  int qdoc[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = qw0 + qb * 32 + l32;
    qdoc[qb] = 0;
    if (qr < S) qdoc[qb] = (int)((masks[2 * (qr / kKV) + 1] >> (qr % kKV)) & 1ull);
  }

  // ---- Q fragments (B operand of S^T = K Q^T): query column l32, dims 16kk + 8hi .. +8
  bf16x8 qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int qr = qw0 + qb * 32 + l32;
    qr = qr < stride ? qr : stride - 1;
    const bf16_t* src = q + (head_row + qr) * HD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[qb][kk] = *reinterpret_cast<const bf16x8*>(src + 16 * kk);
  }

  // ---- global -> LDS mapping
  // K tile: 64 rows x 16 chunks; thread owns chunk (tid & 15) of rows (tid >> 4) + 16 i
  // V^T tile: 128 rows x 8 chunks; thread owns chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int kc = tid & 15, kr0 = tid >> 4;
  const int vc = tid & 7, vr0 = tid >> 3;
  const bf16_t* kbase = k + head_row * HD + kr0 * HD + kc * 8;
  const bf16_t* vbase = vt + ((long)bh * HD + vr0) * stride + vc * 8;
  int k_st[4], v_st[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kr = kr0 + 16 * i;
    const int fk = (kr & 3) | (((kr >> 3) & 1) << 2);
    k_st[i] = kr * 256 + ((kc ^ fk) << 4);
    const int vr = vr0 + 32 * i;
    v_st[i] = KT_BYTES + vr * 128 + ((vc ^ (vr & 7)) << 4);
  }

  u32x4 rk[4], rv[4];
  auto tile_of = [&](int it) { return list ? list[it] : it; };
  auto gload = [&](int t) {
    const long key0 = (long)t * kKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk[i] = *reinterpret_cast<const u32x4*>(kbase + (key0 + 16 * i) * HD);
      rv[i] = *reinterpret_cast<const u32x4*>(vbase + (long)(32 * i) * stride + key0);
    }
    // values of keys >= S are zeroed so that masked keys contribute exactly 0
    if (key0 + kKV > S) {
      const int first = (int)(S - key0) - vc * 8;  // keys of this chunk below S
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e0 = 2 * w;
          uint32_t x = rv[i][w];
          if (e0 >= first) x &= 0xffff0000u;
          if (e0 + 1 >= first) x &= 0x0000ffffu;
          rv[i][w] = x;
        }
      }
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* base = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(base + k_st[i]) = rk[i];
      *reinterpret_cast<u32x4*>(base + v_st[i]) = rv[i];
    }
  };

  // fragment-read offsets
  // K (A operand of S^T): key row kb*32 + sigma(l32), chunk 2kk + hi
  const int krow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);  // bits 2 and 3 swapped
  const int kfk = (krow & 3) | (((krow >> 3) & 1) << 2);
  // V^T (A operand of O^T): row db*32 + l32, chunk kb*4 + cc*2 + hi
  const int vsw = l32 & 7;

  floatx16 o[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][qb][e] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  if (n_iter > 0) {
    gload(tile_of(0));
    lstore(0);
  }
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const int t = tile_of(it);
    const int stage = it & 1;
    if (it + 1 < n_iter) gload(tile_of(it + 1));

    const uint64_t mreal = masks[2 * t], mpad = masks[2 * t + 1];
    const bool need = (wq_real && mreal) || (wq_pad && mpad);
    if (need) {
      const uint8_t* Ks = lds + stage * STAGE;
      const uint8_t* Vs = Ks + KT_BYTES;
      // ---- S^T = K Q^T
      floatx16 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[kb][qb][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = kb * 32 + krow;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + row * 256 + (((2 * kk + hi) ^ kfk) << 4));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][kk], s[kb][qb], 0, 0, 0);
        }
      }
      // ---- document mask (skipped when the tile is entirely in the wave's only document)
      const bool full_real = wq_real && !wq_pad && mreal == ~0ull;
      const bool full_pad = wq_pad && !wq_real && mpad == ~0ull;
      if (!(full_real || full_pad)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const uint64_t msel = qdoc[qb] ? mpad : mreal;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb * 32 + key_of_reg(r, hi);
              if (!((msel >> key) & 1ull)) s[kb][qb][r] = -INFINITY;
            }
        }
      }
      // ---- online softmax (per lane = per query)
      bf16x8 pf[2][2][2];  // [kb][qb][cc]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[qb], mx * c_log2);
        const float base = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[qb] - base);
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            bf16x8 pv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p = fast_exp2(fmaf(s[kb][qb][8 * cc + e], c_log2, -base));
              ls += p;
              pv[e] = (__bf16)p;
            }
            pf[kb][qb][cc] = pv;
          }
        l_run[qb] = l_run[qb] * alpha + ls;
        m_run[qb] = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][qb][e] *= alpha;
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int row = db * 32 + l32;
            const int chunk = kb * 4 + cc * 2 + hi;
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vs + row * 128 + ((chunk ^ vsw) << 4));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][qb][cc], o[db][qb], 0, 0, 0);
          }
    }
    if (it + 1 < n_iter) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query l32 of block qb, dims db*32 + 8i + 4hi + j
  const int W = H * HD;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int qr = qw0 + qb * 32 + l32;
    if (qr >= S) continue;
    bf16_t* dst = out + ((long)b * S + qr) * W + h * HD + 4 * hi;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 pk;
        pk[0] = pack_bf16x2(o[db][qb][4 * i] * inv, o[db][qb][4 * i + 1] * inv);
        pk[1] = pack_bf16x2(o[db][qb][4 * i + 2] * inv, o[db][qb][4 * i + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + db * 32 + 8 * i) = pk;
      }
  }
}

// ---------------------------------------------------------------- fp32 kernel
// Plain kernel for fp32 storage (small workloads, parity): one thread per
// query, keys streamed through LDS 64 at a time, online softmax in fp32.
__global__ void __launch_bounds__(64) k_attn_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                 const float* __restrict__ vt, float* __restrict__ out,
                                                 const uint64_t* __restrict__ masks, int S, int H, int stride,
                                                 float scale) {
  constexpr int HD = 128;
  __shared__ float Ks[kKV][HD + 1];
  __shared__ float Vs[HD][kKV + 1];
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * H + h;
  const int qr = qt * 64 + threadIdx.x;
  const bool valid = qr < S;
  const int qc = valid ? qr : 0;
  const long head_row = (long)bh * stride;
  const int qdoc = (int)((masks[2 * (qc / kKV) + 1] >> (qc % kKV)) & 1ull);
  float qv[HD], ov[HD];
  for (int d = 0; d < HD; ++d) {
    qv[d] = q[(head_row + qc) * HD + d];
    ov[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int nt = (S + kKV - 1) / kKV;
  for (int t = 0; t < nt; ++t) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKV * HD; e += 64) {
      const int r = e / HD, d = e % HD;
      Ks[r][d] = k[(head_row + (long)t * kKV + r) * HD + d];
      const int d2 = e / kKV, r2 = e % kKV;
      Vs[d2][r2] = vt[((long)bh * HD + d2) * stride + (long)t * kKV + r2];
    }
    __syncthreads();
    const uint64_t msel = masks[2 * t + qdoc];
    for (int j = 0; j < kKV; ++j) {
      if (!((msel >> j) & 1ull)) continue;
      float sc = 0.f;
      for (int d = 0; d < HD; ++d) sc += qv[d] * Ks[j][d];
      sc *= scale;
      const float mn = fmaxf(m, sc);
      const float a = expf(m - mn), p = expf(sc - mn);
      l = l * a + p;
      for (int d = 0; d < HD; ++d) ov[d] = ov[d] * a + p * Vs[d][j];
      m = mn;
    }
  }
  if (valid) {
    float* dst = out + ((long)b * S + qr) * (H * HD) + h * HD;
    for (int d = 0; d < HD; ++d) dst[d] = ov[d] / l;
  }
}

template <>
hipError_t launch_attention<bf16_t>(const bf16_t* q, const bf16_t* k, const bf16_t* vt, bf16_t* out,
                                    const int32_t* tags, const uint64_t* masks, const int32_t* list_real,
                                    const int32_t* list_pad, const int32_t* meta, int B, int S, int H, int stride,
                                    float scale, int assume_padless, hipStream_t st) {
  (void)tags;
  (void)assume_padless;
  const int n_qt = (S + kAttnQ - 1) / kAttnQ;
  const int total = n_qt * H * B;
  const float c_log2 = scale * 1.4426950408889634f;
  k_attn_bf16<<<total, 256, 0, st>>>(q, k, vt, out, masks, list_real, list_pad, meta, S, H, stride, c_log2, n_qt,
                                      total);
  return hipGetLastError();
}

template <>
hipError_t launch_attention<float>(const float* q, const float* k, const float* vt, float* out, const int32_t* tags,
                                   const uint64_t* masks, const int32_t* list_real, const int32_t* list_pad,
                                   const int32_t* meta, int B, int S, int H, int stride, float scale,
                                   int assume_padless, hipStream_t st) {
  (void)tags;
  (void)list_real;
  (void)list_pad;
  (void)meta;
  (void)assume_padless;
  dim3 grid((unsigned)((S + 63) / 64), (unsigned)H, (unsigned)B);
  k_attn_f32<<<grid, 64, 0, st>>>(q, k, vt, out, masks, S, H, stride, scale);
  return hipGetLastError();
}

}  // namespace minih3
