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
//   kEpiStoreScaled: C = scale * acc
//   kEpiQKRope     : the QKV projection's tile leaves in the attention
//                    kernel's layouts: q and k per-head RMSNorm + rotary turn
//                    (with the key norms), v transposed
// The store epilogue also takes its A operand split in two arrays along K
// (EpiArgs::a2), so that [x | t] . [W | B]^T of an unmerged low-rank adapter
// needs no concatenated copy of its rows.
//
// bf16 kernel (gfx950): 256x256 output tile per workgroup of 4 waves, one per
// SIMD, each 128x128 as 8x8 v_mfma_f32_16x16x32_bf16 accumulators in AGPRs
// (on random data this shape does about an eighth more work per unit of
// power than 32x32x16, and the chip is power-limited under MFMA load).
// Operands reach LDS by direct buffer->LDS DMA in K steps of 64 through a
// ring of five 32 KiB slots (the A and W halves of a step are loaded at
// different times, see the kernel); fragments are read half a K step ahead.
// The issue order is fixed instruction group by instruction group
// (sched_barrier fences): one DMA instruction per eight MFMAs, so the four
// waves of a CU never queue a burst of DMA at the address unit.
// One barrier per K step. Tiles are ordered so that the workgroups an XCD
// runs together share A and W panels in its L2. Plain (store) tiles are
// staged in LDS and written as whole contiguous rows.
#include <mutex>

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

// q/k/v epilogue of the QKV projection. The staged bf16 tile (256 rows x 256
// columns: two heads of q, k or v) is read from LDS (row pitch RB bytes).
// Page "MiniMaxH3Transformer3DModel", Parameters (per-head query/key norms
// with qk_norm_eps; rotary frequencies on three axes). q and k: 16 lanes per
// row (both of its heads), 8 channels each, normalized and turned exactly as
// the standalone q/k pass does (same function, same table values); keys also
// give their norms from the stored bf16 values. v: a thread owns 8 rows x 8
// channels, transposed in registers, so that each channel leaves as 16
// contiguous bytes of its v^T row.
__device__ __forceinline__ void qkv_tile_epilogue(const uint8_t* lds, int RB, int m0, int n0, int M,
                                                  const EpiArgs& ea) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int H = ea.heads, Wd = H * 128, S = ea.S;
  const long stride = ea.stride;
  const int part = n0 / Wd;               // 0 q, 1 k, 2 v
  const int h0 = (n0 - part * Wd) / 128;  // the tile's first head
  if (part < 2) {
    // 16-lane group gi (of 16) owns rows gi + 16 k, k < 16, both heads of a
    // row (one set of table values); the table values and document words of
    // the next four rows are loaded while the current four are computed.
    const int cl = lane & 15, gi = wid * 4 + (lane >> 4);
    const float* gp = part == 0 ? ea.q_norm : ea.k_norm;
    bf16_t* out = static_cast<bf16_t*>(part == 0 ? ea.q_out : ea.k_out);
    const float2* rope = reinterpret_cast<const float2*>(ea.rope);
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = gp[cl * 8 + e];
    const int np = ea.rope_pairs;
    const bool norms = part == 1 && ea.kmax;
    const int b0 = m0 / S;  // batch item of the tile's first row
    // batch item and position of the lane's rows gi + 16 k, found by stepping
    // 16 rows at a time from the tile's first row (no division per row);
    // positions stay in [0, S) also for rows past M, which are never stored
    int bk[16], sk[16];
    {
      int b = b0, sp = m0 - b0 * S + gi;
      if (sp >= S) {
        b += sp / S;
        sp %= S;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        bk[k] = b;
        sk[k] = sp;
        sp += 16;
        if (sp >= S) {
          b += sp / S;
          sp %= S;
        }
      }
    }
    const long hstride = (long)stride * 128;  // elements between the rows of two heads
    float mx[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    constexpr int U = 4;
    struct Pre {
      float2 t[4];
      uint64_t mk;
    };
    auto fetch = [&](int k, Pre& p) {
      const int s = sk[k];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = cl * 4 + q;
        p.t[q] = j < np ? rope[(long)s * np + j] : make_float2(1.f, 0.f);
      }
      p.mk = norms ? ea.masks[2 * (s >> 6) + 1] : 0ull;
    };
    auto row = [&](int k, const Pre& p) {
      const int rr = gi + 16 * k, m = m0 + rr;
      if (m >= M) return;  // uniform over the 16 lanes of a row
      const int b = bk[k], s = sk[k];
      const int d = (int)((p.mk >> (s & 63)) & 1ull);
      bf16_t* orow = out + ((long)(b * H + h0) * stride + s) * 128 + cl * 8;
      float cs[4], sn[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cs[q] = p.t[q].x;
        sn[q] = p.t[q].y;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(lds + rr * RB + (hh * 128 + cl * 8) * 2);
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(raw[i] << 16);
          v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
        }
        qk_norm_rotate<8, 16>(v, g, cs, sn, ea.qk_eps);
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        *reinterpret_cast<u32x4*>(orow + hh * hstride) = o;
        if (norms) {
          float n2 = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x0 = __uint_as_float(o[i] << 16), x1 = __uint_as_float(o[i] & 0xffff0000u);
            n2 = __builtin_fmaf(x0, x0, n2);
            n2 = __builtin_fmaf(x1, x1, n2);
          }
          n2 = row_sum<16>(n2);
          if (b == b0) {
            const float c0 = fmaxf(mx[hh][0], n2), c1 = fmaxf(mx[hh][1], n2);
            mx[hh][0] = d ? mx[hh][0] : c0;
            mx[hh][1] = d ? c1 : mx[hh][1];
          } else if (cl == 0)  // rows of a second batch item in the tile: straight to memory
            atomicMax(reinterpret_cast<int*>(ea.kmax + 2 * ((long)b * H + h0 + hh) + d),
                      __float_as_int(sqrtf(n2)));
        }
      }
    };
    Pre cur[U], nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) fetch(u, cur[u]);
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += U) {
      if (k0 + U < 16)
#pragma unroll
        for (int u = 0; u < U; ++u) fetch(k0 + U + u, nxt[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) row(k0 + u, cur[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
    if (norms) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          float x = mx[hh][d];
          x = fmaxf(x, __shfl_xor(x, 16, 64));
          x = fmaxf(x, __shfl_xor(x, 32, 64));
          // non-negative floats order as ints
          if (lane == 0 && x > 0.f)
            atomicMax(reinterpret_cast<int*>(ea.kmax + 2 * ((long)b0 * H + h0 + hh) + d), __float_as_int(sqrtf(x)));
        }
    }
  } else {
    bf16_t* vt = static_cast<bf16_t*>(ea.vt_out);
    for (int blk = tid; blk < 1024; blk += 256) {
      const int r0 = (blk & 31) * 8, c0 = (blk >> 5) * 8;  // 8 rows x 8 channels of the tile
      u32x4 in[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) in[i] = *reinterpret_cast<const u32x4*>(lds + (r0 + i) * RB + c0 * 2);
      // out[e]: channel c0 + e of rows r0 .. r0 + 7
      u32x4 outv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = in[2 * w][e / 2], hi = in[2 * w + 1][e / 2];
          outv[e][w] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
      const int hh = c0 / 128, d0 = c0 % 128;
      const int mf = m0 + r0;
      const int b = mf / S, s = mf - b * S;
      if (mf + 7 < M && s + 7 < S && (s & 7) == 0) {
        bf16_t* dst = vt + (((long)b * H + h0 + hh) * 128 + d0) * stride + s;
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(dst + (long)e * stride) = outv[e];
      } else {
        for (int i = 0; i < 8; ++i) {
          const int m = mf + i;
          if (m >= M) break;
          const int bi = m / S, si = m - bi * S;
          bf16_t* dst = vt + (((long)bi * H + h0 + hh) * 128 + d0) * stride + si;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = outv[e][i / 2];
            reinterpret_cast<uint16_t*>(dst)[(long)e * stride] = (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA kernel

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kRowBytes = BK * 2;         // 128: one tile row of one K step
constexpr int kCPR = kRowBytes / 16;      // 16-byte chunks per row
constexpr int kSlotBytes = BM * kRowBytes;  // one operand (A or W) of one K step: 32 KiB
constexpr int kSlots = 5;                 // LDS ring: 160 KiB
constexpr int kWaves = 4;                 // one per SIMD, 128 x 128 outputs each
constexpr int kIPW = kSlotBytes / 1024 / kWaves;  // 1 KiB DMA instructions per wave per slot
static_assert(BM == BN, "A and W slots share a layout");

// Logical chunk c of tile row r sits at chunk c ^ swz(r): the 16 lanes a
// ds_read_b128 serves together read 16 consecutive rows at one chunk, and
// (r * kCPR + physical chunk) mod 16 -- the 16-byte bank group -- is then
// different for all 16.
__device__ __forceinline__ int gemm_swz(int r) { return (r / (16 / kCPR)) % kCPR; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS (buffer form):
// base wave-uniform, voff the lane's byte offset, soff a uniform byte offset.
// Lane L lands at dst + 16 L.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t soff, lds_ptr_t dst) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }


// 256 x 256 output tile per workgroup of four waves; wave (wm, wn) owns the
// 128 x 128 block at (128 wm, 128 wn) as 8 x 8 v_mfma_f32_16x16x32_bf16
// accumulators (256 AGPRs).
//
// K advances in steps of 64. The A and W operands of a step each fill one
// 32 KiB slot of a 5-slot LDS ring (slot of A_k: 2k mod 5, W_k: 2k + 1 mod
// 5), loaded by direct buffer->LDS DMA. Step k runs in two halves (K 32, 64
// MFMAs each) whose fragments are read one half ahead. The first half loads
// A_{k+2} (its slot held W_{k-1}); every wave then waits for its own DMA of
// step k + 1 and one barrier publishes it and frees A_k's and W_k's slots;
// the second half loads W_{k+2} into A_k's slot. A_k has about two K steps
// to arrive, W_k one.
//
// I8: the same kernel on int8 operands (v_mfma_i32_16x16x64_i8): a K step is
// 128 bytes of a row either way, so the LDS ring, the swizzle and the
// fragment reads are unchanged; a step covers 128 int8 columns instead of
// 64 bf16 ones. The int32 accumulators are turned into fp32
// acc * row_scale[m] * col_scale[W row] before the epilogue.
//
// SPLIT: the K steps below K - k2 read A (row stride K - k2), the others
// read ea.a2 (row stride k2); the LDS ring is filled the same way.
//
// HALF: the workgroup computes one 128-row half (bid & 1) of the 256 x 256
// tile pid_base + bid / 2 in the usual tile order: waves of 64 x 128
// outputs, the same K loop with 32 MFMAs per half step, A slots half
// filled. Every output is the same sequence of MFMAs over K as in a whole
// tile, so the values are bit for bit those of the whole-tile kernel.
template <int EPI, int I8, int SPLIT = 0, int HALF = 0>
__device__ __forceinline__ void gemm_body(const uint8_t* __restrict__ A, const uint8_t* __restrict__ W,
                                          void* __restrict__ Cv, int M, int N, int K, const EpiArgs& ea,
                                          int pid_base = 0) {
  static_assert(!HALF || (EPI == kEpiGatedResid && !SPLIT), "half tiles serve the gated-residual epilogue");
  constexpr int WTM = HALF ? 64 : 128, WTN = 128, MI = WTM / 16, NI = WTN / 16;
  constexpr int kIPWA = HALF ? kIPW / 2 : kIPW;  // DMA instructions of A per wave and K step
  constexpr int kEs = I8 ? 1 : 2;  // bytes per element
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kSlotBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid & 1, wn = wid >> 1;

  // ---- tile order: XCD-contiguous ranges, then groups of 4 M-tiles (an
  // XCD's 32 concurrent tiles are 4 M-tiles x 8 N-tiles; groups of 8 M-tiles
  // ran the QKV projection 3 % slower; groups of 2, 3, 6 and 16 were slower
  // too)
  const int MT = (M + BM - 1) / BM, NTL = N / BN;
  const int bid = blockIdx.x;
  int pid, mh = 0;
  if constexpr (HALF) {
    pid = pid_base + (bid >> 1);
    mh = bid & 1;
  } else {
    // the launch covers tiles 0 .. gridDim.x - 1 of the order
    const int G = gridDim.x;
    const int xcd = bid & 7, loc = bid >> 3;
    const int q8 = G >> 3, r8 = G & 7;
    pid = xcd * q8 + (xcd < r8 ? xcd : r8) + loc;
  }
  constexpr int GROUP_M = 4;
  const int npg = GROUP_M * NTL;
  const int g = pid / npg;
  const int first_m = g * GROUP_M;
  const int gsz = MT - first_m < GROUP_M ? MT - first_m : GROUP_M;
  const int tm = first_m + (pid % npg) % gsz;
  const int tn = (pid % npg) / gsz;
  const int m0 = tm * BM + mh * (BM / 2);

  // ---- DMA byte offsets. Wave w fills rows 64 w .. 64 w + 63 of every slot
  // (of an A slot of a half tile rows 32 w .. 32 w + 31): instruction j covers
  // rows 64 w + 8 j .. + 7 (1 KiB); lane L takes row 64 w + 8 j + L / 8,
  // logical chunk (L % 8) ^ swz(row).
  const int K1 = SPLIT ? K - ea.k2 : K;  // row stride of A
  const uint8_t* A2 = static_cast<const uint8_t*>(ea.a2);
  uint32_t voff_a[kIPWA], voff_w[kIPW], voff_a2[SPLIT ? kIPW : 1];
#pragma unroll
  for (int j = 0; j < kIPWA; ++j) {
    const int row = (HALF ? 32 : 64) * wid + 8 * j + lane / kCPR;
    const int c = (lane % kCPR) ^ gemm_swz(row);
    int am = m0 + row;
    am = am < M ? am : M - 1;
    voff_a[j] = (uint32_t)((long)am * K1 * kEs + c * 16);
    if constexpr (SPLIT) voff_a2[j] = (uint32_t)((long)am * ea.k2 * kEs + c * 16);
  }
#pragma unroll
  for (int j = 0; j < kIPW; ++j) {
    const int row = 64 * wid + 8 * j + lane / kCPR;
    const int c = (lane % kCPR) ^ gemm_swz(row);
    int wr;
    if (EPI == kEpiSwiGLU) {
      // wave block of WTN rows: first half gate rows, second half the matching up rows
      const int wblk = row / WTN, sel = (row % WTN) / (WTN / 2), o = row % (WTN / 2);
      wr = sel * ea.ffn_dim + 128 * tn + (WTN / 2) * wblk + o;
    } else {
      wr = tn * BN + row;
    }
    voff_w[j] = (uint32_t)((long)wr * K * kEs + c * 16);
  }
  const int KT = K / (kRowBytes / kEs);
  const int KT1 = K1 / (kRowBytes / kEs);  // K steps served by A
  auto slot_ptr = [&](int s) { return lds + s * kSlotBytes; };
  // DMA instruction j of operand A (or W) of K step k into its ring slot;
  // past the end of K the last step is loaded again (the slot is free).
  auto dma_a1 = [&](int k, int j) {
    const int s = (2 * k) % kSlots;
    const int kc = k < KT ? k : KT - 1;
    if constexpr (SPLIT) {
      const bool second = kc >= KT1;
      dma16(second ? A2 : A, second ? voff_a2[j] : voff_a[j], (uint32_t)((second ? kc - KT1 : kc) * kRowBytes),
            (lds_ptr_t)(slot_ptr(s) + (64 * wid + 8 * j) * kRowBytes));
    } else {
      dma16(A, voff_a[j], (uint32_t)(kc * kRowBytes),
            (lds_ptr_t)(slot_ptr(s) + ((HALF ? 32 : 64) * wid + 8 * j) * kRowBytes));
    }
  };
  auto dma_w1 = [&](int k, int j) {
    const int s = (2 * k + 1) % kSlots;
    const uint32_t soff = (uint32_t)((k < KT ? k : KT - 1) * kRowBytes);
    dma16(W, voff_w[j], soff, (lds_ptr_t)(slot_ptr(s) + (64 * wid + 8 * j) * kRowBytes));
  };

  floatx4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  // fragment reads (16x16x32 operands): row (lane & 15) of a 16-row block,
  // 16-byte chunk 4 h + (lane >> 4) of half h of the K step
  const int fr_row = lane & 15, fr_q = lane >> 4, fr_sw = gemm_swz(fr_row);
  bf16x8 fa[2][MI], fw[2][NI];
  // A half step's reads come from two lane addresses, the A and the W slot of
  // its K step plus the lane's row and chunk, formed once before the half's
  // MFMA stream (and pinned there), so that the reads inside the stream only
  // add immediates: VALU work between the MFMAs slows them (address
  // arithmetic per read cost ~3 % on every projection).
  typedef __attribute__((address_space(3))) const bf16x8* lds_frag_t;
  typedef __attribute__((address_space(3))) const uint8_t* lds_u8_t;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8_t)lds;
  uint32_t la[2], lw[2];  // the lane's byte offset in an A / W slot, half h
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int chunk = ((4 * h + fr_q) ^ fr_sw) << 4;
    la[h] = (uint32_t)((wm * WTM + fr_row) * kRowBytes + chunk);
    lw[h] = (uint32_t)((wn * WTN + fr_row) * kRowBytes + chunk);
  }
  auto frag_base = [&](int k, int h, uint32_t& aA, uint32_t& aW) {
    aA = lds0 + (uint32_t)(((2 * k) % kSlots) * kSlotBytes) + la[h];
    aW = lds0 + (uint32_t)(((2 * k + 1) % kSlots) * kSlotBytes) + lw[h];
    asm volatile("" : "+v"(aA), "+v"(aW));
  };
  // fragment r (0..MI + NI - 1) of the half step whose addresses are aA, aW
  // into register set `set`, in the order the MFMAs first use them:
  // a0 w0..w7 a1..a(MI-1)
  auto read_frag = [&](uint32_t aA, uint32_t aW, int set, int r) {
    if (r >= 1 && r <= NI) {
      fw[set][r - 1] = *(lds_frag_t)(uintptr_t)(aW + (uint32_t)((r - 1) * 16 * kRowBytes));
    } else {
      const int mi = r == 0 ? 0 : r - NI;
      fa[set][mi] = *(lds_frag_t)(uintptr_t)(aA + (uint32_t)(mi * 16 * kRowBytes));
    }
  };
  // C[m][n] for m = row (lane & 15) of block mi, n = 4 (lane >> 4) + e of
  // block ni: the W fragment is the MFMA's A operand, the A fragment its B.
  // Written as an in-place instruction: with the builtin the compiler moves the
  // 4-register accumulators between AGPRs on every K step. The compiler does
  // not see this as an MFMA, so the wait states around the accumulators are
  // explicit (fence_acc, after the zeroing and after the loop); fragment
  // registers are rewritten no sooner than 12 MFMAs after their last use.
  auto mfma1 = [&](int set, int i) {
    const int mi = i / NI, ni = i % NI;
    if constexpr (I8)
      asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[mi][ni]) : "v"(fw[set][ni]), "v"(fa[set][mi]));
    else
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[mi][ni]) : "v"(fw[set][ni]), "v"(fa[set][mi]));
  };
  // Fragment read issued after MFMA i of a half step (-1: none). Whole tile:
  // after every fourth MFMA, in read_frag's order. Half tile (12 fragments
  // over 32 MFMAs): placed so that a register is rewritten no sooner than 12
  // MFMAs after its last use in the previous half step (W fragment ni after
  // MFMA 4 + ni or later) and arrives well before its first use.
  auto read_at = [](int i) {
    if constexpr (HALF) {
      switch (i) {
        case 0: return 0;    // a0
        case 2: return 9;    // a1
        case 5: return 1;    // w0
        case 7: return 2;    // w1
        case 9: return 3;    // w2
        case 11: return 4;   // w3
        case 14: return 10;  // a2
        case 16: return 5;   // w4
        case 18: return 6;   // w5
        case 20: return 7;   // w6
        case 22: return 8;   // w7
        case 25: return 11;  // a3
        default: return -1;
      }
    } else {
      return (i & 3) == 0 ? i >> 2 : -1;
    }
  };
  // One half K step (MI * NI MFMAs) in a fixed issue order: MFMA i, then
  // the fragment read_at(i) of the next half, and DMA instructions of (dk, W
  // or A) spread evenly (eight per half step; the four of a half tile's A
  // after every eighth MFMA); each group is fenced so the DMA of the four
  // waves reaches the address unit evenly.
  auto half = [&](int set, int nk, int nh, bool reads, int dk, bool dw) {
    constexpr int NM = MI * NI;
    uint32_t aA = 0, aW = 0;
    if (reads) frag_base(nk, nh, aA, aW);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      mfma1(set, i);
      if (reads && read_at(i) >= 0) read_frag(aA, aW, set ^ 1, read_at(i));
      if (dk >= 0) {
        if (dw) {
          if (i % (NM / kIPW) == NM / kIPW - 1) dma_w1(dk, i / (NM / kIPW));
        } else {
          if (i % (NM / kIPWA) == NM / kIPWA - 1) dma_a1(dk, i / (NM / kIPWA));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  static_assert(kIPW == 8 && MI * NI == (HALF ? 32 : 64), "eight W DMA instructions per half K step");

  // The accumulators pass through these statements (which the compiler cannot
  // move them across): the first gives the zeroing its wait states before any
  // MFMA reads an accumulator; after the loop the same gives the last MFMAs
  // theirs before the epilogue reads them.
  auto fence_acc = [&](bool after_mfma) {
    if (after_mfma)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]),
                   "+a"(acc[0][3]), "+a"(acc[0][4]), "+a"(acc[0][5]), "+a"(acc[0][6]), "+a"(acc[0][7]));
    else
      asm volatile("s_nop 1" : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                   "+a"(acc[0][4]), "+a"(acc[0][5]), "+a"(acc[0][6]), "+a"(acc[0][7]));
#pragma unroll
    for (int mi = 1; mi < MI; ++mi)
      asm volatile("" : "+a"(acc[mi][0]), "+a"(acc[mi][1]), "+a"(acc[mi][2]), "+a"(acc[mi][3]), "+a"(acc[mi][4]),
                   "+a"(acc[mi][5]), "+a"(acc[mi][6]), "+a"(acc[mi][7]));
  };
  static_assert(NI == 8, "eight accumulators per fence statement");

  // ---- prologue: A0 W0 A1 W1 in flight, wait for step 0
  fence_acc(false);
#pragma unroll
  for (int j = 0; j < kIPWA; ++j) dma_a1(0, j);
#pragma unroll
  for (int j = 0; j < kIPW; ++j) dma_w1(0, j);
#pragma unroll
  for (int j = 0; j < kIPWA; ++j) dma_a1(1, j);
#pragma unroll
  for (int j = 0; j < kIPW; ++j) dma_w1(1, j);
  wait_vmcnt<kIPWA + kIPW>();
  __builtin_amdgcn_s_barrier();
  {
    uint32_t aA, aW;
    frag_base(0, 0, aA, aW);
#pragma unroll
    for (int r = 0; r < MI + NI; ++r) read_frag(aA, aW, 0, r);
  }

  // K step kt: its first half loads A_{kt+2} (the slot of W_{kt-1}) and reads
  // the second half's fragments; every wave then waits for its own DMA of
  // step kt + 1 and one barrier publishes it and frees the slots of A_kt and
  // W_kt; the second half loads W_{kt+2} into A_kt's slot and reads the first
  // fragments of step kt + 1.
  // The last step runs the same code: its DMA (clamped to step KT - 1) goes
  // to freed slots and the fragments it reads for a step KT are never used,
  // so the accumulators leave the loop in place (no copies after it).
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_sched_barrier(0);
    half(0, kt, 1, true, kt + 2, false);
    wait_vmcnt<kIPWA>();  // A_{kt+1}, W_{kt+1} landed; A_{kt+2} may be in flight
    wait_lgkm0();        // this wave's reads of step kt are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    half(1, kt + 1, 0, true, kt + 2, true);
  }
  __builtin_amdgcn_sched_barrier(0);
  fence_acc(true);
  wait_vmcnt<0>();  // no DMA may still write LDS when the workgroup ends

  // ---- epilogue. A lane's accumulators hold row m = tile row
  // (wm*128 + mi*16 + (lane & 15)), columns wn*128 + ni*16 + 4*(lane>>4) + e.
  // Accumulator block (mi, ni) as fp32; with int8 operands the int32 sums
  // times the row's scale and the scale of the W row each column came from.
  auto deq = [&](int mi, int ni) -> floatx4 {
    if constexpr (I8) {
      int m = m0 + wm * WTM + mi * 16 + fr_row;
      m = m < M ? m : M - 1;
      int wrow;
      if constexpr (EPI == kEpiSwiGLU)
        wrow = (ni < NI / 2 ? 0 : ea.ffn_dim) + 128 * tn + (WTN / 2) * wn + (ni % (NI / 2)) * 16 + 4 * fr_q;
      else
        wrow = tn * BN + wn * WTN + ni * 16 + 4 * fr_q;
      const float rs = ea.row_scale[m];
      const floatx4 cs = *reinterpret_cast<const floatx4*>(ea.col_scale + wrow);
      const intx4 ai = __builtin_bit_cast(intx4, acc[mi][ni]);
      floatx4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (float)ai[e] * rs * cs[e];
      return r;
    } else {
      return acc[mi][ni];
    }
  };
  if constexpr (EPI == kEpiGatedResid) {
    // gated residual straight from the accumulators (staging through LDS
    // measured slower, as did staging the SwiGLU output). Per lane row: its
    // table row once, then all eight residual and gate loads before any
    // store, with the storage types fixed outside the loops; a padding row
    // takes gate 0, which leaves its residual bit for bit.
    auto gated = [&](auto resid_tag, auto out_tag) {
      using TR = decltype(resid_tag);
      using TO = decltype(out_tag);
      const TR* resid = static_cast<const TR*>(ea.resid);
      TO* out = static_cast<TO*>(Cv);
      int trs[MI];  // table rows of the lane's rows, loaded together
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        int m = m0 + wm * WTM + mi * 16 + fr_row;
        m = m < M ? m : M - 1;
        const int s = m % ea.S;
        trs[mi] = table_row_of(ea.tags[s], ea.tidx[s], ea.num_tags, ea.num_tvals);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int m = m0 + wm * WTM + mi * 16 + fr_row;
        if (m >= M) continue;
        const int tr = trs[mi];
        const float* grow = ea.table + ((long)(tr >= 0 ? tr : 0) * 6 + ea.gate_slot) * N;
        float r[NI][4];
        floatx4 g[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = tn * BN + wn * WTN + ni * 16 + 4 * fr_q;
          load4<TR>(resid + (long)m * N + n, r[ni]);
          g[ni] = *reinterpret_cast<const floatx4*>(grow + n);
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = tn * BN + wn * WTN + ni * 16 + 4 * fr_q;
          const floatx4 a = deq(mi, ni);
#pragma unroll
          for (int e = 0; e < 4; ++e) r[ni][e] += (tr >= 0 ? g[ni][e] : 0.f) * a[e];
          store4<TO>(out + (long)m * N + n, r[ni]);
        }
      }
    };
    if (ea.resid_f32) {
      if (ea.out_f32)
        gated(float{}, float{});
      else
        gated(float{}, bf16_t{});
    } else {
      if (ea.out_f32)
        gated(bf16_t{}, float{});
      else
        gated(bf16_t{}, bf16_t{});
    }
  } else if constexpr (EPI == kEpiSwiGLU) {
    // silu(gate) * up straight from the accumulators (gate block ni, up block ni + NI/2)
    const int F = ea.ffn_dim;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int m = m0 + wm * WTM + mi * 16 + fr_row;
      if (m >= M) continue;
#pragma unroll
      for (int ni = 0; ni < NI / 2; ++ni) {
        float v[4];
        const floatx4 g = deq(mi, ni), u = deq(mi, ni + NI / 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = silu(g[e]) * u[e];
        const int f = 128 * tn + (WTN / 2) * wn + ni * 16 + 4 * fr_q;
        store4<bf16_t>(static_cast<bf16_t*>(Cv) + (long)m * F + f, v);
      }
    }
  } else {
    // bf16 staging: 256 rows x 256 columns, rows padded by 8 bytes so that the
    // 16 rows an 8-byte ds_write covers hit different bank pairs
    constexpr int RB = BN * 2 + 8;
    __syncthreads();  // every wave is done reading the ring
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int r = wm * WTM + mi * 16 + fr_row, c = wn * WTN + ni * 16 + 4 * fr_q;
        u32x2 pk;
        floatx4 a = deq(mi, ni);
        if constexpr (EPI == kEpiStoreScaled) {
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] *= ea.scale;
        }
        pk[0] = pack_bf16x2(a[0], a[1]);
        pk[1] = pack_bf16x2(a[2], a[3]);
        *reinterpret_cast<u32x2*>(lds + r * RB + c * 2) = pk;
      }
    __syncthreads();
    if constexpr (EPI == kEpiQKRope) {
      qkv_tile_epilogue(lds, RB, m0, tn * BN, M, ea);
    } else {
      // one row (512 bytes) per wave instruction: lane owns columns 4*lane .. +3
      for (int rr = wid; rr < BM; rr += kWaves) {
        const int m = m0 + rr;
        if (m < M)
          *reinterpret_cast<u32x2*>(static_cast<bf16_t*>(Cv) + (long)m * N + tn * BN + 4 * lane) =
              *reinterpret_cast<const u32x2*>(lds + rr * RB + lane * 8);
      }
    }
  }
}

template <int EPI>
__global__ void __launch_bounds__(64 * kWaves, 1)
    k_gemm_bf16(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, void* __restrict__ Cv, int M, int N,
                int K, EpiArgs ea) {
  gemm_body<EPI, 0>(reinterpret_cast<const uint8_t*>(A), reinterpret_cast<const uint8_t*>(W), Cv, M, N, K, ea);
}

template <int EPI>
__global__ void __launch_bounds__(64 * kWaves, 1)
    k_gemm_bf16_split(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, void* __restrict__ Cv, int M, int N,
                      int K, EpiArgs ea) {
  gemm_body<EPI, 0, 1>(reinterpret_cast<const uint8_t*>(A), reinterpret_cast<const uint8_t*>(W), Cv, M, N, K, ea);
}

// The last, partial wave of tiles as half tiles (see gemm_body).
template <int EPI>
__global__ void __launch_bounds__(64 * kWaves, 1)
    k_gemm_bf16_half(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, void* __restrict__ Cv, int M,
                     int N, int K, EpiArgs ea, int pid_base) {
  gemm_body<EPI, 0, 0, 1>(reinterpret_cast<const uint8_t*>(A), reinterpret_cast<const uint8_t*>(W), Cv, M, N, K, ea,
                          pid_base);
}

template <int EPI>
__global__ void __launch_bounds__(64 * kWaves, 1)
    k_gemm_i8(const int8_t* __restrict__ A, const int8_t* __restrict__ W, void* __restrict__ Cv, int M, int N, int K,
              EpiArgs ea) {
  gemm_body<EPI, 1>(reinterpret_cast<const uint8_t*>(A), reinterpret_cast<const uint8_t*>(W), Cv, M, N, K, ea);
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
  const float* A2 = static_cast<const float*>(ea.a2);
  const int K1 = A2 ? K - ea.k2 : K;  // row stride of A
  float acc[NB][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int e = tid; e < TM * TK; e += 256) {
      const int r = e / TK, c = e % TK;
      const int m = m0 + r < M ? m0 + r : M - 1;
      const int kk = k0 + c;
      As[c][r] = kk < K1 ? A[(long)m * K1 + kk] : A2[(long)m * ea.k2 + (kk - K1)];
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
    if (EPI == kEpiStoreScaled)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] *= ea.scale;
    if (EPI == kEpiGatedResid)
      epi_gated<float>(C, ldc, m, n, v, ea);
    else
      store4<float>(C + (long)m * ldc + n, v);
  }
}

// ---------------------------------------------------------------- launchers

// Compute units of the current device (cached per device; 0 on error).
static int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// Shapes the q/k/v epilogue assumes: N = 3 heads 128 with an even head count
// (a 256-column tile holds two heads of one of q, k, v), M whole batch items,
// stride a multiple of 64 not below S, at most 64 rotation pairs.
static bool qk_epi_ok(int M, int N, const EpiArgs& ea) {
  return ea.heads > 0 && ea.heads % 2 == 0 && N == 3 * ea.heads * 128 && ea.S > 0 && M % ea.S == 0 &&
         ea.stride >= ea.S && ea.stride % 64 == 0 && (ea.rope || ea.rope_pairs == 0) && ea.rope_pairs >= 0 &&
         ea.rope_pairs <= 64 && ea.q_out && ea.k_out && ea.vt_out && ea.q_norm && ea.k_norm &&
         (!ea.kmax || ea.masks);
}

template <>
hipError_t launch_gemm<bf16_t>(int epi, const bf16_t* A, const bf16_t* W, void* C, int M, int N, int K,
                               const EpiArgs& ea, hipStream_t st) {
  if (M <= 0 || N % BN != 0 || K % BK != 0) return hipErrorInvalidValue;
  if (epi == kEpiSwiGLU && (N != 2 * ea.ffn_dim || ea.ffn_dim % 128 != 0)) return hipErrorInvalidValue;
  if (epi == kEpiQKRope && !qk_epi_ok(M, N, ea)) return hipErrorInvalidValue;
  // DMA offsets are 32-bit byte offsets into A and W
  if ((unsigned long)M * K * 2 > 0xFFFFFFFFul || (unsigned long)N * K * 2 > 0xFFFFFFFFul) return hipErrorInvalidValue;
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  dim3 grid((unsigned)tiles);
  if (ea.a2) {  // split A operand [A | a2]: both parts whole K steps, any epilogue
    if (ea.k2 <= 0 || ea.k2 >= K || ea.k2 % BK != 0) return hipErrorInvalidValue;
    if ((unsigned long)M * ea.k2 * 2 > 0xFFFFFFFFul) return hipErrorInvalidValue;
    switch (epi) {
      case kEpiStore: k_gemm_bf16_split<kEpiStore><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
      case kEpiQKRope: k_gemm_bf16_split<kEpiQKRope><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
      case kEpiGatedResid:
        k_gemm_bf16_split<kEpiGatedResid><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea);
        break;
      case kEpiSwiGLU: k_gemm_bf16_split<kEpiSwiGLU><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (epi == kEpiGatedResid) {
    // One workgroup per CU: when the tiles end in a wave that fills at most
    // half the CUs, the whole waves run as usual and the rest as half tiles
    // (one wave of at most all CUs, each with half the work).
    const int cus = device_cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int whole = tiles / cus * cus, rest = tiles - whole;
    if (whole > 0 && rest > 0 && 2 * rest <= cus) {
      k_gemm_bf16<kEpiGatedResid><<<dim3((unsigned)whole), 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea);
      k_gemm_bf16_half<kEpiGatedResid><<<dim3((unsigned)(2 * rest)), 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea,
                                                                                          whole);
      return hipGetLastError();
    }
  }
  switch (epi) {
    case kEpiStore: k_gemm_bf16<kEpiStore><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiStoreScaled: k_gemm_bf16<kEpiStoreScaled><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiQKRope: k_gemm_bf16<kEpiQKRope><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiGatedResid: k_gemm_bf16<kEpiGatedResid><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiSwiGLU: k_gemm_bf16<kEpiSwiGLU><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_i8(int epi, const int8_t* A, const int8_t* W, void* C, int M, int N, int K, const EpiArgs& ea,
                          hipStream_t st) {
  if (M <= 0 || N % BN != 0 || K % 128 != 0 || !ea.row_scale || !ea.col_scale || ea.a2) return hipErrorInvalidValue;
  if (epi == kEpiSwiGLU && (N != 2 * ea.ffn_dim || ea.ffn_dim % 128 != 0)) return hipErrorInvalidValue;
  if (epi == kEpiQKRope && !qk_epi_ok(M, N, ea)) return hipErrorInvalidValue;
  if ((unsigned long)M * K > 0xFFFFFFFFul || (unsigned long)N * K > 0xFFFFFFFFul) return hipErrorInvalidValue;
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  dim3 grid((unsigned)tiles);
  switch (epi) {
    case kEpiStore: k_gemm_i8<kEpiStore><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiQKRope: k_gemm_i8<kEpiQKRope><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiGatedResid: k_gemm_i8<kEpiGatedResid><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiSwiGLU: k_gemm_i8<kEpiSwiGLU><<<grid, 64 * kWaves, 0, st>>>(A, W, C, M, N, K, ea); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <>
hipError_t launch_gemm<float>(int epi, const float* A, const float* W, void* Cv, int M, int N, int K,
                              const EpiArgs& ea, hipStream_t st) {
  if (M <= 0 || N % 64 != 0 || K % 16 != 0) return hipErrorInvalidValue;
  float* C = static_cast<float*>(Cv);
  const int ncols = epi == kEpiSwiGLU ? ea.ffn_dim : N;
  if (epi == kEpiSwiGLU && (N != 2 * ea.ffn_dim || ea.ffn_dim % 64 != 0)) return hipErrorInvalidValue;
  if (ea.a2 && (ea.k2 <= 0 || ea.k2 >= K || ea.k2 % 16 != 0)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(ncols / 64), (unsigned)((M + 63) / 64));
  switch (epi) {
    case kEpiStore: k_gemm_f32<kEpiStore><<<grid, 256, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiStoreScaled: k_gemm_f32<kEpiStoreScaled><<<grid, 256, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiGatedResid: k_gemm_f32<kEpiGatedResid><<<grid, 256, 0, st>>>(A, W, C, M, N, K, ea); break;
    case kEpiSwiGLU: k_gemm_f32<kEpiSwiGLU><<<grid, 256, 0, st>>>(A, W, C, M, N, K, ea); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace minih3
