// Host-side launchers of the gfx950 kernels (internal to libminih3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace minih3 {

enum ErrBits : uint32_t {
  kErrTag = 1u, kErrTval = 2u, kErrIndex = 4u, kErrPad = 8u, kErrNeedsMask = 16u
};

struct LayoutDev {
  int S;
  const int32_t* tags;
  const int32_t* tidx;
  const int32_t* pos;
  const int32_t* idx[3];  // video, audio, text
  int n_idx[3];
  int want_tag[3];
  int num_tags, num_tvals;
};

// ---- layout (integer) ----
// Scratch: counts[S] int32, err[1] u32, npad[1] int32. Writes the optional
// per-row / per-tile outputs when non-null.
hipError_t launch_layout_validate(const LayoutDev& L, int assume_padless, int32_t* counts, uint32_t* err,
                                  int32_t* npad, int32_t* table_row, int32_t* doc_id, int32_t* tile_flags,
                                  hipStream_t st);
// Attention tile lists: for each 64-row tile the masks of its non-padding
// and padding rows (u64 each), and the compacted lists of tiles holding
// any non-padding / padding row. meta[0] = #real tiles, meta[1] = #pad tiles.
// masks holds 6 * ceil(S/64) u64: [2t, 2t+1] the masks of tile t, then at
// 2 ntiles + 2i (4 ntiles + 2i) the masks of tile list_real[i] (list_pad[i]).
hipError_t launch_attn_tiles(const int32_t* tags, int S, int assume_padless, uint64_t* masks, int32_t* list_real,
                             int32_t* list_pad, int32_t* meta, hipStream_t st);

// ---- AdaLN ----
template <typename T>
hipError_t launch_adaln(const void* x, bool x_f32, T* y, const float* table, const int32_t* tags,
                        const int32_t* tidx, int B, int S, int D, int which, float eps, int num_tags, int num_tvals,
                        hipStream_t st);  // x: [B*S, D] fp32 if x_f32 else T
template <typename T>
hipError_t launch_cast_f32(const float* x, T* y, long n, hipStream_t st);

// ---- q/k RMSNorm + RoPE + V transpose ----
template <typename T>
hipError_t launch_qk_norm_rope(const T* qkv, const float* gq, const float* gk, const int32_t* pos, T* qo, T* ko,
                               T* vto, int B, int S, int H, int stride, int fd, float theta, float eps,
                               hipStream_t st, const uint64_t* masks = nullptr, float* kmax = nullptr);
// kmax (bf16 only; zeroed by the caller): per (b, h) and document the largest
// |k| of the stored keys, as launch_attention_prep computes it; masks are the
// tile masks of launch_attn_tiles.
hipError_t launch_zero_f32(float* p, int n, hipStream_t st);

// ---- GEMM: C[M,N] = A[M,K] . W[N,K]^T with fused epilogues ----
enum Epi { kEpiStore = 0, kEpiGatedResid = 1, kEpiSwiGLU = 2, kEpiStoreScaled = 3, kEpiQKRope = 4 };
struct EpiArgs {
  const void* resid;     // [M, ldc] gated residual: fp32 if resid_f32 else act
  int resid_f32, out_f32;  // bf16 kernel only: precision of resid and of C (gated residual)
  const float* table;    // adaln table
  const int32_t* tags;   // [S]
  const int32_t* tidx;   // [S]
  int S;                 // rows per batch item (row -> layout row = m % S)
  int num_tags, num_tvals;
  int gate_slot;         // 2 (attention gate) or 5 (FFN gate)
  int ffn_dim;           // SwiGLU: F (W rows [0,F) gate, [F,2F) up)
  const float* row_scale;  // int8 kernel: per A row
  const float* col_scale;  // int8 kernel: per W row
  float scale;           // kEpiStoreScaled: C = scale * acc
  // Split A operand (store epilogue, bf16 and fp32): columns [0, K - k2) of
  // A come from A itself (row stride K - k2), columns [K - k2, K) from a2
  // (row stride k2); null a2: A is one [M, K] array. bf16: K - k2 and k2
  // multiples of 64.
  const void* a2;
  int k2;
  // kEpiQKRope (bf16 kernel, N = 3 heads 128, heads even): the QKV tile (two
  // heads of q, k or v) leaves in the attention layouts: q and k per-head
  // RMS-normalized with q_norm / k_norm and turned by the rope table, as
  // [B, heads, stride, 128]; v transposed, [B, heads, 128, stride]. With kmax
  // (zero on entry) the largest |k| of the stored keys per (b, head) and
  // document (masks: [2t] real rows, [2t + 1] padding rows of 64-row tile t)
  // is recorded at kmax[2 (b heads + h) + doc].
  void *q_out, *k_out, *vt_out;
  const float *q_norm, *k_norm;
  const float* rope;  // [S, rope_pairs] (cos, sin), from launch_rope_table
  int rope_pairs, heads, stride;
  float qk_eps;
  float* kmax;
  const uint64_t* masks;
};
// int8 operands (K % 128 == 0), int32 accumulation, dequantized with
// ea.row_scale[m] * ea.col_scale[W row] ahead of the epilogue (store,
// gated residual or SwiGLU, as with bf16 operands).
hipError_t launch_gemm_i8(int epi, const int8_t* A, const int8_t* W, void* C, int M, int N, int K, const EpiArgs& ea,
                          hipStream_t st);
template <typename T>
hipError_t launch_gemm(int epi, const T* A, const T* W, void* C, int M, int N, int K, const EpiArgs& ea,
                       hipStream_t st);

// ---- attention ----
// scratch: attention_scratch_bytes(B, S, H) bytes (per-head key-norm maxima
// and per-workgroup flags).
size_t attention_scratch_bytes(int B, int S, int H);
// Packed q, k, v [B, S, H, 128] -> the attention kernels' layouts: q, k
// head-major [B, H, stride, 128], v transposed [B, H, 128, stride]; rows
// [S, stride) are written as zeros. stride is a multiple of 64, >= S.
template <typename T>
hipError_t launch_attn_stage(const T* q, const T* k, const T* v, T* qh, T* kh, T* vt, int B, int S, int H, int stride,
                             hipStream_t st);
// Per-document key-norm maxima into scratch (runs before launch_attention).
template <typename T>
hipError_t launch_attention_prep(const T* k, const uint64_t* masks, void* scratch, int B, int S, int H, int stride,
                                 hipStream_t st);
template <typename T>
hipError_t launch_attention(const T* q, const T* k, const T* vt, T* out, const uint64_t* masks,
                            const int32_t* list_real, const int32_t* list_pad, const int32_t* meta, void* scratch,
                            int B, int S, int H, int stride, float scale, hipStream_t st);

// ---- timestep conditioning (AdaLN table build) ----
enum InMode { kInPlain = 0, kInSilu = 1 };
// Row count of the padded conditioning operands: M rounded up to the row
// chunk a launch column covers (16, 32 or 64 rows).
int padded_rows(int M);
// Fragment order of an fp32 [Mpad, K] operand: the 16-byte unit
// (mb * (K / 16) + st) * 64 + lane, lane = r16 + 16 q, holds row 16 mb + r16,
// columns 16 st + 4q .. +3 (an MFMA 16x16x4 operand / accumulator block).
// s = [cos(t f_c), sin(t f_c)] over F columns, f_c = period^(-c / (F/2)),
// in fragment order with padded_rows(M) rows (zero past M); F % 32 == 0.
// With t1 non-null, s1 gets the embedding of t1 in the same launch.
hipError_t launch_sinusoid(const float* t0, const float* t1, float* s0, float* s1, int M, int F, float period,
                           hipStream_t st);
// y = x[M, K] . W[N, K]^T in fp32 (N % 16 == 0, K % 16 == 0) for one or two
// independent chains (x, W, bias, out of chain c at index c) in one launch,
// in one of three modes: kFragToFrag (x in fragment order; act(y + bias)
// written in fragment order with padded_rows(M) rows; one split only),
// kFragToRows (x in fragment order; partial sums [splits][M][N], or with
// one split act(y + bias) row-major), kRowsSilu (x row-major, input
// SiLU(x)). Row-major results go to out row (n / ng) * M + m, column n % ng
// (ng % 16 == 0); bias may be null. The split count actually used is
// skinny_splits(K, splits).
// With x2 set (fragment-order modes), the input is [x | x2] along K: the
// last k2 columns (k2 % 16 == 0) come from x2 [Mpad, k2] in fragment order
// and x holds the first K - k2. scale multiplies the product before the bias
// (one split only when scale != 1).
enum SkinnyMode { kFragToFrag = 0, kFragToRows = 1, kRowsSilu = 2 };
struct SkinnyArgs {
  const float* x[2];
  const float* w[2];
  const float* bias[2];
  float* out[2];
  const float* x2[2] = {nullptr, nullptr};
  int k2 = 0;
  float scale = 1.f;
};
hipError_t launch_skinny_f32(int mode, const SkinnyArgs& args, int chains, int M, int N, int K, int splits, int ng,
                             int act, hipStream_t st);
int skinny_splits(int K, int splits);
// y_c = act(sum of the `splits` partial sums [splits][M][N] of chain c +
// bias_c) (bias may be null); out[M, N] = y_0, or with part1 non-null the
// blend (1 - gate) y_0 + gate y_1. N % 4 == 0.
hipError_t launch_rows_finish(const float* part0, const float* part1, int splits, const float* bias0,
                              const float* bias1, float* out, int M, int N, int act, float gate, hipStream_t st);
// table[(n / ng) * M + m][n % ng] = W[n] . bf16(SiLU(emb[m])) + bias[n] with
// bf16 W [N, K] and bias [N] (may be null), N % 64 == 0, K % 32 == 0.
// a_scratch: padded_rows(M) * K bf16 values (SiLU(emb) in bf16, stored in
// MFMA fragment order).
hipError_t launch_adaln_proj(const float* emb, const uint16_t* w, const uint16_t* bias, uint16_t* a_scratch, float* table,
                             int M, int N, int K, int ng, hipStream_t st);

// ---- model edges (input projections, output heads) ----
// x[b, idx[r]] = W h[b, r] + bias (h [B, nrows, C] fp32, W [D, C] fp32,
// C % 16 == 0, D % 256 == 0); indices clamped into [0, S).
template <typename T>
hipError_t launch_edge_in(const float* h, int nrows, int C, const float* W, const float* bias, const int32_t* idx,
                          int B, int S, int D, T* x, hipStream_t st);
// x[b, idx[k]] = text[b, k] for k < ntext, then x[b, r] = 0 where tags[r] == -1.
template <typename T>
hipError_t launch_edge_rows(const T* text, const int32_t* idx, int ntext, const int32_t* tags, int B, int S, int D,
                            T* x, hipStream_t st);
// W' = W diag(gamma) [C, D], s = W' 1, cv = W beta + b (b may be null).
hipError_t launch_edge_fold(const float* W, const float* b, const float* gamma, const float* beta, int C, int D,
                            float* Wf, float* s, float* cv, hipStream_t st);
// Two output heads in one launch: for head h, y_h[b, r] = (W'_h x_r - mu_r
// s_h) / sigma_r + cv_h, x_r = x[b, idx_h[r]], with the LayerNorm statistics
// of x_r (eps inside the root); C_h in {16, 32, 48, 64, 96, 128} with C_1 <=
// C_0 (head 1 may have no rows), D % 64 == 0; y_h [B, nrows_h, C_h] fp32.
struct EdgeHeads {
  const int32_t* idx[2];
  int nrows[2], C[2];
  const float* Wf[2];
  const float* s[2];
  const float* cv[2];
  float* y[2];
};
template <typename T>
hipError_t launch_edge_out(const T* x, const EdgeHeads& heads, int B, int S, int D, float eps, hipStream_t st);

// ---- rotated W8A8 ----
// Rows of x [M, K] (K % 128 == 0, K <= 16384): blockwise normalised Hadamard
// rotation (128 wide), then symmetric int8 codes q [M, K] and fp32 scales [M].
template <typename T>
hipError_t launch_rot_quant(const T* x, int M, int K, int8_t* q, float* scale, hipStream_t st);

// ---- denoising step: unmerged LoRA, Euler update ----
// out[m] = [x[m, 0:K] | s * t[m, 0:R]] (rows of K + R), 16-byte pieces.
// AdaLN (bf16 semantics) straight to rotated W8A8 codes q [B*S, D] and row
// scales qscale [B*S]; x bf16 or fp32; D % 128 == 0, D <= 8192.
hipError_t launch_adaln_rq(const void* x, bool x_f32, int8_t* q, float* qscale, const float* table,
                           const int32_t* tags, const int32_t* tidx, int B, int S, int D, int which, float eps,
                           int num_tags, int num_tvals, hipStream_t st);
// table [S, 3 fd] of (cos, sin) pairs: the rotary turn of each pair of each row
hipError_t launch_rope_table(const int32_t* pos, float* table, int S, int fd, float theta, hipStream_t st);
// zero rows / columns [S, stride) of the per-head q, k, v^T buffers (BH = B * heads)
hipError_t launch_qk_tail_zero(bf16_t* qo, bf16_t* ko, bf16_t* vto, int BH, int S, int stride, hipStream_t st);
template <typename T>
hipError_t launch_concat_rows(const T* x, const T* t, float s, T* out, long M, int K, int R, hipStream_t st);
// x_next[b, i] = x[b, i] + (sig_next[v] - sig_now[v]) * vel[b, i], v =
// tidx[idx[i]] (indices clamped); x_next may alias x.
hipError_t launch_euler(const float* x, const float* vel, float* x_next, int B, int nrows, int C,
                        const int32_t* idx, const int32_t* tidx, int S, const float* sig_now, const float* sig_next,
                        int ntv, hipStream_t st);

}  // namespace minih3
