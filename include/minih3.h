/*
 * minih3.h: C ABI of libminih3.so, the MI355X (gfx950) forward pass of a
 * MiniMax-H3-style diffusion-transformer block over one packed 1-D sequence.
 *
 * Source of what is computed: the diffusers documentation page
 * "MiniMaxH3Transformer3DModel" (class description, Parameters, `forward`).
 * One block stack runs over one packed sequence of text, conditioning,
 * audio and target-video rows; each row carries a modality tag that selects
 * its AdaLN modulation, a timestep index and a (t, h, w) rotary position;
 * padding rows (tag -1) form their own attention document.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *    owned by the caller. The library never allocates or frees device
 *    memory; scratch space comes from a caller-provided workspace.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; nothing synchronises unless a
 *    flag below says so.
 *  - Tensors are dense, row-major, with the shapes given per argument.
 *    "act" tensors have the dtype `minih3_config.act_dtype` (bfloat16 or
 *    float32); bfloat16 values are stored as IEEE bf16 bit patterns.
 *  - Every call returns an int status (minih3_status) and never aborts.
 *    Argument errors are found on the host before anything is enqueued.
 *  - Sizes (batch, seq_len, M, N, K) are at least 1: an empty sequence or
 *    matrix is the argument error MINIH3_E_ARG. Row counts of one modality
 *    (num_video, num_audio, num_text, the Euler step's num_rows) may be 0:
 *    that modality's part of the call is then skipped.
 *    Layout errors are found only under MINIH3_VALIDATE, which costs one
 *    stream synchronisation. Without it an invalid layout gives unspecified
 *    numbers, but every index the kernels use is clamped into range, so no
 *    access leaves its buffer.
 */
#ifndef MINIH3_H
#define MINIH3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MINIH3_OK = 0,
  MINIH3_E_ARG = -1,           /* null pointer, bad size or unsupported dims   */
  MINIH3_E_WORKSPACE = -2,     /* workspace null or smaller than required      */
  MINIH3_E_UNSUPPORTED = -3,   /* a dims combination the kernels do not cover  */
  MINIH3_E_SCRATCH = -4,       /* request larger than an allocation-free entry point's fixed scratch */
  MINIH3_E_LAYOUT_TAG = -10,   /* a tag outside {-1, 0 .. num_tags-1}          */
  MINIH3_E_LAYOUT_TVAL = -11,  /* timestep index outside [0, num_tvals) on a non-padding row */
  MINIH3_E_LAYOUT_INDEX = -12, /* index out of range, a row addressed twice, or a row of another modality */
  MINIH3_E_LAYOUT_PAD = -13,   /* index addresses a padding row, or a non-padding row is unaddressed */
  MINIH3_E_NEEDS_MASK = -14,   /* padding rows present under MINIH3_ASSUME_PADLESS */
  MINIH3_E_HIP = -20           /* a HIP runtime call failed                    */
} minih3_status;

typedef enum { MINIH3_BF16 = 0, MINIH3_F32 = 1 } minih3_dtype;

enum {
  /* Validate the layout (tags, timestep indices, index tensors) on the
   * device and synchronise the stream to report the first error by the
   * precedence TAG, TVAL, INDEX, PAD, NEEDS_MASK. */
  MINIH3_VALIDATE = 1u,
  /* The caller promises a padless sequence (no tag -1 row): attention
   * treats all rows as one document. With MINIH3_VALIDATE a -1 row gives
   * MINIH3_E_NEEDS_MASK; without it, -1 rows are attended as ordinary rows. */
  MINIH3_ASSUME_PADLESS = 2u,
  /* Time every kernel of minih3_block_forward with HIP events on `stream`;
   * read the totals with minih3_profile_collect. */
  MINIH3_PROFILE = 4u
};

/* Model dimensions (page "MiniMaxH3Transformer3DModel", Parameters). */
typedef struct {
  int32_t hidden;        /* residual width D (5376); multiple of 256, at most
                            8192 for bf16 and 4096 for fp32 blocks            */
  int32_t num_heads;     /* H (56); even for the block entry points (the QKV
                            width 3*H*hd is then a multiple of 256); any for
                            the attention and q/k entry points               */
  int32_t head_dim;      /* hd; must be 128                                      */
  int32_t ffn_dim;       /* F, inner width of each SwiGLU half (14336); multiple of 128 */
  int32_t rope_freq_dim; /* rotary frequencies per axis (16); 6*rope_freq_dim <= head_dim */
  float rope_theta;      /* rotary base (1e4)                                    */
  float norm_eps;        /* eps of the two AdaLN LayerNorms (1e-5)               */
  float qk_norm_eps;     /* eps of the per-head q/k RMSNorms (1e-5)              */
  int32_t num_tags;      /* modality tags that own an AdaLN table (3)            */
  int32_t num_tvals;     /* timestep values per tag in the AdaLN table           */
  int32_t tag_text, tag_video, tag_audio; /* tag value carried by each index tensor's rows */
  int32_t act_dtype;     /* minih3_dtype of activations and weight matrices      */
} minih3_config;

/* One packed layout, shared by every batch item (the batch axis is a pure
 * replication axis; each item is its own sequence). Page `forward`:
 * timestep_indices, token_tags, position_ids, video/audio/text_indices. */
typedef struct {
  int32_t batch;                    /* B >= 1                                   */
  int32_t seq_len;                  /* S >= 1                                   */
  const int32_t* token_tags;        /* [S] modality tag, -1 = padding row        */
  const int32_t* timestep_indices;  /* [S] index into the AdaLN table's timestep axis; ignored on padding rows */
  const int32_t* position_ids;      /* [S, 3] (t, h, w) rotary coordinates       */
  const int32_t* video_indices; int32_t num_video; /* rows of conditioning + target video */
  const int32_t* audio_indices; int32_t num_audio;
  const int32_t* text_indices;  int32_t num_text;  /* index tensors may be NULL when their count is 0;
                                                      they are read only under MINIH3_VALIDATE */
} minih3_layout;

/* Weights of one block. Matrices are act_dtype, row-major [out, in]. */
typedef struct {
  const void* w_qkv;        /* [3W, D], W = H*hd: rows [0,W) q, [W,2W) k, [2W,3W) v; head h = rows [h*hd, (h+1)*hd) of each */
  const void* w_out;        /* [D, W]                                        */
  const void* w_gate_up;    /* [2F, D]: rows [0,F) gate, [F,2F) up            */
  const void* w_down;       /* [D, F]                                        */
  const float* q_norm;      /* [hd] RMSNorm weight shared by all query heads  */
  const float* k_norm;      /* [hd] RMSNorm weight shared by all key heads    */
  const float* adaln_table; /* [num_tags, num_tvals, 6, D] fp32: shift1, scale1, gate1 (attention),
                               shift2, scale2, gate2 (FFN); padding rows use zeros */
} minih3_block_weights;

/* Optional copies of intermediates of the FIRST block (tests). Every field
 * may be NULL. Shapes (S_pad = S rounded up to a multiple of 64):
 *   adaln1, adaln2, attn_proj, ffn_out : [B, S, D] act
 *   x_mid        : [B, S, D] fp32, the residual stream after the attention's
 *                  gated add (the library keeps the residual stream in fp32)
 *   q_rot, k_rot : [B, H, S_pad, hd] act (post RMSNorm + RoPE)
 *   v_t          : [B, H, hd, S_pad] act (values, transposed)
 *   attn_o       : [B, S, W] act;  ffn_h : [B, S, F] act
 *   table_row    : [S] int32 tag*num_tvals + tidx, -1 on padding rows
 *   doc_id       : [S] int32 attention document (1 = padding row)
 *   tile_flags   : [ceil(S/64)] int32 bit0 = tile holds a non-padding row, bit1 = a padding row
 *   num_pad      : [1] int32
 *   block_out    : [B, S, D] fp32, the residual stream after the first
 *                  block before it is rounded to act (for a one-block call
 *                  x_out is exactly this tensor rounded to act) */
typedef struct {
  void *adaln1, *q_rot, *k_rot, *v_t, *attn_o, *attn_proj, *x_mid, *adaln2, *ffn_h, *ffn_out;
  int32_t *table_row, *doc_id, *tile_flags, *num_pad;
  void* block_out;
} minih3_taps;

/* Bytes of workspace minih3_block_forward needs for (batch, seq_len). */
int minih3_workspace_bytes(const minih3_config* cfg, int32_t batch, int32_t seq_len, size_t* bytes);

/* Forward pass of `num_blocks` consecutive blocks (page: num_layers blocks
 * in one stack) over x_in [B, S, D] act -> x_out [B, S, D] act. Per block:
 * AdaLN (LN + (1+scale)/shift chosen by tag and timestep index), QKV
 * projection, per-head q/k RMSNorm, 3-D RoPE, attention within documents
 * (padding rows alone), output projection with gated residual, AdaLN,
 * SwiGLU FFN with gated residual. Padding rows leave the block unchanged.
 * x_out must not alias x_in or the workspace. For bf16 every projection
 * operand (B*S rows of D, H*hd or ffn_dim values) must stay below 4 GiB
 * (MINIH3_E_UNSUPPORTED otherwise). */
int minih3_block_forward(const minih3_config* cfg, const minih3_layout* layout,
                         const minih3_block_weights* blocks, int32_t num_blocks,
                         const void* x_in, void* x_out, void* workspace, size_t workspace_bytes,
                         uint32_t flags, minih3_taps* taps, void* stream);

/* Bytes of workspace minih3_attention_packed needs for (batch, seq_len)
 * with cfg->num_heads heads (q, k and v^T in the kernels' layouts, plus the
 * per-tile document masks). */
int minih3_attention_workspace_bytes(const minih3_config* cfg, int32_t batch, int32_t seq_len, size_t* bytes);

/* Attention over the packed sequence. Page "MiniMaxH3Transformer3DModel",
 * class description: attention is full self-attention over the one packed
 * sequence (text, conditioning, audio and target-video rows alike); a
 * layout that carries padding rows (tag -1) keeps them in their own
 * attention document with a boolean mask; the batch axis replicates the
 * layout, each item its own sequence. The page gives no softmax scale; the
 * library takes 1/sqrt(hd) unless the caller passes one:
 *   out[b, i, h*hd:(h+1)*hd] = sum_j softmax_j(scale * q_i . k_j) v_j,
 * over j < S with doc(j) == doc(i), doc = (tag == -1); under
 * MINIH3_ASSUME_PADLESS every row is in one document.
 * q, k, v : [B, S, H, hd] act, q and k after the per-head norm and the
 *           rotary embedding (as the block applies them before attention)
 * out     : [B, S, H*hd] act (must not alias q, k or v)
 * The inputs are copied into the workspace in the layouts the kernels read
 * (see minih3_attention_headmajor). Only token_tags (and batch, seq_len) of
 * the layout are read; with MINIH3_VALIDATE | MINIH3_ASSUME_PADLESS a -1
 * row gives MINIH3_E_NEEDS_MASK (one stream synchronisation). Reads
 * head_dim (128), num_heads and act_dtype of cfg. */
int minih3_attention_packed(const minih3_config* cfg, const minih3_layout* layout, const void* q, const void* k,
                            const void* v, void* out, float softmax_scale, void* workspace, size_t workspace_bytes,
                            uint32_t flags, void* stream);

/* Bytes of workspace minih3_attention_headmajor needs. */
int minih3_attention_headmajor_workspace_bytes(const minih3_config* cfg, int32_t batch, int32_t seq_len,
                                               size_t* bytes);

/* minih3_attention_packed on inputs already in the kernels' layouts (what
 * the block's QKV projection writes), without the copy:
 * q, k : [B, H, seq_stride, hd] act;  v_t : [B, H, hd, seq_stride] act;
 * out  : [B, S, H*hd] act. seq_stride >= S and a multiple of 64; rows
 * and columns in [S, seq_stride) are never used in the result but must be
 * readable. */
int minih3_attention_headmajor(const minih3_config* cfg, const minih3_layout* layout, const void* q, const void* k,
                               const void* v_t, int32_t seq_stride, void* out, float softmax_scale, void* workspace,
                               size_t workspace_bytes, uint32_t flags, void* stream);

/* One AdaLN modulation. Page "MiniMaxH3Transformer3DModel": Parameters
 * (norm_eps of the pre-attention and pre-feed-forward norms) and class
 * description (the row's modality tag selects its AdaLN modulation
 * parameters; `forward` timestep_indices picks the row's timestep). The
 * page does not write the form; the library takes the non-affine LayerNorm
 * (mean, biased variance) with the modulation as its affine part:
 * y = LN(x) * (1 + scale) + shift per row, with
 * (shift, scale) = adaln_table[tag, tidx, 3*which + {0, 1}] and zeros on
 * padding rows. which = 0 before attention, 1 before the FFN.
 * x, y : [B, S, D] act (may alias); adaln_table [num_tags, num_tvals, 6, D]
 * fp32. Indices out of range are clamped (no layout validation here). */
int minih3_adaln_modulate(const minih3_config* cfg, const minih3_layout* layout, const void* x,
                          const float* adaln_table, int32_t which, void* y, uint32_t flags, void* stream);

/* Per-head RMSNorm of q and k (weights q_norm, k_norm) followed by the
 * 3-D rotary embedding on 6*rope_freq_dim channels: axis a (t, h, w) owns
 * channels [2*fd*a, 2*fd*(a+1)), pair j = channels (2j, 2j+1) in it turns
 * by position[a] * rope_theta^(-j/fd); other channels pass through.
 * qkv   : [B, S, 3W] act (the QKV projection output)
 * q_out, k_out : [B, H, seq_stride, hd] act;  v_t_out : [B, H, hd, seq_stride] act
 * Rows [S, seq_stride) of the outputs are written as zeros. Reads head_dim
 * (128), num_heads (any), act_dtype, rope_freq_dim, rope_theta and
 * qk_norm_eps of cfg. */
int minih3_qk_norm_rope(const minih3_config* cfg, const minih3_layout* layout, const void* qkv,
                        const float* q_norm, const float* k_norm, void* q_out, void* k_out,
                        void* v_t_out, int32_t seq_stride, void* stream);

/* Plain projection c[M, N] = a[M, K] . w[N, K]^T in `dtype`, fp32
 * accumulation. Constraints: N % 256 == 0, K % 64 == 0, M >= 1; for bf16
 * also 2*M*K and 2*N*K below 4 GiB (MINIH3_E_UNSUPPORTED otherwise). */
int minih3_linear(int32_t dtype, const void* a, const void* w, void* c, int32_t M, int32_t N, int32_t K,
                  void* stream);

/* ---- Timestep conditioning: building the AdaLN tables ----
 * Page "MiniMaxH3Transformer3DModel": Parameters freq_dim (sinusoidal
 * timestep embedding; timesteps are used unscaled, in [0, 1]),
 * time_embed_hidden_dim and time_embed_dim (the timestep MLP, whose output
 * is the input of every AdaLN projection), the mixed-precision note (the
 * timestep MLP is float32, the block stack bfloat16), `forward` `timestep`
 * (the distinct timestep values that timestep_indices point at) and the
 * class description (the modality tag selects the AdaLN modulation). Page
 * "HyperFlow for MiniMax-H3", How it works: a second embedder for the step
 * endpoint r is blended with the base one by a fixed gate; conditioning rows
 * keep r = t. Where the pages leave the form open, the library takes:
 * s(t) = [cos(t f_j), sin(t f_j)], f_j = max_period^(-j / (freq_dim/2));
 * E(t) = W2 SiLU(W1 s(t) + b1) + b2; two-time e = (1 - gate) E(t) + gate E'(r);
 * table row (tag k, value v) = W_k SiLU(e_v) + b_k viewed as [6, D]. */
typedef struct {
  int32_t freq_dim;   /* sinusoid width (256); multiple of 32                 */
  int32_t hidden_dim; /* timestep MLP inner width (5376); multiple of 16      */
  int32_t embed_dim;  /* timestep MLP output width (2688); multiple of 16     */
  float max_period;   /* base of the sinusoid frequencies (1e4)               */
} minih3_time_config;

/* fp32 timestep-MLP weights, row-major [out, in]; a NULL bias is zero. */
typedef struct {
  const float* w1; /* [hidden_dim, freq_dim] */
  const float* b1; /* [hidden_dim]           */
  const float* w2; /* [embed_dim, hidden_dim] */
  const float* b2; /* [embed_dim]            */
} minih3_time_mlp;

/* Bytes of workspace minih3_time_embed needs for num_tvals values. */
int minih3_time_embed_workspace_bytes(const minih3_time_config* tc, int32_t num_tvals, size_t* bytes);

/* Time embeddings of num_tvals timestep values, fp32 throughout:
 * emb[v] = E(t[v]), or with `endpoint` non-NULL (two-time conditioning)
 * emb[v] = (1 - gate) E(t[v]) + gate E'(r[v]), E' the MLP with the endpoint
 * weights (r NULL: r = t). t, r : [num_tvals] fp32; emb : [num_tvals,
 * embed_dim] fp32. Split-K partial sums are added in a fixed order, so
 * repeated calls give identical bits. */
int minih3_time_embed(const minih3_time_config* tc, const minih3_time_mlp* base, const float* t,
                      const minih3_time_mlp* endpoint, const float* r, float gate, int32_t num_tvals, float* emb,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Unmerged adapter of one timestep MLP (header table of the HyperFlow page:
 * LoRA on both time embedders), fp32: layer 1 computes
 * W1 s + lora_scale * B1 (A1 s) + b1, layer 2 likewise with A2, B2; each as
 * u = lora_scale * A x, then [x | u] . [W | B]^T with the packed matrices.
 * a1 [rank, freq_dim], packed1 [hidden_dim, freq_dim + rank] = [W1 | B1],
 * a2 [rank, hidden_dim], packed2 [embed_dim, hidden_dim + rank] = [W2 | B2]
 * (minih3_lora_pack_weight with MINIH3_F32). */
typedef struct {
  const float* a1;
  const float* packed1;
  const float* a2;
  const float* packed2;
} minih3_time_mlp_lora;

/* Bytes of workspace minih3_time_embed_lora needs (rank % 16 == 0). */
int minih3_time_embed_lora_workspace_bytes(const minih3_time_config* tc, int32_t num_tvals, int32_t rank,
                                           size_t* bytes);

/* minih3_time_embed with an unmerged adapter on each timestep MLP: base_lora
 * for the base MLP, endpoint_lora for the endpoint one (required when
 * endpoint is set). The w1 and w2 of base / endpoint are not read (the
 * packed matrices hold them); the biases are. lora_scale = scale * alpha /
 * rank. Split-K partial sums are added in a fixed order, so repeated calls
 * give identical bits. */
int minih3_time_embed_lora(const minih3_time_config* tc, const minih3_time_mlp* base,
                           const minih3_time_mlp_lora* base_lora, const float* t, const minih3_time_mlp* endpoint,
                           const minih3_time_mlp_lora* endpoint_lora, const float* r, float gate, int32_t num_tvals,
                           int32_t rank, float lora_scale, float* emb, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of workspace minih3_adaln_table needs (0 for fp32 activations). */
int minih3_adaln_table_workspace_bytes(const minih3_config* cfg, int32_t embed_dim, size_t* bytes);

/* AdaLN table of one block from the time embeddings:
 * table[k, v, c, :] = (W_k SiLU(emb[v]) + b_k)[c*D : (c+1)*D], c = shift1,
 * scale1, gate1, shift2, scale2, gate2 (the layout of
 * minih3_block_weights.adaln_table). Reads hidden (D), num_tags, num_tvals
 * and act_dtype of cfg.
 * emb    : [num_tvals, embed_dim] fp32
 * w_proj : [num_tags, 6 D, embed_dim] act;  b_proj : [num_tags, 6 D] act or NULL
 * table  : [num_tags, num_tvals, 6, D] fp32 (output)
 * bf16: SiLU(emb) is rounded to bf16 for the MFMA product (fp32
 * accumulation, fp32 output); embed_dim % 32 == 0. fp32: embed_dim % 16 == 0. */
int minih3_adaln_table(const minih3_config* cfg, const float* emb, int32_t embed_dim, const void* w_proj,
                       const void* b_proj, float* table, void* workspace, size_t workspace_bytes, void* stream);

/* minih3_adaln_table without a workspace, for callers that cannot
 * allocate device memory: code recorded under HIP graph capture, serving
 * loops that must not call hipMalloc, harnesses that forbid it. The caller
 * passes the inputs and the output as for minih3_adaln_table; the bf16
 * SiLU(emb) operand lives in a fixed 1 MiB device array of the library
 * (one per device, held until the process ends). Limit:
 * minih3_adaln_table_workspace_bytes(cfg, embed_dim) <= 1 MiB (e.g. up to
 * 192 timestep values at embed_dim 2688), else MINIH3_E_SCRATCH before
 * anything is enqueued. Every call on a device shares that array: calls
 * that overlap on one device (other streams, other threads) race; calls
 * in order on one stream do not. Nothing is allocated or freed; the first
 * call on a device looks the array's address up once. */
int minih3_adaln_table_noalloc(const minih3_config* cfg, const float* emb, int32_t embed_dim, const void* w_proj,
                               const void* b_proj, float* table, void* stream);

/* ---- Model edges: the packed sequence in, the velocities out ----
 * Page "MiniMaxH3Transformer3DModel": Parameters in_channels, patch_size,
 * audio_in_channels, final_norm_eps; the mixed-precision note (the input
 * patch projections and the output heads are float32); `forward`
 * (hidden_states: patchified video rows in the order of video_indices;
 * audio_hidden_states in the order of audio_indices; the returned video and
 * audio velocities in those orders). Where the pages leave the form open the
 * library takes: proj_in / audio_proj_in are Linear layers with bias;
 * text rows arrive already embedded (the text refiner is not part of this
 * library); norm_out is a LayerNorm with weight and bias shared by the video
 * and audio rows; proj_out / audio_proj_out are Linear layers with bias. */
typedef struct {
  int32_t video_channels;  /* in_channels * prod(patch_size) (24 * 1*2*2 = 96); one of 16, 32, 48, 64, 96, 128 */
  int32_t audio_channels;  /* audio_in_channels (32); one of 16, 32, 48, 64, 96, 128 */
  float final_norm_eps;    /* eps of norm_out (1e-5) */
  const float* w_in;        /* proj_in weight [D, video_channels] fp32        */
  const float* b_in;        /* proj_in bias [D]                               */
  const float* w_audio_in;  /* audio_proj_in weight [D, audio_channels]       */
  const float* b_audio_in;  /* audio_proj_in bias [D]                         */
  const float* norm_w;      /* norm_out weight [D]                            */
  const float* norm_b;      /* norm_out bias [D]                              */
  const float* w_out;       /* proj_out weight [video_channels, D]            */
  const float* b_out;       /* proj_out bias [video_channels] (NULL = zero)   */
  const float* w_audio_out; /* audio_proj_out weight [audio_channels, D]      */
  const float* b_audio_out; /* audio_proj_out bias [audio_channels] (NULL = zero) */
} minih3_edges;

/* Bytes of workspace minih3_embed_inputs / minih3_output_heads need. */
int minih3_edges_workspace_bytes(const minih3_config* cfg, const minih3_edges* edges, int32_t seq_len, size_t* bytes);

/* The packed sequence x [B, S, D] act from the model inputs:
 * x[b, video_indices[i]] = proj_in(video[b, i]), x[b, audio_indices[j]] =
 * audio_proj_in(audio[b, j]) (fp32 arithmetic, rounded to act),
 * x[b, text_indices[k]] = text[b, k] (copied), and zero on padding rows.
 * video : [B, num_video, video_channels] fp32;  audio : [B, num_audio,
 * audio_channels] fp32;  text : [B, num_text, D] act. Rows that no index
 * tensor addresses and that are not padding rows (only in an invalid
 * layout) are left as they were; MINIH3_VALIDATE checks the layout first.
 * Reads hidden and act_dtype of cfg (and the layout fields under
 * MINIH3_VALIDATE). */
int minih3_embed_inputs(const minih3_config* cfg, const minih3_layout* layout, const minih3_edges* edges,
                        const float* video, const float* audio, const void* text, void* x, void* workspace,
                        size_t workspace_bytes, uint32_t flags, void* stream);

/* The velocities from the final hidden states x [B, S, D] act:
 * video_out[b, i] = proj_out(norm_out(x[b, video_indices[i]])) and
 * audio_out[b, j] = audio_proj_out(norm_out(x[b, audio_indices[j]])), fp32.
 * video_out : [B, num_video, video_channels];  audio_out : [B, num_audio,
 * audio_channels]. norm_out is applied as W diag(w) (x - mean) / sd + (W b +
 * bias) with the statistics of each row. */
int minih3_output_heads(const minih3_config* cfg, const minih3_layout* layout, const minih3_edges* edges,
                        const void* x, float* video_out, float* audio_out, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream);

/* ---- Rotated W8A8 INT8 linear layers ----
 * Page "HyperFlow H3 Flash Brings MiniMax H3 Video to One GPU", How it got
 * smaller and faster: rotated W8A8 INT8 quantization of the linear layers.
 * The library takes: the rotation is the normalised Hadamard transform of
 * every 128-wide block of a row, applied alike to activation rows and
 * weight rows (so x W^T is unchanged); quantization is symmetric int8 per
 * row, code = rint(v * (127 / amax)) in [-127, 127], scale = amax / 127
 * (all-zero rows: codes 0, scale 0); the product accumulates the codes
 * exactly in int32 and dequantizes with the two scales. The butterflies run
 * in stages 1, 2, 4, ..., 64 in fp32 followed by one multiplication by
 * fp32(1/sqrt(128)), and both divisions are correctly rounded fp32, so the
 * codes are reproducible from that definition. */

/* Rotate and quantize the rows of x [M, K] (dtype MINIH3_BF16 or
 * MINIH3_F32; K a multiple of 128, at most 16384): q [M, K] int8 codes,
 * scale [M] fp32. Weight rows [N, K] are prepared the same way, once. */
int minih3_rotate_quantize(int32_t dtype, const void* x, int32_t M, int32_t K, int8_t* q, float* scale,
                           void* stream);

/* Weights of one block for the rotated W8A8 forward: each projection's
 * weight rows as int8 codes with per-row fp32 scales, as
 * minih3_rotate_quantize returns them for the bf16 matrices of
 * minih3_block_weights (same shapes and row order); norms and table as there. */
typedef struct {
  const int8_t* q_qkv;     const float* s_qkv;     /* [3W, D], [3W] */
  const int8_t* q_out;     const float* s_out;     /* [D, W],  [D]  */
  const int8_t* q_gate_up; const float* s_gate_up; /* [2F, D], [2F] */
  const int8_t* q_down;    const float* s_down;    /* [D, F],  [D]  */
  const float* q_norm;
  const float* k_norm;
  const float* adaln_table;
} minih3_block_weights_w8a8;

/* Bytes of workspace minih3_block_forward_w8a8 needs (bf16 configs only). */
int minih3_workspace_bytes_w8a8(const minih3_config* cfg, int32_t batch, int32_t seq_len, size_t* bytes);

/* minih3_block_forward with every projection on rotated W8A8: the bf16 input
 * rows of each projection are rotated and quantized per row, multiplied with
 * the int8 weight codes on int8 MFMAs and dequantized into the same fused
 * epilogues (store, gated residual, SwiGLU). bf16 activations only; D, H*hd
 * and ffn_dim multiples of 128 and at most 16384. Taps as in
 * minih3_block_forward (attn_proj and ffn_out are the W8A8 products). */
int minih3_block_forward_w8a8(const minih3_config* cfg, const minih3_layout* layout,
                              const minih3_block_weights_w8a8* blocks, int32_t num_blocks, const void* x_in,
                              void* x_out, void* workspace, size_t workspace_bytes, uint32_t flags,
                              minih3_taps* taps, void* stream);

/* c[M, N] = bf16((qa . qw^T) * sa[m] * sw[n]): int8 codes qa [M, K] and
 * qw [N, K] with their row scales sa [M], sw [N] (from
 * minih3_rotate_quantize), exact int32 accumulation on int8 MFMAs, fp32
 * dequantization, bf16 output. N % 256 == 0, K % 128 == 0; M*K and N*K
 * below 4 GiB. */
int minih3_linear_w8a8(const int8_t* qa, const float* sa, const int8_t* qw, const float* sw, void* c, int32_t M,
                       int32_t N, int32_t K, void* stream);

/* ---- Denoising step around the blocks: unmerged LoRA, Euler update ----
 * Page "HyperFlow for MiniMax-H3", header table: a PEFT LoRA (rank 256,
 * alpha 256) on the attention and feed-forward layers; sampling on a fixed
 * sigma grid (video shift 12, audio shift 3). Page
 * "MiniMaxH3Transformer3DModel", `forward`: a scale may be applied to the
 * LoRA layers; the model returns the velocities. The library takes the PEFT
 * form y = x W^T + scale * (alpha / rank) * (x A^T) B^T (A [rank, in], B
 * [out, rank]), and the Euler step of the flow x' = x + (sigma_next -
 * sigma_now) * v. */

/* packed [N, K + rank] = [W | B] for minih3_linear_lora (once per layer);
 * dtype MINIH3_BF16 or MINIH3_F32; w [N, K], lora_b [N, rank]. */
int minih3_lora_pack_weight(int32_t dtype, const void* w, const void* lora_b, void* packed, int32_t N, int32_t K,
                            int32_t rank, void* stream);

/* Bytes of workspace minih3_linear_lora needs (M x rank values of dtype). */
int minih3_linear_lora_workspace_bytes(int32_t dtype, int32_t M, int32_t K, int32_t rank, size_t* bytes);

/* c[M, N] = a W^T + lora_scale * (a A^T) B^T with lora_scale = scale *
 * alpha / rank, the base weight left unmerged: t = lora_scale * a A^T
 * (rounded to dtype, kept in the workspace), then one projection over
 * [a | t] and packed = [W | B], its A operand read from a and t in place.
 * a [M, K], lora_a [rank, K], packed [N, K + rank], c [M, N], all dtype.
 * bf16: rank and N multiples of 256, K of 64; fp32: rank and N of 64, K of 16. */
int minih3_linear_lora(int32_t dtype, const void* a, const void* lora_a, const void* packed, float lora_scale,
                       void* c, int32_t M, int32_t N, int32_t K, int32_t rank, void* workspace,
                       size_t workspace_bytes, void* stream);

/* x_next[b, i] = x[b, i] + (sigma_next[v] - sigma_now[v]) * velocity[b, i]
 * for the rows i < num_rows of one modality (x, velocity, x_next [batch,
 * num_rows, channels] fp32, in the order of `indices`), v =
 * timestep_indices[indices[i]] (indices clamped into range). Rows whose
 * timestep value has sigma_next == sigma_now (conditioning rows, r = t)
 * stay as they are. x_next may alias x. */
int minih3_euler_step(const float* x, const float* velocity, float* x_next, int32_t batch, int32_t num_rows,
                      int32_t channels, const int32_t* indices, const int32_t* timestep_indices, int32_t seq_len,
                      const float* sigma_now, const float* sigma_next, int32_t num_tvals, void* stream);

/* Unmerged adapters of a block's four projections (header table of the
 * HyperFlow page: LoRA on the attention and feed-forward layers; `forward`
 * of the model page: a scale for the LoRA layers). Projection P with base
 * weight W [N, K] computes x W^T + lora_scale * (x A^T) B^T, evaluated as in
 * minih3_linear_lora: t = lora_scale * x A^T (act, in the workspace), then
 * one projection of [x | t] against packed = [W | B] with P's fused
 * epilogue (q/k norm + rotary, gated residual, SwiGLU). */
typedef struct {
  const void* a_qkv;     const void* packed_qkv;      /* [rank, D], [3W, D + rank] */
  const void* a_out;     const void* packed_out;      /* [rank, W], [D, W + rank]  */
  const void* a_gate_up; const void* packed_gate_up;  /* [rank, D], [2F, D + rank] */
  const void* a_down;    const void* packed_down;     /* [rank, F], [D, F + rank]  */
} minih3_block_lora;

/* Bytes of workspace minih3_block_forward_lora needs. */
int minih3_workspace_bytes_lora(const minih3_config* cfg, int32_t batch, int32_t seq_len, int32_t rank,
                                size_t* bytes);

/* minih3_block_forward with an unmerged adapter on every projection of
 * every block: loras[i] belongs to blocks[i], whose w_qkv, w_out,
 * w_gate_up and w_down are not read (packed holds them); q_norm, k_norm
 * and adaln_table are. lora_scale = scale * alpha / rank. bf16: rank a
 * multiple of 256; fp32: of 64. Taps as in minih3_block_forward (attn_proj
 * and ffn_out include the adapter). */
int minih3_block_forward_lora(const minih3_config* cfg, const minih3_layout* layout,
                              const minih3_block_weights* blocks, const minih3_block_lora* loras, int32_t num_blocks,
                              int32_t rank, float lora_scale, const void* x_in, void* x_out, void* workspace,
                              size_t workspace_bytes, uint32_t flags, minih3_taps* taps, void* stream);

/* One denoising step of the model on the packed layout: the input
 * projections build x from the video / audio latents and the embedded text
 * rows (minih3_embed_inputs), the block chain runs on it
 * (minih3_block_forward, or minih3_block_forward_w8a8 when qblocks is set),
 * the heads give the velocities (minih3_output_heads), and the Euler update
 * moves the latents in place (minih3_euler_step with sigma_now /
 * sigma_next, the pair of each row's timestep value; conditioning rows carry
 * r = t and stay). The AdaLN tables inside the block weights are built by
 * the caller for this step's timestep values (minih3_time_embed,
 * minih3_adaln_table). video [B, num_video, video_channels] and audio
 * [B, num_audio, audio_channels] fp32 are read and overwritten; text
 * [B, num_text, D] act. */
typedef struct {
  int32_t num_blocks;
  const minih3_block_weights* blocks;        /* bf16 / fp32 blocks, or NULL  */
  const minih3_block_weights_w8a8* qblocks;  /* W8A8 blocks (bf16 only), or NULL; exactly one of the two */
  const minih3_edges* edges;
  const float* sigma_now;                    /* [num_tvals] */
  const float* sigma_next;                   /* [num_tvals] */
  const minih3_block_lora* loras;            /* per block, or NULL (not with qblocks) */
  int32_t lora_rank;                         /* rank of loras                */
  float lora_scale;                          /* scale * alpha / rank         */
} minih3_step_weights;

/* Bytes of workspace minih3_denoise_step needs. */
int minih3_denoise_step_workspace_bytes(const minih3_config* cfg, const minih3_step_weights* weights, int32_t batch,
                                        int32_t seq_len, int32_t num_video, int32_t num_audio, size_t* bytes);

int minih3_denoise_step(const minih3_config* cfg, const minih3_layout* layout, const minih3_step_weights* weights,
                        float* video, float* audio, const void* text, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream);

/* Kernel timing under MINIH3_PROFILE. Synchronises the recorded events,
 * writes for each kernel id k < n the summed milliseconds and the number of
 * launches since the last collect, then resets. Returns the number of
 * kernel ids. */
int minih3_profile_collect(double* total_ms, int32_t* launches, int32_t n);
const char* minih3_kernel_name(int32_t id);

const char* minih3_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MINIH3_H */
