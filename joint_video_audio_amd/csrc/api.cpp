// C ABI of libminih3: argument checks, workspace carving, the launch
// sequence of one block and of a chain of blocks, kernel timing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <utility>
#include <vector>

#include "../../include/minih3.h"
#include "common.h"
#include "kernels.h"

using namespace minih3;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---- the allocation-free AdaLN table build ----
// Scratch of minih3_adaln_table_noalloc: the bf16 SiLU(emb) operand of the
// table projection (padded rows, fragment order). A device variable: every
// device the library runs on holds its own copy until the process ends, and
// every call on that device shares it.
constexpr size_t kNoallocScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (the array's name is a host-side stand-in, not a device address).
int noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MINIH3_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MINIH3_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MINIH3_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MINIH3_OK;
}

// Kernel ids reported by minih3_profile_collect.
enum KernelId {
  kKLayout = 0, kKTiles, kKAdaLN1, kKQKV, kKQKNormRope, kKAttnPrep, kKAttention, kKOutProj, kKAdaLN2, kKGateUp,
  kKDown, kKNumIds
};
const char* kKernelNames[kKNumIds] = {"layout_validate", "attention_tiles", "adaln_pre_attention",
                                      "qkv_projection", "qk_norm_rope", "attention_key_norms", "attention",
                                      "out_projection_gated_residual", "adaln_pre_ffn", "gate_up_swiglu",
                                      "down_projection_gated_residual"};

struct Profiler {
  std::mutex mu;
  struct Rec { int id; hipEvent_t a, b; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler g_prof;

// Records HIP events around the launches of one kernel when enabled.
struct Timed {
  bool on;
  int id;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(bool on_, int id_, hipStream_t st_) : on(on_), id(id_), st(st_) {
    if (!on) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    a = g_prof.get();
    b = g_prof.get();
    if (a && b) (void)hipEventRecord(a, st);
  }
  ~Timed() {
    if (!on || !a || !b) return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.recs.push_back({id, a, b});
  }
};

int act_size(int dtype) { return dtype == MINIH3_BF16 ? 2 : 4; }

int check_config(const minih3_config* c) {
  if (!c) return MINIH3_E_ARG;
  if (c->act_dtype != MINIH3_BF16 && c->act_dtype != MINIH3_F32) return MINIH3_E_ARG;
  if (c->head_dim != 128) return MINIH3_E_UNSUPPORTED;
  if (c->num_heads < 1 || c->hidden < 256 || c->hidden % 256 != 0) return MINIH3_E_UNSUPPORTED;
  if (c->ffn_dim < 128 || c->ffn_dim % 128 != 0) return MINIH3_E_UNSUPPORTED;
  if ((3L * c->num_heads * c->head_dim) % 256 != 0) return MINIH3_E_UNSUPPORTED;
  const int vec = c->act_dtype == MINIH3_BF16 ? 8 : 4;
  if (c->hidden / vec > 1024) return MINIH3_E_UNSUPPORTED;
  if (c->rope_freq_dim < 0 || 6 * c->rope_freq_dim > c->head_dim) return MINIH3_E_UNSUPPORTED;
  if (!(c->rope_theta > 0.f) || !(c->norm_eps >= 0.f) || !(c->qk_norm_eps >= 0.f)) return MINIH3_E_ARG;
  if (c->num_tags < 1 || c->num_tvals < 1) return MINIH3_E_ARG;
  return MINIH3_OK;
}

// Attention reads only head_dim, num_heads and act_dtype of the config.
int check_config_attention(const minih3_config* c) {
  if (!c) return MINIH3_E_ARG;
  if (c->act_dtype != MINIH3_BF16 && c->act_dtype != MINIH3_F32) return MINIH3_E_ARG;
  if (c->head_dim != 128 || c->num_heads < 1) return MINIH3_E_UNSUPPORTED;
  return MINIH3_OK;
}

// q/k norm + RoPE reads head_dim, num_heads, act_dtype, the rotary fields and
// qk_norm_eps of the config (any head count).
int check_config_qk(const minih3_config* c) {
  int s = check_config_attention(c);
  if (s) return s;
  if (c->rope_freq_dim < 0 || 6 * c->rope_freq_dim > c->head_dim) return MINIH3_E_UNSUPPORTED;
  if (!(c->rope_theta > 0.f) || !(c->qk_norm_eps >= 0.f)) return MINIH3_E_ARG;
  return MINIH3_OK;
}

// The bf16 projection kernel addresses each operand with 32-bit byte offsets.
bool gemm_fits(long M, long N, long K) { return M * K * 2 <= 0xFFFFFFFFL && N * K * 2 <= 0xFFFFFFFFL; }

int check_layout(const minih3_layout* L, bool need_indices) {
  if (!L) return MINIH3_E_ARG;
  if (L->batch < 1 || L->seq_len < 1) return MINIH3_E_ARG;
  if ((long)L->batch * L->seq_len > (1L << 30)) return MINIH3_E_UNSUPPORTED;
  if (!L->token_tags || !L->timestep_indices || !L->position_ids) return MINIH3_E_ARG;
  if (L->num_video < 0 || L->num_audio < 0 || L->num_text < 0) return MINIH3_E_ARG;
  if (need_indices) {
    if ((L->num_video && !L->video_indices) || (L->num_audio && !L->audio_indices) ||
        (L->num_text && !L->text_indices))
      return MINIH3_E_ARG;
  }
  return MINIH3_OK;
}

struct Workspace {
  void *a, *qkvh, *qn, *kn, *vt, *o, *xmid, *xping;
  float* rope;    // bf16: [S, 3 rope_freq_dim] (cos, sin) of every rotation pair of every row
  int8_t* qx;     // rotated W8A8: int8 codes of a projection's input rows
  float* sx;      // and their scales
  void* lora_t;   // unmerged adapters: lora_scale * x A^T of one projection [M, rank]
  uint64_t* masks;
  void* attn_scratch;
  int32_t *list_real, *list_pad, *meta, *counts, *npad;
  uint32_t* err;
  size_t total;
};

// Attention scratch: tile masks and lists, then the kernels' own scratch.
size_t tiles_bytes(int B, int S, int H, int32_t** list_real, int32_t** list_pad, int32_t** meta, uint64_t** masks,
                   void** scratch, char* base) {
  const size_t nt = (size_t)(S + 63) / 64;
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t o = off;
    off += align_up(n);
    return base ? base + o : nullptr;
  };
  char* p;
  p = take(48 * nt);  // per-tile masks, then the masks of each list entry (two lists)
  if (masks) *masks = (uint64_t*)p;
  p = take(4 * nt);
  if (list_real) *list_real = (int32_t*)p;
  p = take(4 * nt);
  if (list_pad) *list_pad = (int32_t*)p;
  p = take(16);
  if (meta) *meta = (int32_t*)p;
  p = take(attention_scratch_bytes(B, S, H));
  if (scratch) *scratch = p;
  return off;
}

Workspace carve(const minih3_config* c, int B, int S, char* base, bool w8a8 = false, int lora_rank = 0) {
  Workspace w{};
  const size_t e = act_size(c->act_dtype);
  const size_t D = c->hidden, H = c->num_heads, hd = c->head_dim, F = c->ffn_dim;
  const size_t Wd = H * hd;
  const size_t M = (size_t)B * S;
  const size_t Sp = (size_t)(S + 63) / 64 * 64;
  size_t off = 0;
  auto take = [&](size_t n) -> char* {
    size_t o = off;
    off += align_up(n);
    return base ? base + o : nullptr;
  };
  w.a = take(M * D * e);
  w.qkvh = take(M * (3 * Wd > F ? 3 * Wd : F) * e);
  w.qn = take((size_t)B * H * Sp * hd * e);
  w.kn = take((size_t)B * H * Sp * hd * e);
  w.vt = take((size_t)B * H * Sp * hd * e);
  w.o = take(M * Wd * e);
  w.xmid = take(M * D * 4);   // fp32 residual stream
  w.xping = take(M * D * 4);
  char* tb = take(tiles_bytes(B, S, (int)H, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr));
  if (base) tiles_bytes(B, S, (int)H, &w.list_real, &w.list_pad, &w.meta, &w.masks, &w.attn_scratch, tb);
  w.counts = (int32_t*)take(4 * (size_t)S);
  w.npad = (int32_t*)take(4);
  w.err = (uint32_t*)take(4);
  if (c->act_dtype == MINIH3_BF16) w.rope = (float*)take((size_t)S * 3 * c->rope_freq_dim * 8);
  if (w8a8) {
    const size_t kmax = D > Wd ? (D > F ? D : F) : (Wd > F ? Wd : F);
    w.qx = (int8_t*)take(M * kmax);
    w.sx = (float*)take(4 * M);
  }
  if (lora_rank > 0) w.lora_t = take(M * (size_t)lora_rank * e);
  w.total = off;
  return w;
}

int status_from_err(uint32_t err) {
  if (err & kErrTag) return MINIH3_E_LAYOUT_TAG;
  if (err & kErrTval) return MINIH3_E_LAYOUT_TVAL;
  if (err & kErrIndex) return MINIH3_E_LAYOUT_INDEX;
  if (err & kErrPad) return MINIH3_E_LAYOUT_PAD;
  if (err & kErrNeedsMask) return MINIH3_E_NEEDS_MASK;
  return MINIH3_OK;
}

#define HIPCHECK(x)                               \
  do {                                            \
    if ((x) != hipSuccess) return MINIH3_E_HIP;   \
  } while (0)

// One block after another. With qblocks (bf16 only) every projection runs on
// rotated W8A8: its bf16 input rows are rotated and quantized into w.qx /
// w.sx, and the int8 kernel applies the same fused epilogue.
template <typename T>
int run_blocks(const minih3_config* c, const minih3_layout* L, const minih3_block_weights* blocks, int nb,
               const T* x_in, T* x_out, Workspace& w, uint32_t flags, minih3_taps* taps, hipStream_t st,
               const minih3_block_weights_w8a8* qblocks = nullptr, const minih3_block_lora* loras = nullptr,
               int lora_rank = 0, float lora_scale = 0.f) {
  const int B = L->batch, S = L->seq_len;
  const int D = c->hidden, H = c->num_heads, hd = c->head_dim, F = c->ffn_dim;
  const int Wd = H * hd;
  const int M = B * S;
  const int Sp = (S + 63) / 64 * 64;
  const bool prof = flags & MINIH3_PROFILE;
  const int padless = (flags & MINIH3_ASSUME_PADLESS) ? 1 : 0;
  const size_t e = sizeof(T);

  const int fd = c->rope_freq_dim;
  {
    Timed tm(prof, kKTiles, st);
    HIPCHECK(launch_attn_tiles(L->token_tags, S, padless, w.masks, w.list_real, w.list_pad, w.meta, st));
    if (sizeof(T) == 2) {
      // bf16: the QKV projection normalizes and rotates q and k itself; the
      // rotary table is built once per call, and the rows past S of the
      // per-head buffers (never written by it) are cleared once
      if (fd > 0) HIPCHECK(launch_rope_table(L->position_ids, w.rope, S, fd, c->rope_theta, st));
      HIPCHECK(launch_qk_tail_zero((bf16_t*)w.qn, (bf16_t*)w.kn, (bf16_t*)w.vt, B * H, S, Sp, st));
    }
  }

  T* a = (T*)w.a;
  T* qkv = (T*)w.qkvh;
  T* hbuf = (T*)w.qkvh;  // the SwiGLU output reuses the QKV buffer
  T *qn = (T*)w.qn, *kn = (T*)w.kn, *vt = (T*)w.vt, *o = (T*)w.o;
  // The residual stream stays fp32 between the block's two gated adds and
  // between blocks; only x_out is rounded to the activation type.
  float *xmid = (float*)w.xmid, *ping = (float*)w.xping;
  const float scale = 1.f / sqrtf((float)hd);

  const void* src = x_in;
  bool src_f32 = sizeof(T) == 4;
  for (int i = 0; i < nb; ++i) {
    minih3_block_weights bw{};
    if (qblocks) {
      bw.q_norm = qblocks[i].q_norm;
      bw.k_norm = qblocks[i].k_norm;
      bw.adaln_table = qblocks[i].adaln_table;
    } else {
      bw = blocks[i];
    }
    // C = A . W^T with epilogue `epi`; `which` picks the weight (0 qkv, 1 out, 2 gate/up, 3 down)
    // With quantized set, A's rows are already rotated and quantized in
    // w.qx / w.sx (by the AdaLN kernel).
    auto proj = [&](int epi, const T* A, int which, void* C, int N, int K, EpiArgs& ea,
                    bool quantized = false) -> hipError_t {
      if (loras) {
        // unmerged adapter: t = lora_scale * A . La^T, then [A | t] . [W | B]^T
        const minih3_block_lora& lb = loras[i];
        const void* La = which == 0 ? lb.a_qkv : which == 1 ? lb.a_out : which == 2 ? lb.a_gate_up : lb.a_down;
        const void* Pw =
            which == 0 ? lb.packed_qkv : which == 1 ? lb.packed_out : which == 2 ? lb.packed_gate_up : lb.packed_down;
        EpiArgs et{};
        et.scale = lora_scale;
        hipError_t r = launch_gemm<T>(kEpiStoreScaled, A, (const T*)La, w.lora_t, M, lora_rank, K, et, st);
        if (r != hipSuccess) return r;
        EpiArgs e2 = ea;
        e2.a2 = w.lora_t;
        e2.k2 = lora_rank;
        return launch_gemm<T>(epi, A, (const T*)Pw, C, M, N, K + lora_rank, e2, st);
      }
      if (!qblocks) {
        const void* W = which == 0 ? bw.w_qkv : which == 1 ? bw.w_out : which == 2 ? bw.w_gate_up : bw.w_down;
        return launch_gemm<T>(epi, A, (const T*)W, C, M, N, K, ea, st);
      }
      const minih3_block_weights_w8a8& qb = qblocks[i];
      const int8_t* QW = which == 0 ? qb.q_qkv : which == 1 ? qb.q_out : which == 2 ? qb.q_gate_up : qb.q_down;
      const float* SW = which == 0 ? qb.s_qkv : which == 1 ? qb.s_out : which == 2 ? qb.s_gate_up : qb.s_down;
      if (!quantized) {
        hipError_t r = launch_rot_quant<bf16_t>(reinterpret_cast<const bf16_t*>(A), M, K, w.qx, w.sx, st);
        if (r != hipSuccess) return r;
      }
      ea.row_scale = w.sx;
      ea.col_scale = SW;
      hipError_t r = launch_gemm_i8(epi, w.qx, QW, C, M, N, K, ea, st);
      ea.row_scale = ea.col_scale = nullptr;
      return r;
    };
    const bool last = i == nb - 1;
    void* dst = last ? (void*)x_out : (void*)ping;  // ping may be src: src is consumed before dst is written
    const bool tap = taps && i == 0;
    EpiArgs ea{};
    ea.table = bw.adaln_table;
    ea.tags = L->token_tags;
    ea.tidx = L->timestep_indices;
    ea.S = S;
    ea.num_tags = c->num_tags;
    ea.num_tvals = c->num_tvals;
    ea.ffn_dim = F;

    // W8A8: the AdaLN kernels write the rotated int8 rows the next
    // projection reads (unless the bf16 rows are asked for as a tap)
    const bool fuse_q1 = qblocks && D % 128 == 0 && D <= 8192 && !(tap && taps->adaln1);
    const bool fuse_q2 = qblocks && D % 128 == 0 && D <= 8192 && !(tap && taps->adaln2);
    {
      Timed tm(prof, kKAdaLN1, st);
      if (fuse_q1)
        HIPCHECK(launch_adaln_rq(src, src_f32, w.qx, w.sx, bw.adaln_table, L->token_tags, L->timestep_indices, B, S,
                                 D, 0, c->norm_eps, c->num_tags, c->num_tvals, st));
      else
        HIPCHECK(launch_adaln<T>(src, src_f32, a, bw.adaln_table, L->token_tags, L->timestep_indices, B, S, D, 0,
                                 c->norm_eps, c->num_tags, c->num_tvals, st));
    }
    if (tap && taps->adaln1) HIPCHECK(hipMemcpyAsync(taps->adaln1, a, (size_t)M * D * e, hipMemcpyDeviceToDevice, st));
    if (sizeof(T) == 2) {
      // q/k RMSNorm + RoPE, the key norms and the v transpose in the
      // projection's epilogue
      Timed tm(prof, kKQKV, st);
      float* kmax = static_cast<float*>(w.attn_scratch);
      HIPCHECK(launch_zero_f32(kmax, 2 * B * H, st));
      EpiArgs eq = ea;
      eq.q_out = qn;
      eq.k_out = kn;
      eq.vt_out = vt;
      eq.q_norm = bw.q_norm;
      eq.k_norm = bw.k_norm;
      eq.rope = w.rope;
      eq.rope_pairs = 3 * fd;
      eq.heads = H;
      eq.stride = Sp;
      eq.qk_eps = c->qk_norm_eps;
      eq.kmax = kmax;
      eq.masks = w.masks;
      HIPCHECK(proj(kEpiQKRope, a, 0, nullptr, 3 * Wd, D, eq, fuse_q1));
    } else {
      {
        Timed tm(prof, kKQKV, st);
        HIPCHECK(proj(kEpiStore, a, 0, qkv, 3 * Wd, D, ea));
      }
      Timed tm(prof, kKQKNormRope, st);
      HIPCHECK(launch_qk_norm_rope<T>(qkv, bw.q_norm, bw.k_norm, L->position_ids, qn, kn, vt, B, S, H, Sp,
                                      c->rope_freq_dim, c->rope_theta, c->qk_norm_eps, st, nullptr, nullptr));
    }
    if (tap) {
      const size_t hb = (size_t)B * H * Sp * hd * e;
      if (taps->q_rot) HIPCHECK(hipMemcpyAsync(taps->q_rot, qn, hb, hipMemcpyDeviceToDevice, st));
      if (taps->k_rot) HIPCHECK(hipMemcpyAsync(taps->k_rot, kn, hb, hipMemcpyDeviceToDevice, st));
      if (taps->v_t) HIPCHECK(hipMemcpyAsync(taps->v_t, vt, hb, hipMemcpyDeviceToDevice, st));
    }
    {
      Timed tm(prof, kKAttention, st);
      HIPCHECK(launch_attention<T>(qn, kn, vt, o, w.masks, w.list_real, w.list_pad, w.meta, w.attn_scratch, B, S, H,
                                   Sp, scale, st));
    }
    if (tap && taps->attn_o) HIPCHECK(hipMemcpyAsync(taps->attn_o, o, (size_t)M * Wd * e, hipMemcpyDeviceToDevice, st));
    if (tap && taps->attn_proj) HIPCHECK(proj(kEpiStore, o, 1, taps->attn_proj, D, Wd, ea));
    {
      Timed tm(prof, kKOutProj, st);
      ea.resid = src;
      ea.resid_f32 = src_f32;
      ea.out_f32 = 1;
      ea.gate_slot = 2;
      HIPCHECK(proj(kEpiGatedResid, o, 1, xmid, D, Wd, ea));
    }
    if (tap && taps->x_mid) HIPCHECK(hipMemcpyAsync(taps->x_mid, xmid, (size_t)M * D * 4, hipMemcpyDeviceToDevice, st));
    {
      Timed tm(prof, kKAdaLN2, st);
      if (fuse_q2)
        HIPCHECK(launch_adaln_rq(xmid, true, w.qx, w.sx, bw.adaln_table, L->token_tags, L->timestep_indices, B, S, D,
                                 1, c->norm_eps, c->num_tags, c->num_tvals, st));
      else
        HIPCHECK(launch_adaln<T>(xmid, true, a, bw.adaln_table, L->token_tags, L->timestep_indices, B, S, D, 1,
                                 c->norm_eps, c->num_tags, c->num_tvals, st));
    }
    if (tap && taps->adaln2) HIPCHECK(hipMemcpyAsync(taps->adaln2, a, (size_t)M * D * e, hipMemcpyDeviceToDevice, st));
    {
      Timed tm(prof, kKGateUp, st);
      HIPCHECK(proj(kEpiSwiGLU, a, 2, hbuf, 2 * F, D, ea, fuse_q2));
    }
    if (tap && taps->ffn_h) HIPCHECK(hipMemcpyAsync(taps->ffn_h, hbuf, (size_t)M * F * e, hipMemcpyDeviceToDevice, st));
    if (tap && taps->ffn_out) HIPCHECK(proj(kEpiStore, hbuf, 3, taps->ffn_out, D, F, ea));
    {
      Timed tm(prof, kKDown, st);
      ea.resid = xmid;
      ea.resid_f32 = 1;
      ea.out_f32 = last ? (sizeof(T) == 4) : 1;
      ea.gate_slot = 5;
      HIPCHECK(proj(kEpiGatedResid, hbuf, 3, dst, D, F, ea));
    }
    if (tap && taps->block_out) {
      // the fp32 residual stream after the first block: the chain's own
      // buffer, or (when x_out holds the rounded result) the same epilogue
      // run again with an fp32 destination
      if (!last || sizeof(T) == 4) {
        HIPCHECK(hipMemcpyAsync(taps->block_out, dst, (size_t)M * D * 4, hipMemcpyDeviceToDevice, st));
      } else {
        ea.out_f32 = 1;
        HIPCHECK(proj(kEpiGatedResid, hbuf, 3, taps->block_out, D, F, ea));
      }
    }
    src = dst;
    src_f32 = !last || sizeof(T) == 4;
  }
  return MINIH3_OK;
}

LayoutDev make_layout_dev(const minih3_config* c, const minih3_layout* L) {
  LayoutDev d{};
  d.S = L->seq_len;
  d.tags = L->token_tags;
  d.tidx = L->timestep_indices;
  d.pos = L->position_ids;
  d.idx[0] = L->video_indices;
  d.idx[1] = L->audio_indices;
  d.idx[2] = L->text_indices;
  d.n_idx[0] = L->num_video;
  d.n_idx[1] = L->num_audio;
  d.n_idx[2] = L->num_text;
  d.want_tag[0] = c->tag_video;
  d.want_tag[1] = c->tag_audio;
  d.want_tag[2] = c->tag_text;
  d.num_tags = c->num_tags;
  d.num_tvals = c->num_tvals;
  return d;
}


// ---- timestep conditioning ----
constexpr int kTimeSplits = 16;  // K splits of the timestep MLP's second layer

int check_time_config(const minih3_time_config* tc) {
  if (!tc) return MINIH3_E_ARG;
  if (tc->freq_dim < 32 || tc->freq_dim % 32 != 0) return MINIH3_E_UNSUPPORTED;
  if (tc->hidden_dim < 16 || tc->hidden_dim % 16 != 0) return MINIH3_E_UNSUPPORTED;
  if (tc->embed_dim < 16 || tc->embed_dim % 16 != 0) return MINIH3_E_UNSUPPORTED;
  if (!(tc->max_period > 0.f)) return MINIH3_E_ARG;
  return MINIH3_OK;
}

struct TimeWorkspace {
  float *s[2], *h[2], *part[2], *u1[2], *u2[2];
  size_t total;
};

// Per chain (base, endpoint): the sinusoid and the hidden activations in
// fragment order, and the split-K partial sums of the second layer; with
// adapters of rank R also each layer's scaled low-rank input (fragment order).
TimeWorkspace carve_time(const minih3_time_config* tc, int M, char* base, int rank = 0) {
  TimeWorkspace w{};
  const int Kl2 = tc->hidden_dim + rank;  // contraction of the second layer
  const size_t sb = align_up((size_t)padded_rows(M) * tc->freq_dim * 4);
  const size_t hb = align_up((size_t)padded_rows(M) * tc->hidden_dim * 4);
  const size_t pb = align_up((size_t)skinny_splits(Kl2, kTimeSplits) * M * tc->embed_dim * 4);
  const size_t ub = rank > 0 ? align_up((size_t)padded_rows(M) * rank * 4) : 0;
  size_t off = 0;
  auto take = [&](size_t n) {
    float* p = base ? (float*)(base + off) : nullptr;
    off += n;
    return p;
  };
  for (int c = 0; c < 2; ++c) {
    w.s[c] = take(sb);
    w.h[c] = take(hb);
    w.part[c] = take(pb);
    if (rank > 0) {
      w.u1[c] = take(ub);
      w.u2[c] = take(ub);
    }
  }
  w.total = off;
  return w;
}

// The timestep MLP over M timesteps, with the endpoint MLP on r alongside it
// when `ep` is set (one launch per layer for both); emb = E(t), or the blend
// (1 - gate) E(t) + gate E'(r). With adapters (la, and lep for the endpoint
// MLP) each layer runs unmerged: u = ls * A x, then [x | u] . [W | B]^T
// (the packed matrices replace w1 and w2; the biases stay).
int time_mlps(const minih3_time_config* tc, const minih3_time_mlp* m, const float* t, const minih3_time_mlp* ep,
              const float* r, float gate, int M, float* emb, TimeWorkspace& w, hipStream_t st,
              const minih3_time_mlp_lora* la = nullptr, const minih3_time_mlp_lora* lep = nullptr, int rank = 0,
              float ls = 0.f) {
  const int F = tc->freq_dim, Hd = tc->hidden_dim, E = tc->embed_dim;
  const int chains = ep ? 2 : 1;
  const int R = la ? rank : 0;
  HIPCHECK(launch_sinusoid(t, ep ? r : nullptr, w.s[0], w.s[1], M, F, tc->max_period, st));
  SkinnyArgs l1{{w.s[0], w.s[1]}, {m->w1, ep ? ep->w1 : nullptr}, {m->b1, ep ? ep->b1 : nullptr}, {w.h[0], w.h[1]}};
  if (R) {
    SkinnyArgs u{{w.s[0], w.s[1]}, {la->a1, ep ? lep->a1 : nullptr}, {nullptr, nullptr}, {w.u1[0], w.u1[1]}};
    u.scale = ls;
    HIPCHECK(launch_skinny_f32(kFragToFrag, u, chains, M, R, F, 1, R, 0, st));
    l1.w[0] = la->packed1;
    l1.w[1] = ep ? lep->packed1 : nullptr;
    l1.x2[0] = w.u1[0];
    l1.x2[1] = w.u1[1];
    l1.k2 = R;
  }
  HIPCHECK(launch_skinny_f32(kFragToFrag, l1, chains, M, Hd, F + R, 1, Hd, 1, st));
  const int splits = skinny_splits(Hd + R, kTimeSplits);  // what the launch below uses
  SkinnyArgs l2{{w.h[0], w.h[1]}, {m->w2, ep ? ep->w2 : nullptr}, {nullptr, nullptr}, {w.part[0], w.part[1]}};
  if (R) {
    SkinnyArgs u{{w.h[0], w.h[1]}, {la->a2, ep ? lep->a2 : nullptr}, {nullptr, nullptr}, {w.u2[0], w.u2[1]}};
    u.scale = ls;
    HIPCHECK(launch_skinny_f32(kFragToFrag, u, chains, M, R, Hd, 1, R, 0, st));
    l2.w[0] = la->packed2;
    l2.w[1] = ep ? lep->packed2 : nullptr;
    l2.x2[0] = w.u2[0];
    l2.x2[1] = w.u2[1];
    l2.k2 = R;
  }
  HIPCHECK(launch_skinny_f32(kFragToRows, l2, chains, M, E, Hd + R, kTimeSplits, E, 0, st));
  HIPCHECK(launch_rows_finish(w.part[0], ep ? w.part[1] : nullptr, splits, m->b2, ep ? ep->b2 : nullptr, emb, M, E,
                              0, gate, st));
  return MINIH3_OK;
}


// ---- model edges ----
int check_edges(const minih3_config* c, const minih3_edges* e) {
  if (!c || !e) return MINIH3_E_ARG;
  if (c->act_dtype != MINIH3_BF16 && c->act_dtype != MINIH3_F32) return MINIH3_E_ARG;
  if (c->hidden < 256 || c->hidden % 256 != 0) return MINIH3_E_UNSUPPORTED;
  for (int ch : {e->video_channels, e->audio_channels})
    if (ch < 16 || ch > 128 || ch % 16 != 0 || ch == 80 || ch == 112) return MINIH3_E_UNSUPPORTED;
  if (!(e->final_norm_eps >= 0.f)) return MINIH3_E_ARG;
  if (!e->w_in || !e->b_in || !e->w_audio_in || !e->b_audio_in || !e->norm_w || !e->norm_b || !e->w_out ||
      !e->w_audio_out)
    return MINIH3_E_ARG;
  return MINIH3_OK;
}

struct EdgeWorkspace {
  int32_t *counts, *npad;
  uint32_t* err;
  float *wf, *s, *cv;  // folded heads: video rows first, then audio
  size_t total;
};

EdgeWorkspace carve_edges(const minih3_config* c, const minih3_edges* e, int S, char* base) {
  EdgeWorkspace w{};
  const size_t C = (size_t)e->video_channels + e->audio_channels;
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t o = off;
    off += align_up(n);
    return base ? base + o : nullptr;
  };
  w.counts = (int32_t*)take(4 * (size_t)S);
  w.npad = (int32_t*)take(4);
  w.err = (uint32_t*)take(4);
  w.wf = (float*)take(4 * C * c->hidden);
  w.s = (float*)take(4 * C);
  w.cv = (float*)take(4 * C);
  w.total = off;
  return w;
}

// Layout validation on the device, reported after one stream synchronisation.
int validate_layout(const minih3_config* c, const minih3_layout* L, uint32_t flags, EdgeWorkspace& w,
                    hipStream_t st) {
  LayoutDev ld = make_layout_dev(c, L);
  HIPCHECK(launch_layout_validate(ld, (flags & MINIH3_ASSUME_PADLESS) ? 1 : 0, w.counts, w.err, w.npad, nullptr,
                                  nullptr, nullptr, st));
  uint32_t err = 0;
  HIPCHECK(hipMemcpyAsync(&err, w.err, 4, hipMemcpyDeviceToHost, st));
  HIPCHECK(hipStreamSynchronize(st));
  return status_from_err(err);
}

// Shapes an unmerged adapter of rank `rank` needs on top of the plain block.
int check_lora(const minih3_config* c, const minih3_block_lora* loras, int num_blocks, int rank) {
  if (!loras) return MINIH3_OK;
  if (rank < 1) return MINIH3_E_ARG;
  if (c->act_dtype == MINIH3_BF16 ? rank % 256 != 0 : rank % 64 != 0) return MINIH3_E_UNSUPPORTED;
  for (int i = 0; i < num_blocks; ++i) {
    const minih3_block_lora& b = loras[i];
    if (!b.a_qkv || !b.packed_qkv || !b.a_out || !b.packed_out || !b.a_gate_up || !b.packed_gate_up || !b.a_down ||
        !b.packed_down)
      return MINIH3_E_ARG;
  }
  return MINIH3_OK;
}

int block_forward(const minih3_config* c, const minih3_layout* L, const minih3_block_weights* blocks,
                  const minih3_block_weights_w8a8* qblocks, int32_t num_blocks, const void* x_in, void* x_out,
                  void* workspace, size_t workspace_bytes, uint32_t flags, minih3_taps* taps, void* stream,
                  const minih3_block_lora* loras = nullptr, int lora_rank = 0, float lora_scale = 0.f) {
  int s = check_config(c);
  if (s) return s;
  const bool validate = flags & MINIH3_VALIDATE;
  s = check_layout(L, validate);
  if (s) return s;
  if (num_blocks < 1 || (!blocks && !qblocks) || !x_in || !x_out || x_in == x_out) return MINIH3_E_ARG;
  for (int i = 0; i < num_blocks; ++i) {
    if (qblocks) {
      const minih3_block_weights_w8a8& b = qblocks[i];
      if (!b.q_qkv || !b.s_qkv || !b.q_out || !b.s_out || !b.q_gate_up || !b.s_gate_up || !b.q_down || !b.s_down ||
          !b.q_norm || !b.k_norm || !b.adaln_table)
        return MINIH3_E_ARG;
    } else {
      const minih3_block_weights& b = blocks[i];
      if (!b.q_norm || !b.k_norm || !b.adaln_table) return MINIH3_E_ARG;
      if (!loras && (!b.w_qkv || !b.w_out || !b.w_gate_up || !b.w_down)) return MINIH3_E_ARG;
    }
  }
  if (loras && qblocks) return MINIH3_E_UNSUPPORTED;
  s = check_lora(c, loras, num_blocks, lora_rank);
  if (s) return s;
  if (qblocks) {
    if (c->act_dtype != MINIH3_BF16) return MINIH3_E_UNSUPPORTED;
    const long Wq = (long)c->num_heads * c->head_dim;
    if (c->hidden % 128 != 0 || Wq % 128 != 0 || c->ffn_dim % 128 != 0 || c->ffn_dim > 16384 ||
        c->hidden > 16384 || Wq > 16384)
      return MINIH3_E_UNSUPPORTED;
  }
  if (c->act_dtype == MINIH3_BF16) {
    const long rows = (long)L->batch * L->seq_len, D = c->hidden, W = (long)c->num_heads * c->head_dim;
    const long F = c->ffn_dim;
    const long R = loras ? lora_rank : 0;
    if (!gemm_fits(rows, 3 * W, D + R) || !gemm_fits(rows, D, W + R) || !gemm_fits(rows, 2 * F, D + R) ||
        !gemm_fits(rows, D, F + R))
      return MINIH3_E_UNSUPPORTED;
  }
  Workspace w = carve(c, L->batch, L->seq_len, (char*)workspace, qblocks != nullptr, loras ? lora_rank : 0);
  if (!workspace || workspace_bytes < w.total) return MINIH3_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const bool prof = flags & MINIH3_PROFILE;

  const bool int_taps = taps && (taps->table_row || taps->doc_id || taps->tile_flags || taps->num_pad);
  if (validate || int_taps) {
    LayoutDev ld = make_layout_dev(c, L);
    if (!validate) ld.n_idx[0] = ld.n_idx[1] = ld.n_idx[2] = 0;
    {
      Timed tm(prof, kKLayout, st);
      if (launch_layout_validate(ld, (flags & MINIH3_ASSUME_PADLESS) ? 1 : 0, w.counts, w.err, w.npad,
                                 taps ? taps->table_row : nullptr, taps ? taps->doc_id : nullptr,
                                 taps ? taps->tile_flags : nullptr, st) != hipSuccess)
        return MINIH3_E_HIP;
    }
    if (taps && taps->num_pad)
      HIPCHECK(hipMemcpyAsync(taps->num_pad, w.npad, 4, hipMemcpyDeviceToDevice, st));
    if (validate) {
      uint32_t err = 0;
      HIPCHECK(hipMemcpyAsync(&err, w.err, 4, hipMemcpyDeviceToHost, st));
      HIPCHECK(hipStreamSynchronize(st));
      s = status_from_err(err);
      if (s) return s;
    }
  }
  if (c->act_dtype == MINIH3_BF16)
    return run_blocks<bf16_t>(c, L, blocks, num_blocks, (const bf16_t*)x_in, (bf16_t*)x_out, w, flags, taps, st,
                              qblocks, loras, lora_rank, lora_scale);
  return run_blocks<float>(c, L, blocks, num_blocks, (const float*)x_in, (float*)x_out, w, flags, taps, st, nullptr,
                           loras, lora_rank, lora_scale);
}

// Workspace of a denoising step: the packed sequence twice (input and
// output of the chain), the velocities, the edges' and the chain's workspaces.
struct StepWorkspace {
  char *x0, *x1, *vel_v, *vel_a, *edges, *blocks;
  size_t edges_bytes, blocks_bytes, total;
};

int carve_step(const minih3_config* c, const minih3_step_weights* sw, int B, int S, int nv, int na, char* base,
               StepWorkspace& w) {
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t o = off;
    off += align_up(n);
    return base ? base + o : nullptr;
  };
  const size_t xb = (size_t)B * S * c->hidden * act_size(c->act_dtype);
  w.x0 = take(xb);
  w.x1 = take(xb);
  w.vel_v = take((size_t)B * nv * sw->edges->video_channels * 4);
  w.vel_a = take((size_t)B * na * sw->edges->audio_channels * 4);
  w.edges_bytes = carve_edges(c, sw->edges, S, nullptr).total;
  w.edges = take(w.edges_bytes);
  w.blocks_bytes = carve(c, B, S, nullptr, sw->qblocks != nullptr, sw->loras ? sw->lora_rank : 0).total;
  w.blocks = take(w.blocks_bytes);
  w.total = off;
  return MINIH3_OK;
}

int check_step(const minih3_config* c, const minih3_step_weights* sw) {
  if (!c || !sw || !sw->edges || !sw->sigma_now || !sw->sigma_next || sw->num_blocks < 1) return MINIH3_E_ARG;
  if ((sw->blocks == nullptr) == (sw->qblocks == nullptr)) return MINIH3_E_ARG;
  if (sw->loras && sw->qblocks) return MINIH3_E_UNSUPPORTED;
  int s = check_config(c);
  if (s) return s;
  return check_edges(c, sw->edges);
}

// Bytes of the packed attention entry's workspace: q, k, v^T in the kernels'
// layouts, then the tile masks and lists with the kernels' scratch.
size_t attention_packed_bytes(const minih3_config* c, int B, int S, size_t* stage_each) {
  const size_t Sp = (size_t)(S + 63) / 64 * 64;
  const size_t each = align_up((size_t)B * c->num_heads * Sp * c->head_dim * act_size(c->act_dtype));
  if (stage_each) *stage_each = each;
  return 3 * each + tiles_bytes(B, S, c->num_heads, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
}

// Attention on q, k [B, H, stride, hd] and v^T [B, H, hd, stride] (arguments
// checked by the caller); the workspace holds the tile masks and lists.
int attention_run(const minih3_config* c, const minih3_layout* L, const void* q, const void* k, const void* v_t,
                  int stride, void* out, float softmax_scale, void* workspace, size_t workspace_bytes, uint32_t flags,
                  hipStream_t st) {
  const int S = L->seq_len;
  int32_t *list_real, *list_pad, *meta;
  uint64_t* masks;
  void* scratch;
  const size_t need = tiles_bytes(L->batch, S, c->num_heads, &list_real, &list_pad, &meta, &masks, &scratch,
                                  (char*)workspace);
  if (!workspace || workspace_bytes < need) return MINIH3_E_WORKSPACE;
  const int padless = (flags & MINIH3_ASSUME_PADLESS) ? 1 : 0;
  if ((flags & MINIH3_VALIDATE) && padless) {
    HIPCHECK(launch_attn_tiles(L->token_tags, S, 0, masks, list_real, list_pad, meta, st));
    int32_t m[2] = {0, 0};
    HIPCHECK(hipMemcpyAsync(m, meta, 8, hipMemcpyDeviceToHost, st));
    HIPCHECK(hipStreamSynchronize(st));
    if (m[1] > 0) return MINIH3_E_NEEDS_MASK;
  }
  HIPCHECK(launch_attn_tiles(L->token_tags, S, padless, masks, list_real, list_pad, meta, st));
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf((float)c->head_dim);
  if (c->act_dtype == MINIH3_BF16) {
    HIPCHECK(launch_attention_prep<bf16_t>((const bf16_t*)k, masks, scratch, L->batch, S, c->num_heads, stride, st));
    HIPCHECK(launch_attention<bf16_t>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v_t, (bf16_t*)out, masks,
                                      list_real, list_pad, meta, scratch, L->batch, S, c->num_heads, stride, scale,
                                      st));
  } else {
    HIPCHECK(launch_attention<float>((const float*)q, (const float*)k, (const float*)v_t, (float*)out, masks,
                                     list_real, list_pad, meta, scratch, L->batch, S, c->num_heads, stride, scale,
                                     st));
  }
  return MINIH3_OK;
}

}  // namespace

extern "C" {

const char* minih3_status_string(int s) {
  switch (s) {
    case MINIH3_OK: return "ok";
    case MINIH3_E_ARG: return "invalid argument";
    case MINIH3_E_WORKSPACE: return "workspace missing or too small";
    case MINIH3_E_UNSUPPORTED: return "unsupported dimensions";
    case MINIH3_E_SCRATCH: return "request exceeds the fixed scratch of an allocation-free entry point";
    case MINIH3_E_LAYOUT_TAG: return "layout: tag outside {-1, 0 .. num_tags-1}";
    case MINIH3_E_LAYOUT_TVAL: return "layout: timestep index outside [0, num_tvals) on a non-padding row";
    case MINIH3_E_LAYOUT_INDEX: return "layout: index out of range, duplicated, or addressing another modality";
    case MINIH3_E_LAYOUT_PAD: return "layout: index addresses a padding row, or a non-padding row is unaddressed";
    case MINIH3_E_NEEDS_MASK: return "layout: padding rows need the masked attention path";
    case MINIH3_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* minih3_kernel_name(int32_t id) { return (id >= 0 && id < kKNumIds) ? kKernelNames[id] : nullptr; }

int minih3_workspace_bytes(const minih3_config* c, int32_t batch, int32_t seq_len, size_t* bytes) {
  int s = check_config(c);
  if (s) return s;
  if (!bytes || batch < 1 || seq_len < 1) return MINIH3_E_ARG;
  *bytes = carve(c, batch, seq_len, nullptr).total;
  return MINIH3_OK;
}

int minih3_attention_headmajor_workspace_bytes(const minih3_config* c, int32_t batch, int32_t seq_len,
                                               size_t* bytes) {
  int s = check_config_attention(c);
  if (s) return s;
  if (!bytes || seq_len < 1 || batch < 1) return MINIH3_E_ARG;
  *bytes = tiles_bytes(batch, seq_len, c->num_heads, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  return MINIH3_OK;
}

int minih3_attention_workspace_bytes(const minih3_config* c, int32_t batch, int32_t seq_len, size_t* bytes) {
  int s = check_config_attention(c);
  if (s) return s;
  if (!bytes || seq_len < 1 || batch < 1) return MINIH3_E_ARG;
  *bytes = attention_packed_bytes(c, batch, seq_len, nullptr);
  return MINIH3_OK;
}

int minih3_block_forward(const minih3_config* c, const minih3_layout* L, const minih3_block_weights* blocks,
                         int32_t num_blocks, const void* x_in, void* x_out, void* workspace, size_t workspace_bytes,
                         uint32_t flags, minih3_taps* taps, void* stream) {
  return block_forward(c, L, blocks, nullptr, num_blocks, x_in, x_out, workspace, workspace_bytes, flags, taps,
                       stream);
}

int minih3_workspace_bytes_lora(const minih3_config* c, int32_t batch, int32_t seq_len, int32_t rank, size_t* bytes) {
  int s = check_config(c);
  if (s) return s;
  if (!bytes || batch < 1 || seq_len < 1 || rank < 1) return MINIH3_E_ARG;
  *bytes = carve(c, batch, seq_len, nullptr, false, rank).total;
  return MINIH3_OK;
}

int minih3_block_forward_lora(const minih3_config* c, const minih3_layout* L, const minih3_block_weights* blocks,
                              const minih3_block_lora* loras, int32_t num_blocks, int32_t rank, float lora_scale,
                              const void* x_in, void* x_out, void* workspace, size_t workspace_bytes, uint32_t flags,
                              minih3_taps* taps, void* stream) {
  if (!loras) return MINIH3_E_ARG;
  return block_forward(c, L, blocks, nullptr, num_blocks, x_in, x_out, workspace, workspace_bytes, flags, taps, stream,
                       loras, rank, lora_scale);
}

int minih3_workspace_bytes_w8a8(const minih3_config* c, int32_t batch, int32_t seq_len, size_t* bytes) {
  int s = check_config(c);
  if (s) return s;
  if (c->act_dtype != MINIH3_BF16) return MINIH3_E_UNSUPPORTED;
  if (!bytes || batch < 1 || seq_len < 1) return MINIH3_E_ARG;
  *bytes = carve(c, batch, seq_len, nullptr, true).total;
  return MINIH3_OK;
}

int minih3_block_forward_w8a8(const minih3_config* c, const minih3_layout* L, const minih3_block_weights_w8a8* blocks,
                              int32_t num_blocks, const void* x_in, void* x_out, void* workspace,
                              size_t workspace_bytes, uint32_t flags, minih3_taps* taps, void* stream) {
  return block_forward(c, L, nullptr, blocks, num_blocks, x_in, x_out, workspace, workspace_bytes, flags, taps,
                       stream);
}

int minih3_attention_headmajor(const minih3_config* c, const minih3_layout* L, const void* q, const void* k,
                               const void* v_t, int32_t seq_stride, void* out, float softmax_scale, void* workspace,
                               size_t workspace_bytes, uint32_t flags, void* stream) {
  int s = check_config_attention(c);
  if (s) return s;
  if (!L || L->batch < 1 || L->seq_len < 1 || !L->token_tags) return MINIH3_E_ARG;
  if (!q || !k || !v_t || !out) return MINIH3_E_ARG;
  const int S = L->seq_len;
  if (seq_stride < S || seq_stride % 64 != 0) return MINIH3_E_ARG;
  if ((long)L->batch * c->num_heads * seq_stride > (1L << 31) - 1) return MINIH3_E_UNSUPPORTED;
  return attention_run(c, L, q, k, v_t, seq_stride, out, softmax_scale, workspace, workspace_bytes, flags,
                       (hipStream_t)stream);
}

int minih3_attention_packed(const minih3_config* c, const minih3_layout* L, const void* q, const void* k,
                            const void* v, void* out, float softmax_scale, void* workspace, size_t workspace_bytes,
                            uint32_t flags, void* stream) {
  int s = check_config_attention(c);
  if (s) return s;
  if (!L || L->batch < 1 || L->seq_len < 1 || !L->token_tags) return MINIH3_E_ARG;
  if (!q || !k || !v || !out || out == q || out == k || out == v) return MINIH3_E_ARG;
  const int B = L->batch, S = L->seq_len, H = c->num_heads;
  const int Sp = (S + 63) / 64 * 64;
  if ((long)B * H * Sp > (1L << 31) - 1) return MINIH3_E_UNSUPPORTED;
  size_t each = 0;
  const size_t need = attention_packed_bytes(c, B, S, &each);
  if (!workspace || workspace_bytes < need) return MINIH3_E_WORKSPACE;
  char* base = (char*)workspace;
  void *qh = base, *kh = base + each, *vt = base + 2 * each;
  hipStream_t st = (hipStream_t)stream;
  if (c->act_dtype == MINIH3_BF16)
    HIPCHECK(launch_attn_stage<bf16_t>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)qh,
                                       (bf16_t*)kh, (bf16_t*)vt, B, S, H, Sp, st));
  else
    HIPCHECK(launch_attn_stage<float>((const float*)q, (const float*)k, (const float*)v, (float*)qh, (float*)kh,
                                      (float*)vt, B, S, H, Sp, st));
  return attention_run(c, L, qh, kh, vt, Sp, out, softmax_scale, base + 3 * each, workspace_bytes - 3 * each, flags,
                       st);
}

int minih3_adaln_modulate(const minih3_config* c, const minih3_layout* L, const void* x, const float* table,
                          int32_t which, void* y, uint32_t flags, void* stream) {
  (void)flags;
  int s = check_config(c);
  if (s) return s;
  if (!L || L->batch < 1 || L->seq_len < 1 || !L->token_tags || !L->timestep_indices) return MINIH3_E_ARG;
  if (!x || !table || !y || (which != 0 && which != 1)) return MINIH3_E_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (c->act_dtype == MINIH3_BF16)
    HIPCHECK(launch_adaln<bf16_t>(x, false, (bf16_t*)y, table, L->token_tags, L->timestep_indices, L->batch,
                                  L->seq_len, c->hidden, which, c->norm_eps, c->num_tags, c->num_tvals, st));
  else
    HIPCHECK(launch_adaln<float>(x, false, (float*)y, table, L->token_tags, L->timestep_indices, L->batch,
                                 L->seq_len, c->hidden, which, c->norm_eps, c->num_tags, c->num_tvals, st));
  return MINIH3_OK;
}

int minih3_qk_norm_rope(const minih3_config* c, const minih3_layout* L, const void* qkv, const float* q_norm,
                        const float* k_norm, void* q_out, void* k_out, void* v_t_out, int32_t seq_stride,
                        void* stream) {
  int s = check_config_qk(c);
  if (s) return s;
  if (!L || L->batch < 1 || L->seq_len < 1 || !L->position_ids) return MINIH3_E_ARG;
  if (!qkv || !q_norm || !k_norm || !q_out || !k_out || !v_t_out) return MINIH3_E_ARG;
  if (seq_stride < L->seq_len || seq_stride % 64 != 0) return MINIH3_E_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (c->act_dtype == MINIH3_BF16)
    HIPCHECK(launch_qk_norm_rope<bf16_t>((const bf16_t*)qkv, q_norm, k_norm, L->position_ids, (bf16_t*)q_out,
                                         (bf16_t*)k_out, (bf16_t*)v_t_out, L->batch, L->seq_len, c->num_heads,
                                         seq_stride, c->rope_freq_dim, c->rope_theta, c->qk_norm_eps, st));
  else
    HIPCHECK(launch_qk_norm_rope<float>((const float*)qkv, q_norm, k_norm, L->position_ids, (float*)q_out,
                                        (float*)k_out, (float*)v_t_out, L->batch, L->seq_len, c->num_heads,
                                        seq_stride, c->rope_freq_dim, c->rope_theta, c->qk_norm_eps, st));
  return MINIH3_OK;
}

int minih3_linear(int32_t dtype, const void* a, const void* w, void* c, int32_t M, int32_t N, int32_t K,
                  void* stream) {
  if (!a || !w || !c || M < 1 || N < 1 || K < 1) return MINIH3_E_ARG;
  hipStream_t st = (hipStream_t)stream;
  EpiArgs ea{};
  if (dtype == MINIH3_BF16) {
    if (N % 256 != 0 || K % 64 != 0 || !gemm_fits(M, N, K)) return MINIH3_E_UNSUPPORTED;
    HIPCHECK(launch_gemm<bf16_t>(kEpiStore, (const bf16_t*)a, (const bf16_t*)w, (bf16_t*)c, M, N, K, ea, st));
  } else if (dtype == MINIH3_F32) {
    if (N % 64 != 0 || K % 16 != 0) return MINIH3_E_UNSUPPORTED;
    HIPCHECK(launch_gemm<float>(kEpiStore, (const float*)a, (const float*)w, (float*)c, M, N, K, ea, st));
  } else {
    return MINIH3_E_ARG;
  }
  return MINIH3_OK;
}

int minih3_time_embed_workspace_bytes(const minih3_time_config* tc, int32_t num_tvals, size_t* bytes) {
  int s = check_time_config(tc);
  if (s) return s;
  if (num_tvals < 1 || !bytes) return MINIH3_E_ARG;
  *bytes = carve_time(tc, num_tvals, nullptr).total;
  return MINIH3_OK;
}

int minih3_time_embed(const minih3_time_config* tc, const minih3_time_mlp* base, const float* t,
                      const minih3_time_mlp* endpoint, const float* r, float gate, int32_t num_tvals, float* emb,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int s = check_time_config(tc);
  if (s) return s;
  if (num_tvals < 1 || !base || !base->w1 || !base->w2 || !t || !emb) return MINIH3_E_ARG;
  if (endpoint && (!endpoint->w1 || !endpoint->w2)) return MINIH3_E_ARG;
  if ((long)num_tvals * tc->hidden_dim > (1L << 28) || (long)num_tvals * tc->embed_dim > (1L << 28))
    return MINIH3_E_UNSUPPORTED;
  TimeWorkspace w = carve_time(tc, num_tvals, (char*)workspace);
  if (!workspace || workspace_bytes < w.total) return MINIH3_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  return time_mlps(tc, base, t, endpoint, r ? r : t, gate, num_tvals, emb, w, st);
}

int minih3_time_embed_lora_workspace_bytes(const minih3_time_config* tc, int32_t num_tvals, int32_t rank,
                                           size_t* bytes) {
  int s = check_time_config(tc);
  if (s) return s;
  if (num_tvals < 1 || rank < 16 || rank % 16 != 0 || !bytes) return MINIH3_E_ARG;
  *bytes = carve_time(tc, num_tvals, nullptr, rank).total;
  return MINIH3_OK;
}

int minih3_time_embed_lora(const minih3_time_config* tc, const minih3_time_mlp* base,
                           const minih3_time_mlp_lora* base_lora, const float* t, const minih3_time_mlp* endpoint,
                           const minih3_time_mlp_lora* endpoint_lora, const float* r, float gate, int32_t num_tvals,
                           int32_t rank, float lora_scale, float* emb, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int s = check_time_config(tc);
  if (s) return s;
  if (num_tvals < 1 || !base || !base_lora || !t || !emb) return MINIH3_E_ARG;
  if (rank < 16 || rank % 16 != 0) return MINIH3_E_UNSUPPORTED;
  if (endpoint && !endpoint_lora) return MINIH3_E_ARG;
  for (const minih3_time_mlp_lora* l : {base_lora, endpoint ? endpoint_lora : base_lora})
    if (!l->a1 || !l->packed1 || !l->a2 || !l->packed2) return MINIH3_E_ARG;
  if ((long)num_tvals * tc->hidden_dim > (1L << 28) || (long)num_tvals * tc->embed_dim > (1L << 28))
    return MINIH3_E_UNSUPPORTED;
  TimeWorkspace w = carve_time(tc, num_tvals, (char*)workspace, rank);
  if (!workspace || workspace_bytes < w.total) return MINIH3_E_WORKSPACE;
  return time_mlps(tc, base, t, endpoint, r ? r : t, gate, num_tvals, emb, w, (hipStream_t)stream, base_lora,
                   endpoint ? endpoint_lora : nullptr, rank, lora_scale);
}

int minih3_adaln_table_workspace_bytes(const minih3_config* c, int32_t embed_dim, size_t* bytes) {
  if (!c || !bytes || c->num_tvals < 1 || embed_dim < 1) return MINIH3_E_ARG;
  *bytes = c->act_dtype == MINIH3_BF16 ? align_up((size_t)padded_rows(c->num_tvals) * embed_dim * 2) : 0;
  return MINIH3_OK;
}

int minih3_adaln_table(const minih3_config* c, const float* emb, int32_t embed_dim, const void* w_proj,
                       const void* b_proj, float* table, void* workspace, size_t workspace_bytes, void* stream) {
  if (!c || (c->act_dtype != MINIH3_BF16 && c->act_dtype != MINIH3_F32)) return MINIH3_E_ARG;
  if (c->hidden < 256 || c->hidden % 256 != 0) return MINIH3_E_UNSUPPORTED;
  if (c->num_tags < 1 || c->num_tvals < 1 || embed_dim < 1) return MINIH3_E_ARG;
  if (!emb || !w_proj || !table) return MINIH3_E_ARG;
  const long ng = 6L * c->hidden, N = ng * c->num_tags, M = c->num_tvals;
  if (N * embed_dim > (1L << 31) || M * N > (1L << 31) || M > (1L << 20)) return MINIH3_E_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (c->act_dtype == MINIH3_F32) {
    if (embed_dim % 16 != 0) return MINIH3_E_UNSUPPORTED;
    SkinnyArgs g{{emb, nullptr}, {(const float*)w_proj, nullptr}, {(const float*)b_proj, nullptr}, {table, nullptr}};
    HIPCHECK(launch_skinny_f32(kRowsSilu, g, 1, (int)M, (int)N, embed_dim, 1, (int)ng, 0, st));
    return MINIH3_OK;
  }
  if (embed_dim % 32 != 0) return MINIH3_E_UNSUPPORTED;
  const size_t need = align_up((size_t)padded_rows((int)M) * embed_dim * 2);
  if (!workspace || workspace_bytes < need) return MINIH3_E_WORKSPACE;
  HIPCHECK(launch_adaln_proj(emb, (const bf16_t*)w_proj, (const bf16_t*)b_proj, (bf16_t*)workspace, table, (int)M,
                             (int)N, embed_dim, (int)ng, st));
  return MINIH3_OK;
}


int minih3_adaln_table_noalloc(const minih3_config* c, const float* emb, int32_t embed_dim, const void* w_proj,
                               const void* b_proj, float* table, void* stream) {
  size_t need = 0;
  int s = minih3_adaln_table_workspace_bytes(c, embed_dim, &need);
  if (s) return s;
  if (need > kNoallocScratchBytes) return MINIH3_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    s = noalloc_scratch(&ws);
    if (s) return s;
  }
  return minih3_adaln_table(c, emb, embed_dim, w_proj, b_proj, table, ws, need, stream);
}

int minih3_edges_workspace_bytes(const minih3_config* c, const minih3_edges* e, int32_t seq_len, size_t* bytes) {
  int s = check_edges(c, e);
  if (s) return s;
  if (seq_len < 1 || !bytes) return MINIH3_E_ARG;
  *bytes = carve_edges(c, e, seq_len, nullptr).total;
  return MINIH3_OK;
}

int minih3_embed_inputs(const minih3_config* c, const minih3_layout* L, const minih3_edges* e, const float* video,
                        const float* audio, const void* text, void* x, void* workspace, size_t workspace_bytes,
                        uint32_t flags, void* stream) {
  int s = check_edges(c, e);
  if (s) return s;
  s = check_layout(L, true);
  if (s) return s;
  if (!x || (L->num_video && !video) || (L->num_audio && !audio) || (L->num_text && !text)) return MINIH3_E_ARG;
  EdgeWorkspace w = carve_edges(c, e, L->seq_len, (char*)workspace);
  if (!workspace || workspace_bytes < w.total) return MINIH3_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (flags & MINIH3_VALIDATE) {
    s = validate_layout(c, L, flags, w, st);
    if (s) return s;
  }
  const int B = L->batch, S = L->seq_len, D = c->hidden;
  if (c->act_dtype == MINIH3_BF16) {
    bf16_t* xo = (bf16_t*)x;
    HIPCHECK(launch_edge_in<bf16_t>(video, L->num_video, e->video_channels, e->w_in, e->b_in, L->video_indices, B, S,
                                    D, xo, st));
    HIPCHECK(launch_edge_in<bf16_t>(audio, L->num_audio, e->audio_channels, e->w_audio_in, e->b_audio_in,
                                    L->audio_indices, B, S, D, xo, st));
    HIPCHECK(launch_edge_rows<bf16_t>((const bf16_t*)text, L->text_indices, L->num_text, L->token_tags, B, S, D, xo,
                                      st));
  } else {
    float* xo = (float*)x;
    HIPCHECK(launch_edge_in<float>(video, L->num_video, e->video_channels, e->w_in, e->b_in, L->video_indices, B, S,
                                   D, xo, st));
    HIPCHECK(launch_edge_in<float>(audio, L->num_audio, e->audio_channels, e->w_audio_in, e->b_audio_in,
                                   L->audio_indices, B, S, D, xo, st));
    HIPCHECK(launch_edge_rows<float>((const float*)text, L->text_indices, L->num_text, L->token_tags, B, S, D, xo,
                                     st));
  }
  return MINIH3_OK;
}

int minih3_output_heads(const minih3_config* c, const minih3_layout* L, const minih3_edges* e, const void* x,
                        float* video_out, float* audio_out, void* workspace, size_t workspace_bytes, uint32_t flags,
                        void* stream) {
  int s = check_edges(c, e);
  if (s) return s;
  s = check_layout(L, true);
  if (s) return s;
  if (!x || (L->num_video && !video_out) || (L->num_audio && !audio_out)) return MINIH3_E_ARG;
  EdgeWorkspace w = carve_edges(c, e, L->seq_len, (char*)workspace);
  if (!workspace || workspace_bytes < w.total) return MINIH3_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (flags & MINIH3_VALIDATE) {
    s = validate_layout(c, L, flags, w, st);
    if (s) return s;
  }
  const int B = L->batch, S = L->seq_len, D = c->hidden, Cv = e->video_channels, Ca = e->audio_channels;
  float* wf_a = w.wf + (size_t)Cv * D;
  HIPCHECK(launch_edge_fold(e->w_out, e->b_out, e->norm_w, e->norm_b, Cv, D, w.wf, w.s, w.cv, st));
  HIPCHECK(launch_edge_fold(e->w_audio_out, e->b_audio_out, e->norm_w, e->norm_b, Ca, D, wf_a, w.s + Cv, w.cv + Cv,
                            st));
  // the wider head first (the kernel sizes its LDS ring by head 0)
  const int wide = Ca > Cv ? 1 : 0;
  EdgeHeads hd{};
  const int32_t* idxs[2] = {L->video_indices, L->audio_indices};
  const int nr[2] = {L->num_video, L->num_audio}, Cs[2] = {Cv, Ca};
  float* Wfs[2] = {w.wf, wf_a};
  float* outs[2] = {video_out, audio_out};
  for (int k = 0; k < 2; ++k) {
    const int h = wide ? 1 - k : k;
    hd.idx[k] = idxs[h];
    hd.nrows[k] = nr[h];
    hd.C[k] = Cs[h];
    hd.Wf[k] = Wfs[h];
    hd.s[k] = w.s + (h ? Cv : 0);
    hd.cv[k] = w.cv + (h ? Cv : 0);
    hd.y[k] = outs[h];
  }
  if (hd.nrows[0] == 0) {  // only the narrower head has rows: run it alone
    std::swap(hd.idx[0], hd.idx[1]);
    std::swap(hd.nrows[0], hd.nrows[1]);
    std::swap(hd.C[0], hd.C[1]);
    std::swap(hd.Wf[0], hd.Wf[1]);
    std::swap(hd.s[0], hd.s[1]);
    std::swap(hd.cv[0], hd.cv[1]);
    std::swap(hd.y[0], hd.y[1]);
  }
  const float eps = e->final_norm_eps;
  if (c->act_dtype == MINIH3_BF16)
    HIPCHECK(launch_edge_out<bf16_t>((const bf16_t*)x, hd, B, S, D, eps, st));
  else
    HIPCHECK(launch_edge_out<float>((const float*)x, hd, B, S, D, eps, st));
  return MINIH3_OK;
}

int minih3_rotate_quantize(int32_t dtype, const void* x, int32_t M, int32_t K, int8_t* q, float* scale,
                           void* stream) {
  if (!x || !q || !scale || M < 1 || K < 1) return MINIH3_E_ARG;
  if (K % 128 != 0 || K > 16384 || (long)M * K > (1L << 40)) return MINIH3_E_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == MINIH3_BF16)
    HIPCHECK(launch_rot_quant<bf16_t>((const bf16_t*)x, M, K, q, scale, st));
  else if (dtype == MINIH3_F32)
    HIPCHECK(launch_rot_quant<float>((const float*)x, M, K, q, scale, st));
  else
    return MINIH3_E_ARG;
  return MINIH3_OK;
}

int minih3_linear_w8a8(const int8_t* qa, const float* sa, const int8_t* qw, const float* sw, void* c, int32_t M,
                       int32_t N, int32_t K, void* stream) {
  if (!qa || !sa || !qw || !sw || !c || M < 1 || N < 1 || K < 1) return MINIH3_E_ARG;
  if (N % 256 != 0 || K % 128 != 0 || (long)M * K > 0xFFFFFFFFL || (long)N * K > 0xFFFFFFFFL)
    return MINIH3_E_UNSUPPORTED;
  EpiArgs ea{};
  ea.row_scale = sa;
  ea.col_scale = sw;
  HIPCHECK(launch_gemm_i8(kEpiStore, qa, qw, c, M, N, K, ea, (hipStream_t)stream));
  return MINIH3_OK;
}

int minih3_lora_pack_weight(int32_t dtype, const void* w, const void* lora_b, void* packed, int32_t N, int32_t K,
                            int32_t rank, void* stream) {
  if (!w || !lora_b || !packed || N < 1 || K < 1 || rank < 1) return MINIH3_E_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == MINIH3_BF16) {
    if (K % 8 != 0 || rank % 8 != 0) return MINIH3_E_UNSUPPORTED;
    HIPCHECK(launch_concat_rows<bf16_t>((const bf16_t*)w, (const bf16_t*)lora_b, 1.f, (bf16_t*)packed, N, K, rank,
                                        st));
  } else if (dtype == MINIH3_F32) {
    if (K % 4 != 0 || rank % 4 != 0) return MINIH3_E_UNSUPPORTED;
    HIPCHECK(launch_concat_rows<float>((const float*)w, (const float*)lora_b, 1.f, (float*)packed, N, K, rank, st));
  } else {
    return MINIH3_E_ARG;
  }
  return MINIH3_OK;
}

int minih3_linear_lora_workspace_bytes(int32_t dtype, int32_t M, int32_t K, int32_t rank, size_t* bytes) {
  if (!bytes || M < 1 || K < 1 || rank < 1 || (dtype != MINIH3_BF16 && dtype != MINIH3_F32)) return MINIH3_E_ARG;
  *bytes = align_up((size_t)M * rank * act_size(dtype));  // t
  return MINIH3_OK;
}

int minih3_linear_lora(int32_t dtype, const void* a, const void* lora_a, const void* packed, float lora_scale,
                       void* c, int32_t M, int32_t N, int32_t K, int32_t rank, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!a || !lora_a || !packed || !c || M < 1 || N < 1 || K < 1 || rank < 1) return MINIH3_E_ARG;
  if (dtype != MINIH3_BF16 && dtype != MINIH3_F32) return MINIH3_E_ARG;
  if (!workspace || workspace_bytes < align_up((size_t)M * rank * act_size(dtype))) return MINIH3_E_WORKSPACE;
  void* t = workspace;
  hipStream_t st = (hipStream_t)stream;
  // t = lora_scale * a A^T (stored in dtype), then one projection whose A
  // operand is [a | t] read from the two arrays, against packed = [W | B]
  EpiArgs et{};
  et.scale = lora_scale;
  EpiArgs ec{};
  ec.a2 = t;
  ec.k2 = rank;
  const int Kc = K + rank;
  if (dtype == MINIH3_BF16) {
    if (rank % 256 != 0 || N % 256 != 0 || K % 64 != 0 || !gemm_fits(M, rank, K) || !gemm_fits(M, N, Kc))
      return MINIH3_E_UNSUPPORTED;
    HIPCHECK(launch_gemm<bf16_t>(kEpiStoreScaled, (const bf16_t*)a, (const bf16_t*)lora_a, t, M, rank, K, et, st));
    HIPCHECK(launch_gemm<bf16_t>(kEpiStore, (const bf16_t*)a, (const bf16_t*)packed, c, M, N, Kc, ec, st));
  } else {
    if (rank % 64 != 0 || N % 64 != 0 || K % 16 != 0) return MINIH3_E_UNSUPPORTED;
    HIPCHECK(launch_gemm<float>(kEpiStoreScaled, (const float*)a, (const float*)lora_a, t, M, rank, K, et, st));
    HIPCHECK(launch_gemm<float>(kEpiStore, (const float*)a, (const float*)packed, c, M, N, Kc, ec, st));
  }
  return MINIH3_OK;
}

int minih3_euler_step(const float* x, const float* velocity, float* x_next, int32_t batch, int32_t num_rows,
                      int32_t channels, const int32_t* indices, const int32_t* timestep_indices, int32_t seq_len,
                      const float* sigma_now, const float* sigma_next, int32_t num_tvals, void* stream) {
  if (batch < 1 || num_rows < 0 || channels < 1 || seq_len < 1 || num_tvals < 1) return MINIH3_E_ARG;
  if (num_rows == 0) return MINIH3_OK;
  if (!x || !velocity || !x_next || !indices || !timestep_indices || !sigma_now || !sigma_next) return MINIH3_E_ARG;
  HIPCHECK(launch_euler(x, velocity, x_next, batch, num_rows, channels, indices, timestep_indices, seq_len, sigma_now,
                        sigma_next, num_tvals, (hipStream_t)stream));
  return MINIH3_OK;
}

int minih3_denoise_step_workspace_bytes(const minih3_config* c, const minih3_step_weights* sw, int32_t batch,
                                        int32_t seq_len, int32_t num_video, int32_t num_audio, size_t* bytes) {
  int s = check_step(c, sw);
  if (s) return s;
  if (!bytes || batch < 1 || seq_len < 1 || num_video < 0 || num_audio < 0) return MINIH3_E_ARG;
  StepWorkspace w{};
  carve_step(c, sw, batch, seq_len, num_video, num_audio, nullptr, w);
  *bytes = w.total;
  return MINIH3_OK;
}

int minih3_denoise_step(const minih3_config* c, const minih3_layout* L, const minih3_step_weights* sw, float* video,
                        float* audio, const void* text, void* workspace, size_t workspace_bytes, uint32_t flags,
                        void* stream) {
  int s = check_step(c, sw);
  if (s) return s;
  s = check_layout(L, true);
  if (s) return s;
  if ((L->num_video && !video) || (L->num_audio && !audio) || (L->num_text && !text)) return MINIH3_E_ARG;
  StepWorkspace w{};
  carve_step(c, sw, L->batch, L->seq_len, L->num_video, L->num_audio, (char*)workspace, w);
  if (!workspace || workspace_bytes < w.total) return MINIH3_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  s = minih3_embed_inputs(c, L, sw->edges, video, audio, text, w.x0, w.edges, w.edges_bytes, flags, stream);
  if (s) return s;
  const uint32_t bflags = flags & ~(uint32_t)MINIH3_VALIDATE;  // validated once above
  s = block_forward(c, L, sw->blocks, sw->qblocks, sw->num_blocks, w.x0, w.x1, w.blocks, w.blocks_bytes, bflags,
                    nullptr, stream, sw->loras, sw->lora_rank, sw->lora_scale);
  if (s) return s;
  s = minih3_output_heads(c, L, sw->edges, w.x1, (float*)w.vel_v, (float*)w.vel_a, w.edges, w.edges_bytes, 0, stream);
  if (s) return s;
  const int B = L->batch, S = L->seq_len;
  HIPCHECK(launch_euler(video, (const float*)w.vel_v, video, B, L->num_video, sw->edges->video_channels,
                        L->video_indices, L->timestep_indices, S, sw->sigma_now, sw->sigma_next, c->num_tvals, st));
  HIPCHECK(launch_euler(audio, (const float*)w.vel_a, audio, B, L->num_audio, sw->edges->audio_channels,
                        L->audio_indices, L->timestep_indices, S, sw->sigma_now, sw->sigma_next, c->num_tvals, st));
  return MINIH3_OK;
}

int minih3_profile_collect(double* total_ms, int32_t* launches, int32_t n) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int i = 0; i < n; ++i) {
    if (total_ms) total_ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (auto& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess && r.id < n) {
      if (total_ms) total_ms[r.id] += ms;
      if (launches) launches[r.id] += 1;
    }
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  return kKNumIds;
}

}  // extern "C"
