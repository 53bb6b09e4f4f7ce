// Staging of the attention boundary: packed q, k, v [B, S, H, 128] into the
// layouts the attention kernels read (q, k head-major [B, H, stride, 128],
// v transposed [B, H, 128, stride]), rows past S as zeros.
//
// Page "MiniMaxH3Transformer3DModel", `forward`: the block takes one packed
// sequence, rows in packed order; the attention entry point of the library
// accepts q, k, v in that order and turns them here into the per-head
// layouts of csrc/attention.hip, in the caller's workspace.
#include "common.h"
#include "kernels.h"

namespace minih3 {

constexpr int kKV = 64;   // rows per workgroup: one key tile of the attention kernels
constexpr int HD = 128;

// Packed q, k, v [B, S, H, 128] into the layouts above. One workgroup per 64
// rows of one head: q and k rows move as 16-byte chunks (a row of a head is
// one contiguous run on both sides); v goes through LDS, where the 64 x 128
// block is turned, so that each channel leaves as one contiguous run of its
// v^T row. Rows past S are zeros.
template <typename T>
__global__ void __launch_bounds__(256) k_attn_stage(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, T* __restrict__ qh, T* __restrict__ kh,
                                                    T* __restrict__ vt, int S, int H, int stride) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = HD / EPC;        // chunks per row of a head
  typedef u32x4 chunk_t;
  __shared__ T tv[HD][kKV + EPC];      // v block, channel-major
  const int s0 = blockIdx.x * kKV, h = blockIdx.y, b = blockIdx.z;
  const long src_row = (long)H * HD;   // elements between consecutive rows of the packed inputs
  const long head = (long)b * H + h;
  for (int c = threadIdx.x; c < kKV * CPR; c += 256) {
    const int r = c / CPR, cc = c % CPR, s = s0 + r;
    chunk_t zq = {0u, 0u, 0u, 0u}, zk = zq, zv = zq;
    if (s < S) {
      const long off = ((long)b * S + s) * src_row + (long)h * HD + cc * EPC;
      zq = *reinterpret_cast<const chunk_t*>(q + off);
      zk = *reinterpret_cast<const chunk_t*>(k + off);
      zv = *reinterpret_cast<const chunk_t*>(v + off);
    }
    const long dst = (head * stride + s) * HD + cc * EPC;
    *reinterpret_cast<chunk_t*>(qh + dst) = zq;
    *reinterpret_cast<chunk_t*>(kh + dst) = zk;
    const T* e = reinterpret_cast<const T*>(&zv);
#pragma unroll
    for (int i = 0; i < EPC; ++i) tv[cc * EPC + i][r] = e[i];
  }
  __syncthreads();
  constexpr int RPC = kKV / EPC;  // chunks per 64-key run of a v^T row
  for (int c = threadIdx.x; c < HD * RPC; c += 256) {
    const int d = c / RPC, j = c % RPC;
    chunk_t o;
    T* e = reinterpret_cast<T*>(&o);
#pragma unroll
    for (int i = 0; i < EPC; ++i) e[i] = tv[d][j * EPC + i];
    *reinterpret_cast<chunk_t*>(vt + (head * HD + d) * stride + s0 + j * EPC) = o;
  }
}

template <typename T>
hipError_t launch_attn_stage(const T* q, const T* k, const T* v, T* qh, T* kh, T* vt, int B, int S, int H, int stride,
                             hipStream_t st) {
  if (B < 1 || S < 1 || H < 1 || stride < S || stride % kKV != 0) return hipErrorInvalidValue;
  k_attn_stage<T><<<dim3((unsigned)(stride / kKV), (unsigned)H, (unsigned)B), 256, 0, st>>>(q, k, v, qh, kh, vt, S,
                                                                                          H, stride);
  return hipGetLastError();
}
template hipError_t launch_attn_stage<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*, bf16_t*, bf16_t*,
                                              int, int, int, int, hipStream_t);
template hipError_t launch_attn_stage<float>(const float*, const float*, const float*, float*, float*, float*, int,
                                             int, int, int, hipStream_t);

}  // namespace minih3
