// Layout description and validation (integer work) and the attention tile
// lists. Follows the MiniMaxH3Transformer3DModel page: `forward` parameters
// token_tags, timestep_indices and the video/audio/text index tensors, and
// the class description's rule that padding rows (tag -1) sit in their own
// attention document.
#include "common.h"
#include "kernels.h"

namespace minih3 {

__global__ void k_layout_clear(int32_t* counts, int S, uint32_t* err, int32_t* npad, int32_t* tile_flags,
                               int ntiles) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < S) counts[i] = 0;
  if (tile_flags && i < ntiles) tile_flags[i] = 0;
  if (i == 0) {
    *err = 0u;
    *npad = 0;
  }
}

__global__ void k_layout_rows(LayoutDev L, int assume_padless, uint32_t* err, int32_t* npad, int32_t* table_row,
                              int32_t* doc_id, int32_t* tile_flags) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= L.S) return;
  int tag = L.tags[i];
  int tv = L.tidx[i];
  uint32_t e = 0;
  bool pad = tag == -1;
  if (!pad && (tag < 0 || tag >= L.num_tags)) e |= kErrTag;
  if (!pad && (tv < 0 || tv >= L.num_tvals)) e |= kErrTval;
  if (pad && assume_padless) e |= kErrNeedsMask;
  if (e) atomicOr(err, e);
  if (pad) atomicAdd(npad, 1);
  if (table_row) table_row[i] = table_row_of(tag, tv, L.num_tags, L.num_tvals);
  if (doc_id) doc_id[i] = pad ? 1 : 0;
  if (tile_flags) atomicOr(&tile_flags[i >> 6], pad ? 2 : 1);
}

__global__ void k_layout_index(LayoutDev L, int32_t* counts, uint32_t* err) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  int t = 0;
  while (t < 3 && e >= L.n_idx[t]) {
    e -= L.n_idx[t];
    ++t;
  }
  if (t >= 3) return;
  int i = L.idx[t][e];
  if (i < 0 || i >= L.S) {
    atomicOr(err, (uint32_t)kErrIndex);
    return;
  }
  atomicAdd(&counts[i], 1);
  int tag = L.tags[i];
  if (tag == -1)
    atomicOr(err, (uint32_t)kErrPad);
  else if (tag != L.want_tag[t])
    atomicOr(err, (uint32_t)kErrIndex);
}

__global__ void k_layout_cover(LayoutDev L, const int32_t* counts, uint32_t* err) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= L.S) return;
  int c = counts[i];
  if (c > 1) atomicOr(err, (uint32_t)kErrIndex);
  if (c == 0 && L.tags[i] != -1) atomicOr(err, (uint32_t)kErrPad);
}

hipError_t launch_layout_validate(const LayoutDev& L, int assume_padless, int32_t* counts, uint32_t* err,
                                  int32_t* npad, int32_t* table_row, int32_t* doc_id, int32_t* tile_flags,
                                  hipStream_t st) {
  const int tb = 256;
  int ntiles = (L.S + 63) / 64;
  int nclear = L.S > ntiles ? L.S : ntiles;
  k_layout_clear<<<(nclear + tb - 1) / tb, tb, 0, st>>>(counts, L.S, err, npad, tile_flags, ntiles);
  k_layout_rows<<<(L.S + tb - 1) / tb, tb, 0, st>>>(L, assume_padless, err, npad, table_row, doc_id, tile_flags);
  int nidx = L.n_idx[0] + L.n_idx[1] + L.n_idx[2];
  if (nidx > 0) k_layout_index<<<(nidx + tb - 1) / tb, tb, 0, st>>>(L, counts, err);
  k_layout_cover<<<(L.S + tb - 1) / tb, tb, 0, st>>>(L, counts, err);
  return hipGetLastError();
}

// One workgroup of 1024 threads builds, for the 64-row tiles of the
// sequence, the masks of non-padding and padding rows and the ordered
// lists of tiles that hold at least one row of each document.
__global__ void __launch_bounds__(1024) k_attn_tiles(const int32_t* tags, int S, int assume_padless,
                                                     uint64_t* masks, int32_t* list_real, int32_t* list_pad,
                                                     int32_t* meta) {
  __shared__ int wave_tot[2][16];
  __shared__ int base[2];
  const int ntiles = (S + 63) / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) base[0] = base[1] = 0;
  __syncthreads();
  for (int t0 = 0; t0 < ntiles; t0 += 1024) {
    int t = t0 + threadIdx.x;
    uint64_t mr = 0, mp = 0;
    if (t < ntiles) {
      int r0 = t * 64;
      int n = S - r0 < 64 ? S - r0 : 64;
      for (int k = 0; k < n; ++k) {
        bool pad = !assume_padless && tags[r0 + k] == -1;
        if (pad)
          mp |= 1ull << k;
        else
          mr |= 1ull << k;
      }
      masks[2 * t] = mr;
      masks[2 * t + 1] = mp;
    }
    uint64_t br = __ballot(mr != 0), bp = __ballot(mp != 0);
    uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int pr = __popcll(br & below), pp = __popcll(bp & below);
    if (lane == 0) {
      wave_tot[0][wid] = __popcll(br);
      wave_tot[1][wid] = __popcll(bp);
    }
    __syncthreads();
    int offr = base[0], offp = base[1];
    for (int w = 0; w < wid; ++w) {
      offr += wave_tot[0][w];
      offp += wave_tot[1][w];
    }
    // the masks of each listed tile again, aligned with the list (records
    // [2 ntiles, 4 ntiles) for the non-padding list, [4 ntiles, 6 ntiles)
    // for the padding list), so a walk over a list reads them with its entries
    if (mr) {
      list_real[offr + pr] = t;
      masks[2 * ntiles + 2 * (offr + pr)] = mr;
      masks[2 * ntiles + 2 * (offr + pr) + 1] = mp;
    }
    if (mp) {
      list_pad[offp + pp] = t;
      masks[4 * ntiles + 2 * (offp + pp)] = mr;
      masks[4 * ntiles + 2 * (offp + pp) + 1] = mp;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 0; w < 16; ++w) {
        base[0] += wave_tot[0][w];
        base[1] += wave_tot[1][w];
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    meta[0] = base[0];
    meta[1] = base[1];
  }
}

hipError_t launch_attn_tiles(const int32_t* tags, int S, int assume_padless, uint64_t* masks, int32_t* list_real,
                             int32_t* list_pad, int32_t* meta, hipStream_t st) {
  k_attn_tiles<<<1, 1024, 0, st>>>(tags, S, assume_padless, masks, list_real, list_pad, meta);
  return hipGetLastError();
}

}  // namespace minih3
