// Compact TwELL: capacity W < 64 slots per (row, tile) instead of 64.
//
// [IN] "Слитые CUDA-ядра для инференса и гибрид для обучения": training keeps
// the well-sparse rows in a compact sparse matrix and sends rows with many
// active values to a dense branch; [GE] / [GI] paragraph 1 report lower peak
// memory.  With a fixed capacity W, tile (i, j) sits at (i*NT + j)*W*16 and
// needs no offset table; a row with more than W non-zeros in some tile is
// flagged (ovf) and the backward sends it to the dense branch, which
// recomputes its activations from x.  The saved state between a layer's
// forward and backward shrinks from T*F*5 bytes of values and indices to
// T*F*5*W/64 (plus the per-(row, tile) counts and masks).
#include "common.hpp"
#include "internal.hpp"

namespace twell {

// One wave per tile: the first min(width, W) slots (16 rows each) move
// between the capacity-64 and the capacity-W layouts.
template <bool EXPAND>
__global__ __launch_bounds__(256) void compact_tiles_kernel(CompactArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= a.ntiles) return;
  const int w = min(EXPAND ? (int)a.cwidth[tile] : (int)a.width[tile], a.W);
  if (lane == 0) {
    if (!EXPAND) a.cwidth[tile] = (uint8_t)w;
    else if (a.width != a.cwidth) a.width[tile] = (uint8_t)w;
  }
  const int64_t fb = tile * (64 * 16), cb = tile * ((int64_t)a.W * 16);
  for (int e = lane; e < w * 16; e += 64) {
    if (EXPAND) {
      a.val[fb + e] = a.cval[cb + e];
      a.idx[fb + e] = a.cidx[cb + e];
    } else {
      a.cval[cb + e] = a.val[fb + e];
      a.cidx[cb + e] = a.idx[fb + e];
    }
  }
}

// One wave per row: counts and masks move over; compacting also flags the
// rows with a tile count above W.
template <bool EXPAND>
__global__ __launch_bounds__(256) void compact_rows_kernel(CompactArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  bool over = false;
  for (int j = lane; j < a.NT; j += 64) {
    const int64_t o = (int64_t)t * a.NT + j;
    if (EXPAND) {
      a.cnt[o] = a.ccnt[o];
      a.mask[o] = a.cmask[o];
    } else {
      const uint8_t c = a.cnt[o];
      a.ccnt[o] = c;
      a.cmask[o] = a.mask[o];
      over |= c > a.W;
    }
  }
  const uint64_t any = ballot(over);
  if (!EXPAND && lane == 0) a.ovf[t] = any ? 1 : 0;
}

// After a gate GEMM that packed straight into the capacity-W arrays (the
// epilogue keeps the first W slots of every tile and records the true counts
// and widths): the overflow flag of every row, and each tile's width clamped
// to W, the convention of the compact form.  Workgroups [0, nrow) take four
// rows each, the rest 256 tiles each.
__global__ __launch_bounds__(256) void compact_finish_kernel(CompactArgs a, int nrow) {
  if ((int)blockIdx.x < nrow) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    bool over = false;
    for (int j = lane; j < a.NT; j += 64) over |= a.ccnt[(int64_t)t * a.NT + j] > a.W;
    const uint64_t any = ballot(over);
    if (lane == 0) a.ovf[t] = any ? 1 : 0;
  } else {
    const int64_t tile = (int64_t)(blockIdx.x - nrow) * 256 + threadIdx.x;
    if (tile < a.ntiles && a.cwidth[tile] > a.W) a.cwidth[tile] = (uint8_t)a.W;
  }
}

hipError_t launch_compact_finish(const CompactArgs& a, hipStream_t s) {
  const int nrow = (a.T + 3) / 4;
  const int ntb = (int)((a.ntiles + 255) / 256);
  if (nrow + ntb > 0) hipLaunchKernelGGL(compact_finish_kernel, dim3(nrow + ntb), dim3(256), 0, s, a, nrow);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, bool expand, hipStream_t s) {
  if (a.ntiles > 0) {
    const dim3 g((unsigned)((a.ntiles + 3) / 4));
    if (expand) hipLaunchKernelGGL(compact_tiles_kernel<true>, g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(compact_tiles_kernel<false>, g, dim3(256), 0, s, a);
  }
  if (a.T > 0) {
    const dim3 g((unsigned)((a.T + 3) / 4));
    if (expand) hipLaunchKernelGGL(compact_rows_kernel<true>, g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(compact_rows_kernel<false>, g, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace twell
