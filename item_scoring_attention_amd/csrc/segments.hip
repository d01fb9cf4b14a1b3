// Segment-descriptor builder (From Generation to Scoring, §4.1: Eq. 3
// packing, the reused position-id rule and the Eq. 4 mask; items closed by a
// delimiter token as in the LinkedIn SGLang blog's multi-item format).
//
// Three small kernels, stream-ordered:
//   items   one thread per item: absolute first token and readout position
//           (the item's last token, its closing delimiter)
//   tokens  one thread per token: item id (-1 = prefix) and position id
//   tiles   one thread per block_m x block_n tile: class 0/1/2 from visible
//           cell counts over in-range cells, counted row by row in closed
//           form (segments are contiguous, so each row's visible keys are
//           the prefix keys up to the row plus its own item's keys up to it)
#include "mis_internal.h"

namespace mis {
namespace {

// Largest r in [0, n) with a[r] <= x, for non-decreasing a with a[0] <= x.
__device__ __forceinline__ int last_le(const int32_t *a, int n, int32_t x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Request owning global item n: largest r with cu_items[r] <= n < cu_items[r+1].
__device__ __forceinline__ int request_of_item(const int32_t *cu_items, int B, int n) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_items[mid] <= n) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void items_kernel(int B, int N, const int32_t *__restrict__ cu_seqlens,
                             const int32_t *__restrict__ cu_items,
                             const int32_t *__restrict__ item_starts, int32_t *__restrict__ item_begin,
                             int32_t *__restrict__ readout_pos) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const int r = request_of_item(cu_items, B, n);
  const int32_t base = cu_seqlens[r];
  const int32_t stop = (n + 1 < cu_items[r + 1]) ? item_starts[n + 1] : cu_seqlens[r + 1] - base;
  item_begin[n] = base + item_starts[n];
  readout_pos[n] = base + stop - 1;
}

__global__ void tokens_kernel(int B, int T, const int32_t *__restrict__ cu_seqlens,
                              const int32_t *__restrict__ prefix_lens,
                              const int32_t *__restrict__ cu_items,
                              const int32_t *__restrict__ item_starts, int32_t *__restrict__ item_id,
                              int32_t *__restrict__ pos_id) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int r = last_le(cu_seqlens, B, t);
  const int32_t u = t - cu_seqlens[r];
  const int32_t lq = prefix_lens[r];
  if (u < lq) {
    item_id[t] = -1;
    pos_id[t] = u;
    return;
  }
  const int a = cu_items[r];
  const int i = a + last_le(item_starts + a, cu_items[r + 1] - a, u);
  item_id[t] = i;
  pos_id[t] = lq + (u - item_starts[i]);
}

__global__ void tiles_kernel(int B, int num_tiles, int bm, int bn,
                             const int32_t *__restrict__ cu_seqlens,
                             const int32_t *__restrict__ prefix_lens,
                             const int32_t *__restrict__ cu_tiles,
                             const int32_t *__restrict__ item_id,
                             const int32_t *__restrict__ item_begin, int8_t *__restrict__ tile_class) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= num_tiles) return;
  const int r = last_le(cu_tiles, B, g);
  const int32_t base = cu_seqlens[r];
  const int32_t Tr = cu_seqlens[r + 1] - base;
  const int32_t lq = prefix_lens[r];
  const int32_t nkt = (Tr + bn - 1) / bn;
  const int32_t local = g - cu_tiles[r];
  const int32_t qt = local / nkt, kt = local - qt * nkt;
  const int32_t j0 = qt * bm, j1 = min(Tr, j0 + bm);
  const int32_t k0 = kt * bn, k1 = min(Tr, k0 + bn);
  int64_t visible = 0;
  for (int32_t j = j0; j < j1; ++j) {
    // prefix keys k < Lq with k <= j
    const int32_t pe = min(min(lq, j + 1), k1);
    visible += max(0, pe - k0);
    if (j >= lq) {  // own-item keys in [begin of j's item, j]
      const int32_t sb = item_begin[item_id[base + j]] - base;
      visible += max(0, min(j + 1, k1) - max(sb, k0));
    }
  }
  const int64_t cells = int64_t(j1 - j0) * int64_t(k1 - k0);
  tile_class[g] = visible == 0 ? int8_t(0) : (visible == cells ? int8_t(2) : int8_t(1));
}

}  // namespace

hipError_t launch_segments(const mis_segments &seg, const int32_t *item_starts, hipStream_t st) {
  const int B = seg.num_requests, T = seg.total_tokens, N = seg.total_items;
  constexpr int kThreads = 256;
  if (N > 0) {
    items_kernel<<<(N + kThreads - 1) / kThreads, kThreads, 0, st>>>(
        B, N, seg.cu_seqlens, seg.cu_items, item_starts, const_cast<int32_t *>(seg.item_begin),
        const_cast<int32_t *>(seg.readout_pos));
  }
  tokens_kernel<<<(T + kThreads - 1) / kThreads, kThreads, 0, st>>>(
      B, T, seg.cu_seqlens, seg.prefix_lens, seg.cu_items, item_starts,
      const_cast<int32_t *>(seg.item_id), const_cast<int32_t *>(seg.pos_id));
  tiles_kernel<<<(seg.num_tiles + kThreads - 1) / kThreads, kThreads, 0, st>>>(
      B, seg.num_tiles, seg.block_m, seg.block_n, seg.cu_seqlens, seg.prefix_lens, seg.cu_tiles,
      seg.item_id, seg.item_begin, const_cast<int8_t *>(seg.tile_class));
  return hipGetLastError();
}

}  // namespace mis
