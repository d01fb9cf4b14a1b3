// Segment-descriptor builder (From Generation to Scoring, §4.1: Eq. 3
// packing, the reused position-id rule and the Eq. 4 mask; items closed by a
// delimiter token as in the LinkedIn SGLang blog's multi-item format).
//
// One launch with three independent roles:
//   tokens  one thread per token: item id (-1 = prefix) and position id
//   items   one thread per item: absolute first token and readout position
//           (the item's last token, its closing delimiter)
//   tiles   one thread per block_m x block_n tile: class 0/1/2 from the
//           number of visible in-range cells. Segments are contiguous, so a
//           row's visible keys are the prefix keys up to the row plus its own
//           item's keys up to the row; the count over the rows of one
//           segment is an arithmetic series, so a tile costs one step per
//           segment it overlaps.
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

// Sum over a in [lo, hi] (inclusive) of max(0, min(a, k1) - m0).
__device__ __forceinline__ int64_t sum_clip(int64_t lo, int64_t hi, int64_t m0, int64_t k1) {
  int64_t total = 0;
  const int64_t a1 = max(lo, m0 + 1), b1 = min(hi, k1);  // rising part: a - m0
  if (b1 >= a1) total += (b1 - a1 + 1) * ((a1 - m0) + (b1 - m0)) / 2;
  const int64_t a2 = max(lo, k1 + 1);  // flat part: k1 - m0
  if (hi >= a2 && k1 > m0) total += (hi - a2 + 1) * (k1 - m0);
  return total;
}

// The three roles by block range: tokens, items, tiles. No role reads
// another role's output, so they need no ordering.
__device__ __forceinline__ void build_roles(
    int B, int T, int N, int num_tiles, int bm, int bn, int tok_blocks, int item_blocks,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ prefix_lens,
    const int32_t *__restrict__ cu_items, const int32_t *__restrict__ item_starts,
    const int32_t *__restrict__ cu_tiles, int32_t *__restrict__ item_id, int32_t *__restrict__ pos_id,
    int32_t *__restrict__ item_begin, int32_t *__restrict__ readout_pos, int8_t *__restrict__ tile_class) {
  const int blk = blockIdx.x;
  if (blk < tok_blocks) {  // ---- per token: item id and reused position id
    const int t = blk * blockDim.x + threadIdx.x;
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
    return;
  }
  if (blk < tok_blocks + item_blocks) {  // ---- per item: first token and readout token
    const int n = (blk - tok_blocks) * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const int r = request_of_item(cu_items, B, n);
    const int32_t base = cu_seqlens[r];
    const int32_t stop = (n + 1 < cu_items[r + 1]) ? item_starts[n + 1] : cu_seqlens[r + 1] - base;
    item_begin[n] = base + item_starts[n];
    readout_pos[n] = base + stop - 1;
    return;
  }
  // ---- per tile: visible cells in closed form, segment by segment
  const int g = (blk - tok_blocks - item_blocks) * blockDim.x + threadIdx.x;
  if (g >= num_tiles) return;
  const int r = last_le(cu_tiles, B, g);
  const int32_t Tr = cu_seqlens[r + 1] - cu_seqlens[r];
  const int32_t lq = prefix_lens[r];
  const int32_t nkt = (Tr + bn - 1) / bn;
  const int32_t local = g - cu_tiles[r];
  const int32_t qt = local / nkt, kt = local - qt * nkt;
  const int32_t j0 = qt * bm, j1 = min(Tr, j0 + bm);
  const int32_t k0 = kt * bn, k1 = min(Tr, k0 + bn);
  int64_t visible = 0;
  // prefix rows j in [j0, min(j1, Lq)): keys k in [k0, k1) with k <= j
  if (j0 < lq) visible += sum_clip(j0 + 1, min(j1, lq), k0, k1);
  // item rows: the prefix keys of the tile plus own-item keys up to the row
  const int32_t r0 = max(j0, lq);
  if (r0 < j1) {
    const int a = cu_items[r], b = cu_items[r + 1];
    const int64_t cp = max(0, min(k1, lq) - k0);
    for (int i = a + last_le(item_starts + a, b - a, r0); i < b && item_starts[i] < j1; ++i) {
      const int32_t s0 = item_starts[i];
      const int32_t e0 = (i + 1 < b) ? item_starts[i + 1] : Tr;
      const int32_t ra = max(s0, j0), rb = min(e0, j1);
      visible += cp * (rb - ra) + sum_clip(ra + 1, rb, max(s0, k0), k1);
    }
  }
  const int64_t cells = int64_t(j1 - j0) * int64_t(k1 - k0);
  tile_class[g] = visible == 0 ? int8_t(0) : (visible == cells ? int8_t(2) : int8_t(1));
}

// Metadata already staged in device memory by a copy.
__global__ __launch_bounds__(256) void builder_kernel(
    int B, int T, int N, int num_tiles, int bm, int bn, int tok_blocks, int item_blocks,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ prefix_lens,
    const int32_t *__restrict__ cu_items, const int32_t *__restrict__ item_starts,
    const int32_t *__restrict__ cu_tiles, int32_t *__restrict__ item_id, int32_t *__restrict__ pos_id,
    int32_t *__restrict__ item_begin, int32_t *__restrict__ readout_pos, int8_t *__restrict__ tile_class) {
  build_roles(B, T, N, num_tiles, bm, bn, tok_blocks, item_blocks, cu_seqlens, prefix_lens, cu_items,
              item_starts, cu_tiles, item_id, pos_id, item_begin, readout_pos, tile_class);
}

// Small batches: the metadata travels in the kernel arguments (no separate
// host-to-device copy and launch). Every thread first copies its share of
// the arrays to their places in the segment buffer (the later kernels read
// them there), then runs its role on the argument copy.
__global__ __launch_bounds__(256) void builder_inline_kernel(
    int B, int T, int N, int num_tiles, int bm, int bn, int tok_blocks, int item_blocks, InlineLayout lay,
    InlineMeta meta, int32_t *__restrict__ stage, int32_t *__restrict__ item_id, int32_t *__restrict__ pos_id,
    int32_t *__restrict__ item_begin, int32_t *__restrict__ readout_pos, int8_t *__restrict__ tile_class) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  const int nthreads = gridDim.x * blockDim.x;
#pragma unroll
  for (int a = 0; a < kInlineArrays; ++a)
    for (int i = g; i < lay.len[a]; i += nthreads) stage[lay.dst[a] + i] = meta.w[lay.src[a] + i];
  const int32_t *w = meta.w;
  build_roles(B, T, N, num_tiles, bm, bn, tok_blocks, item_blocks, w + lay.src[0], w + lay.src[1], w + lay.src[2],
              w + lay.src[4], w + lay.src[3], item_id, pos_id, item_begin, readout_pos, tile_class);
}

}  // namespace

hipError_t launch_segments_inline(const mis_segments &seg, const InlineLayout &lay, const InlineMeta &meta,
                                  int32_t *stage, hipStream_t st) {
  constexpr int kThreads = 256;
  const int tok_blocks = (seg.total_tokens + kThreads - 1) / kThreads;
  const int item_blocks = (seg.total_items + kThreads - 1) / kThreads;
  const int tile_blocks = (seg.num_tiles + kThreads - 1) / kThreads;
  builder_inline_kernel<<<tok_blocks + item_blocks + tile_blocks, kThreads, 0, st>>>(
      seg.num_requests, seg.total_tokens, seg.total_items, seg.num_tiles, seg.block_m, seg.block_n,
      tok_blocks, item_blocks, lay, meta, stage, const_cast<int32_t *>(seg.item_id),
      const_cast<int32_t *>(seg.pos_id), const_cast<int32_t *>(seg.item_begin),
      const_cast<int32_t *>(seg.readout_pos), const_cast<int8_t *>(seg.tile_class));
  return hipGetLastError();
}

hipError_t launch_segments(const mis_segments &seg, const int32_t *item_starts, hipStream_t st) {
  constexpr int kThreads = 256;
  const int tok_blocks = (seg.total_tokens + kThreads - 1) / kThreads;
  const int item_blocks = (seg.total_items + kThreads - 1) / kThreads;
  const int tile_blocks = (seg.num_tiles + kThreads - 1) / kThreads;
  builder_kernel<<<tok_blocks + item_blocks + tile_blocks, kThreads, 0, st>>>(
      seg.num_requests, seg.total_tokens, seg.total_items, seg.num_tiles, seg.block_m, seg.block_n,
      tok_blocks, item_blocks, seg.cu_seqlens, seg.prefix_lens, seg.cu_items, item_starts, seg.cu_tiles,
      const_cast<int32_t *>(seg.item_id), const_cast<int32_t *>(seg.pos_id),
      const_cast<int32_t *>(seg.item_begin), const_cast<int32_t *>(seg.readout_pos),
      const_cast<int8_t *>(seg.tile_class));
  return hipGetLastError();
}

}  // namespace mis
