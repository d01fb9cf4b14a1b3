// Host side of the C ABI: argument and metadata validation (before anything
// is enqueued), device-buffer carving, query-tile scheduling, launch dispatch
// and the thread-local error text.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mis_internal.h"

namespace {

thread_local std::string g_error;

// Kernel variants forced by mis_set_kernel_choice on this thread (tests and
// A/B comparisons); Auto = each call picks by shape.
thread_local mis::AttnForce g_attn_force = mis::AttnForce::Auto;
thread_local mis::ScoreForce g_score_force = mis::ScoreForce::Auto;
thread_local int g_score_force_ni = 0;
thread_local char g_kernel_name[64];

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return MIS_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(MIS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x);

// Byte offset of the readout positions inside the scoring workspace (after
// the partial maxima, partial sums and label logits of n rows).
size_t score_ws_positions_offset(size_t n, size_t nvt, int32_t num_labels) {
  return align_up(sizeof(float) * n * nvt) * 2 + align_up(sizeof(float) * n * size_t(num_labels));
}

// Pinned host staging for metadata uploads. A copy from pageable memory makes
// the host wait for the stream, so the next launches could not be queued
// ahead of the GPU. Each device gets a small ring of page-locked slots; a slot
// is reused only after the event recorded behind its last copy has completed.
// The slots live until the process ends (never freed: freeing during static
// destruction could run after the HIP runtime has shut down).
class StageRing {
 public:
  static constexpr int kSlots = 8;
  static constexpr int kMaxDevices = 64;

  // Copies `bytes` of `src` to `dst` (device) on `stream` through a pinned slot.
  hipError_t upload(void *dst, const void *src, size_t bytes, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu_);
    Slot &s = slots_[dev][next_[dev]];
    next_[dev] = (next_[dev] + 1) % kSlots;
    if (!s.event) {
      e = hipEventCreateWithFlags(&s.event, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    } else if (s.busy) {
      e = hipEventSynchronize(s.event);
      if (e != hipSuccess) return e;
    }
    if (s.cap < bytes) {
      void *old = s.host;
      s.host = nullptr;
      s.cap = 0;
      if (old) {
        e = hipHostFree(old);
        if (e != hipSuccess) return e;
      }
      const size_t cap = std::max<size_t>(bytes, 64 * 1024);
      e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
      if (e != hipSuccess) return e;
      s.cap = cap;
    }
    std::memcpy(s.host, src, bytes);
    e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return e;
    e = hipEventRecord(s.event, stream);
    s.busy = (e == hipSuccess);
    return e;
  }

 private:
  struct Slot {
    void *host = nullptr;
    size_t cap = 0;
    hipEvent_t event = nullptr;
    bool busy = false;
  };
  std::mutex mu_;
  Slot slots_[kMaxDevices][kSlots];
  int next_[kMaxDevices] = {};
};

StageRing &stage_ring() {
  static StageRing *ring = new StageRing();  // intentionally leaked
  return *ring;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_block(int32_t b) { return b >= 16 && b <= 256 && b % 16 == 0; }

// Offsets of every array inside the caller's segment buffer. The first
// region ("stage") is one host->device copy; the rest is written by kernels.
struct SegLayout {
  size_t cu_seqlens, prefix_lens, cu_items, cu_tiles, item_starts, work, stage_end;
  size_t item_begin, readout_pos, item_id, pos_id, tile_class, total;
};

SegLayout seg_layout(int64_t B, int64_t T, int64_t N, int64_t tiles, int64_t work) {
  SegLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.cu_seqlens = take(sizeof(int32_t) * (B + 1));
  L.prefix_lens = take(sizeof(int32_t) * B);
  L.cu_items = take(sizeof(int32_t) * (B + 1));
  L.cu_tiles = take(sizeof(int32_t) * (B + 1));
  L.item_starts = take(sizeof(int32_t) * std::max<int64_t>(N, 1));
  L.work = take(sizeof(int32_t) * 4 * std::max<int64_t>(work, 1));
  L.stage_end = off;
  L.item_begin = take(sizeof(int32_t) * std::max<int64_t>(N, 1));
  L.readout_pos = take(sizeof(int32_t) * std::max<int64_t>(N, 1));
  L.item_id = take(sizeof(int32_t) * T);
  L.pos_id = take(sizeof(int32_t) * T);
  L.tile_class = take(sizeof(int8_t) * std::max<int64_t>(tiles, 1));
  L.total = off;
  return L;
}

// Checks cu_seqlens and returns tile and query-tile counts.
int check_seqlens(int32_t B, const int32_t *cu, int32_t bm, int32_t bn, int64_t *tiles,
                  int64_t *work, int32_t *max_len) {
  if (B < 1) return fail(MIS_ERR_ARG, "num_requests must be >= 1 (got %d)", B);
  if (!cu) return fail(MIS_ERR_ARG, "cu_seqlens is NULL");
  if (!valid_block(bm) || !valid_block(bn))
    return fail(MIS_ERR_UNSUPPORTED, "block_m/block_n must be multiples of 16 in [16, 256] (got %d x %d)",
                bm, bn);
  if (cu[0] != 0) return fail(MIS_ERR_SEGMENTS, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  int64_t t = 0, w = 0;
  int32_t mx = 0;
  for (int32_t r = 0; r < B; ++r) {
    int64_t len = int64_t(cu[r + 1]) - int64_t(cu[r]);
    if (len < 1)
      return fail(MIS_ERR_SEGMENTS, "request %d has %lld tokens; cu_seqlens must strictly increase",
                  r, (long long)len);
    t += ceil_div(len, bm) * ceil_div(len, bn);
    w += ceil_div(len, bm);
    mx = std::max<int32_t>(mx, int32_t(len));
  }
  if (t > INT32_MAX) return fail(MIS_ERR_SEGMENTS, "tile count %lld overflows int32", (long long)t);
  *tiles = t;
  *work = w;
  *max_len = mx;
  return MIS_OK;
}

}  // namespace

extern "C" {

const char *mis_last_error(void) { return g_error.c_str(); }

const char *mis_version(void) { return "mis-gfx950 0.1"; }

int mis_segments_bytes(int32_t num_requests, const int32_t *cu_seqlens_h, int32_t total_items,
                       int32_t block_m, int32_t block_n, size_t *bytes) {
  if (!bytes) return fail(MIS_ERR_ARG, "bytes is NULL");
  if (total_items < 0) return fail(MIS_ERR_ARG, "total_items must be >= 0");
  int64_t tiles, work;
  int32_t mx;
  int rc = check_seqlens(num_requests, cu_seqlens_h, block_m, block_n, &tiles, &work, &mx);
  if (rc) return rc;
  *bytes = seg_layout(num_requests, cu_seqlens_h[num_requests], total_items, tiles, work).total;
  return ok();
}

int mis_build_segments(int32_t B, const int32_t *cu_seqlens_h, const int32_t *prefix_lens_h,
                       const int32_t *cu_items_h, const int32_t *item_starts_h, int32_t block_m,
                       int32_t block_n, void *dev_buf, size_t dev_bytes, mis_segments *out,
                       void *stream) {
  if (!out) return fail(MIS_ERR_ARG, "out is NULL");
  if (!prefix_lens_h || !cu_items_h) return fail(MIS_ERR_ARG, "prefix_lens or cu_items is NULL");
  if (!dev_buf) return fail(MIS_ERR_ARG, "dev_buf is NULL");
  int64_t tiles, work;
  int32_t max_len;
  int rc = check_seqlens(B, cu_seqlens_h, block_m, block_n, &tiles, &work, &max_len);
  if (rc) return rc;
  const int32_t T = cu_seqlens_h[B];
  if (cu_items_h[0] != 0) return fail(MIS_ERR_SEGMENTS, "cu_items[0] must be 0 (got %d)", cu_items_h[0]);
  for (int32_t r = 0; r < B; ++r)
    if (cu_items_h[r + 1] < cu_items_h[r])
      return fail(MIS_ERR_SEGMENTS, "cu_items must be non-decreasing (request %d)", r);
  const int32_t N = cu_items_h[B];
  if (N > 0 && !item_starts_h) return fail(MIS_ERR_ARG, "item_starts is NULL");

  // Metadata checks: items tile [Lq, T_r) contiguously, in order.
  for (int32_t r = 0; r < B; ++r) {
    const int32_t Tr = cu_seqlens_h[r + 1] - cu_seqlens_h[r];
    const int32_t lq = prefix_lens_h[r];
    if (lq < 0 || lq > Tr)
      return fail(MIS_ERR_SEGMENTS, "request %d: prefix length %d outside [0, %d]", r, lq, Tr);
    const int32_t a = cu_items_h[r], b = cu_items_h[r + 1];
    if (a == b) {
      if (lq != Tr)
        return fail(MIS_ERR_SEGMENTS, "request %d has no items but prefix %d != length %d", r, lq, Tr);
      continue;
    }
    if (item_starts_h[a] != lq)
      return fail(MIS_ERR_SEGMENTS, "request %d: first item starts at %d, not at the prefix length %d",
                  r, item_starts_h[a], lq);
    for (int32_t i = a; i < b; ++i) {
      const int32_t end = (i + 1 < b) ? item_starts_h[i + 1] : Tr;
      if (end <= item_starts_h[i] || end > Tr)
        return fail(MIS_ERR_SEGMENTS,
                    "request %d: item %d [%d, %d) is empty, out of order or outside the request",
                    r, i, item_starts_h[i], end);
    }
  }

  const SegLayout L = seg_layout(B, T, N, tiles, work);
  if (dev_bytes < L.total)
    return fail(MIS_ERR_WORKSPACE, "dev_bytes %zu < required %zu", dev_bytes, L.total);

  // Host image of the staged region.
  std::vector<uint8_t> img(L.stage_end, 0);
  auto put = [&](size_t off, const int32_t *src, size_t n) {
    if (n) std::memcpy(img.data() + off, src, n * sizeof(int32_t));
  };
  put(L.cu_seqlens, cu_seqlens_h, B + 1);
  put(L.prefix_lens, prefix_lens_h, B);
  put(L.cu_items, cu_items_h, B + 1);
  put(L.item_starts, item_starts_h, N);
  int32_t *cu_tiles = reinterpret_cast<int32_t *>(img.data() + L.cu_tiles);
  cu_tiles[0] = 0;

  // Query-tile work list. For query tile [j0, j1) of request r the visible
  // keys are the prefix keys [0, min(Lq, j1)) and, for item rows, the keys
  // from the start of the item holding row max(j0, Lq) up to j1; key tiles
  // strictly between the two ranges hold only other items' tokens and are
  // never visited. Ordered by visited-tile count, longest first.
  struct Work {
    int32_t r, qt, a_end, b_lo, cost;
  };
  std::vector<Work> wl;
  wl.reserve(size_t(work));
  for (int32_t r = 0; r < B; ++r) {
    const int32_t Tr = cu_seqlens_h[r + 1] - cu_seqlens_h[r];
    const int32_t lq = prefix_lens_h[r];
    const int32_t nqt = int32_t(ceil_div(Tr, block_m)), nkt = int32_t(ceil_div(Tr, block_n));
    cu_tiles[r + 1] = cu_tiles[r] + nqt * nkt;
    const int32_t a = cu_items_h[r], b = cu_items_h[r + 1];
    for (int32_t qt = 0; qt < nqt; ++qt) {
      const int32_t j0 = qt * block_m, j1 = std::min(Tr, j0 + block_m);
      int32_t a_end = int32_t(ceil_div(std::min(lq, j1), block_n));
      const int32_t b_hi = int32_t(ceil_div(j1, block_n));
      int32_t b_lo = b_hi;
      if (j1 > lq) {
        const int32_t first_row = std::max(j0, lq);
        // start of the item that holds first_row
        const int32_t *s = item_starts_h + a;
        const int32_t idx = int32_t(std::upper_bound(s, s + (b - a), first_row) - s) - 1;
        b_lo = s[idx] / block_n;
      }
      if (b_lo <= a_end) {  // ranges touch: one contiguous range
        a_end = std::max(a_end, b_hi);
        b_lo = b_hi;
      }
      const int32_t cost = a_end + (b_hi - std::max(b_lo, a_end));
      wl.push_back({r, qt, a_end, b_lo, cost});
    }
  }
  std::stable_sort(wl.begin(), wl.end(), [](const Work &x, const Work &y) { return x.cost > y.cost; });
  int64_t visits = 0;
  for (const Work &x : wl) visits += x.cost;
  int32_t *wdst = reinterpret_cast<int32_t *>(img.data() + L.work);
  for (size_t i = 0; i < wl.size(); ++i) {
    wdst[4 * i + 0] = wl[i].r;
    wdst[4 * i + 1] = wl[i].qt;
    wdst[4 * i + 2] = wl[i].a_end;
    wdst[4 * i + 3] = wl[i].b_lo;
  }

  uint8_t *base = static_cast<uint8_t *>(dev_buf);
  mis_segments s{};
  s.num_requests = B;
  s.total_tokens = T;
  s.total_items = N;
  s.block_m = block_m;
  s.block_n = block_n;
  s.num_tiles = int32_t(tiles);
  s.num_work = int32_t(work);
  s.max_seqlen = max_len;
  s.num_visits = int32_t(visits);  // at most num_tiles
  s.cu_seqlens = reinterpret_cast<const int32_t *>(base + L.cu_seqlens);
  s.prefix_lens = reinterpret_cast<const int32_t *>(base + L.prefix_lens);
  s.cu_items = reinterpret_cast<const int32_t *>(base + L.cu_items);
  s.cu_tiles = reinterpret_cast<const int32_t *>(base + L.cu_tiles);
  s.item_begin = reinterpret_cast<const int32_t *>(base + L.item_begin);
  s.readout_pos = reinterpret_cast<const int32_t *>(base + L.readout_pos);
  s.item_id = reinterpret_cast<const int32_t *>(base + L.item_id);
  s.pos_id = reinterpret_cast<const int32_t *>(base + L.pos_id);
  s.tile_class = reinterpret_cast<const int8_t *>(base + L.tile_class);
  s.work = reinterpret_cast<const int32_t *>(base + L.work);

  hipStream_t st = static_cast<hipStream_t>(stream);
  // Small batches: the staged arrays travel in the builder's kernel
  // arguments, which saves a separate copy and its launch; larger ones go
  // through pinned memory and one copy.
  const size_t counts[mis::kInlineArrays] = {size_t(B) + 1, size_t(B), size_t(B) + 1, size_t(B) + 1, size_t(N),
                                             4 * size_t(work)};
  const size_t offs[mis::kInlineArrays] = {L.cu_seqlens, L.prefix_lens, L.cu_items, L.cu_tiles, L.item_starts, L.work};
  size_t inline_words = 0;
  for (size_t c : counts) inline_words += c;
  hipError_t e;
  if (inline_words <= size_t(mis::kInlineWords)) {
    mis::InlineMeta meta{};
    mis::InlineLayout lay{};
    int32_t at = 0;
    for (int a = 0; a < mis::kInlineArrays; ++a) {
      lay.src[a] = at;
      lay.dst[a] = int32_t(offs[a] / sizeof(int32_t));
      lay.len[a] = int32_t(counts[a]);
      if (counts[a]) std::memcpy(meta.w + at, img.data() + offs[a], counts[a] * sizeof(int32_t));
      at += int32_t(counts[a]);
    }
    e = mis::launch_segments_inline(s, lay, meta, static_cast<int32_t *>(dev_buf), st);
    if (e != hipSuccess) return hip_fail(e, "segment builder launch");
  } else {
    e = stage_ring().upload(dev_buf, img.data(), L.stage_end, st);
    if (e != hipSuccess) return hip_fail(e, "staging segment metadata");
    e = mis::launch_segments(s, reinterpret_cast<const int32_t *>(base + L.item_starts), st);
    if (e != hipSuccess) return hip_fail(e, "segment builder launch");
  }
  *out = s;
  return ok();
}

int mis_attention_tile_shape(mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                             int32_t *block_m, int32_t *block_n) {
  if (!block_m || !block_n) return fail(MIS_ERR_ARG, "block_m or block_n is NULL");
  if (hq < 1 || hkv < 1 || hq % hkv)
    return fail(MIS_ERR_ARG, "need hq >= 1, hkv >= 1 and hq %% hkv == 0 (got %d, %d)", hq, hkv);
  if (head_dim != 64 && head_dim != 128)
    return fail(MIS_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (dt != MIS_F32 && dt != MIS_BF16) return fail(MIS_ERR_UNSUPPORTED, "unknown dtype %d", int(dt));
  if (dt == MIS_BF16 && head_dim != 128)
    return fail(MIS_ERR_UNSUPPORTED, "bf16 attention is built for head_dim 128 (got %d)", head_dim);
  *block_m = mis::kAttnBlockM;
  *block_n = mis::kAttnBlockN;
  return ok();
}

namespace {

// Inverse frequencies theta^(-2i/D) of the rotary embedding, i < D/2.
mis::RopeFreq rope_freq(float theta, int head_dim) {
  mis::RopeFreq f{};
  for (int i = 0; i < head_dim / 2; ++i) f.inv[i] = std::pow(double(theta), -2.0 * i / head_dim);
  return f;
}

// rope_table: NULL, or the rotary table of table_positions positions (Q is
// then rotated inside the kernel).
int attention_call(const mis_segments *seg, const void *q, const void *k, const void *v, void *o,
                   mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim, float softmax_scale,
                   int items_only, const void *rope_table, int32_t table_positions, void *stream) {
  if (!seg) return fail(MIS_ERR_ARG, "seg is NULL");
  if (!q || !k || !v || !o) return fail(MIS_ERR_ARG, "q, k, v and o must be non-NULL");
  int32_t bm, bn;
  int rc = mis_attention_tile_shape(dt, hq, hkv, head_dim, &bm, &bn);
  if (rc) return rc;
  if (seg->block_m != bm || seg->block_n != bn)
    return fail(MIS_ERR_UNSUPPORTED, "segments built for %d x %d tiles; this kernel needs %d x %d",
                seg->block_m, seg->block_n, bm, bn);
  if (seg->total_tokens < 1 || !seg->work || !seg->tile_class || !seg->item_id)
    return fail(MIS_ERR_ARG, "seg is not a built segment descriptor");
  if (!std::isfinite(softmax_scale)) return fail(MIS_ERR_ARG, "softmax_scale is not finite");
  if (rope_table) {
    if (dt != MIS_BF16) return fail(MIS_ERR_UNSUPPORTED, "Q rotation inside attention is bf16 only");
    if (table_positions < seg->max_seqlen)
      return fail(MIS_ERR_ARG, "rotary table of %d positions is short: requests reach %d tokens", table_positions,
                  seg->max_seqlen);
  }
  // The bf16 kernels address a request's Q, K and V rows with 32-bit byte
  // offsets from the request start (up to the end of its last 64-row tile).
  if (dt == MIS_BF16 &&
      (uint64_t(seg->max_seqlen) + 64) * uint64_t(hq) * uint64_t(head_dim) * 2u >= (uint64_t(1) << 32))
    return fail(MIS_ERR_UNSUPPORTED,
                "a request of %d tokens with %d query heads of %d dims exceeds the 4 GiB per-request range of the "
                "bf16 kernels",
                seg->max_seqlen, hq, head_dim);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(head_dim));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dt == MIS_BF16
                     ? mis::launch_attention_bf16(*seg, q, k, v, o, hq, hkv, head_dim, scale, items_only,
                                                  mis::pick_attention_bf16(*seg, hq, hkv, g_attn_force),
                                                  static_cast<const float *>(rope_table), st)
                     : mis::launch_attention_f32(*seg, static_cast<const float *>(q),
                                                 static_cast<const float *>(k),
                                                 static_cast<const float *>(v), static_cast<float *>(o),
                                                 hq, hkv, head_dim, scale, items_only, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

}  // namespace

int mis_attention_prefill(const mis_segments *seg, const void *q, const void *k, const void *v,
                          void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                          float softmax_scale, void *stream) {
  return attention_call(seg, q, k, v, o, dt, hq, hkv, head_dim, softmax_scale, 0, nullptr, 0, stream);
}

int mis_attention_append(const mis_segments *seg, const void *q, const void *k, const void *v,
                         void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                         float softmax_scale, void *stream) {
  return attention_call(seg, q, k, v, o, dt, hq, hkv, head_dim, softmax_scale, 1, nullptr, 0, stream);
}

int mis_attention_prefill_rope(const mis_segments *seg, const void *q, const void *k, const void *v,
                               void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                               float softmax_scale, const void *rope_table, int32_t table_positions,
                               void *stream) {
  if (!rope_table) return fail(MIS_ERR_ARG, "rope_table is NULL");
  return attention_call(seg, q, k, v, o, dt, hq, hkv, head_dim, softmax_scale, 0, rope_table, table_positions,
                        stream);
}

int mis_attention_append_rope(const mis_segments *seg, const void *q, const void *k, const void *v,
                              void *o, mis_dtype dt, int32_t hq, int32_t hkv, int32_t head_dim,
                              float softmax_scale, const void *rope_table, int32_t table_positions,
                              void *stream) {
  if (!rope_table) return fail(MIS_ERR_ARG, "rope_table is NULL");
  return attention_call(seg, q, k, v, o, dt, hq, hkv, head_dim, softmax_scale, 1, rope_table, table_positions,
                        stream);
}

int mis_apply_rope(const mis_segments *seg, void *q, void *k, mis_dtype dt, int32_t hq, int32_t hkv,
                   int32_t head_dim, float theta, void *stream) {
  if (!seg) return fail(MIS_ERR_ARG, "seg is NULL");
  if (!k) return fail(MIS_ERR_ARG, "k must be non-NULL");
  if (hq < 1 || hkv < 1 || hq % hkv)
    return fail(MIS_ERR_ARG, "need hq >= 1, hkv >= 1 and hq %% hkv == 0 (got %d, %d)", hq, hkv);
  if (head_dim != 64 && head_dim != 128)
    return fail(MIS_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (dt != MIS_F32 && dt != MIS_BF16) return fail(MIS_ERR_UNSUPPORTED, "unknown dtype %d", int(dt));
  if (!(theta > 0.f) || !std::isfinite(theta)) return fail(MIS_ERR_ARG, "theta must be a positive finite number");
  if (seg->total_tokens < 1 || !seg->pos_id) return fail(MIS_ERR_ARG, "seg is not a built segment descriptor");
  const mis::RopeFreq f = rope_freq(theta, head_dim);
  hipError_t e =
      mis::launch_rope(*seg, q, k, dt, q ? hq : 0, hkv, head_dim, f, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  return ok();
}

int mis_rope_table_bytes(int32_t num_positions, int32_t head_dim, size_t *bytes) {
  if (!bytes) return fail(MIS_ERR_ARG, "bytes is NULL");
  if (num_positions < 1) return fail(MIS_ERR_ARG, "num_positions must be >= 1 (got %d)", num_positions);
  if (head_dim != 64 && head_dim != 128)
    return fail(MIS_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  *bytes = size_t(num_positions) * size_t(head_dim) * sizeof(float);
  return ok();
}

int mis_rope_table(int32_t num_positions, int32_t head_dim, float theta, void *table, size_t table_bytes,
                   void *stream) {
  size_t need = 0;
  int rc = mis_rope_table_bytes(num_positions, head_dim, &need);
  if (rc) return rc;
  if (!table) return fail(MIS_ERR_ARG, "table is NULL");
  if (table_bytes < need) return fail(MIS_ERR_ARG, "table of %zu bytes, need %zu", table_bytes, need);
  if (!(theta > 0.f) || !std::isfinite(theta)) return fail(MIS_ERR_ARG, "theta must be a positive finite number");
  const mis::RopeFreq f = rope_freq(theta, head_dim);
  hipError_t e = mis::launch_rope_table(static_cast<float *>(table), num_positions, head_dim, f,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  return ok();
}

int mis_score_workspace_bytes(int32_t num_items, int32_t vocab, int32_t num_labels, int32_t hidden,
                              mis_dtype dt, size_t *bytes) {
  if (!bytes) return fail(MIS_ERR_ARG, "bytes is NULL");
  if (num_items < 0 || vocab < 1 || hidden < 1)
    return fail(MIS_ERR_ARG, "need num_items >= 0, vocab >= 1, hidden >= 1");
  if (num_labels < 1 || num_labels > MIS_MAX_LABELS)
    return fail(MIS_ERR_LABEL, "num_labels must be in [1, %d] (got %d)", MIS_MAX_LABELS, num_labels);
  if (dt != MIS_F32 && dt != MIS_BF16) return fail(MIS_ERR_UNSUPPORTED, "unknown dtype %d", int(dt));
  const size_t nvt = size_t(mis::score_vocab_tiles(vocab));
  const size_t n = size_t(std::max(num_items, 1));
  *bytes = score_ws_positions_offset(n, nvt, num_labels) + align_up(sizeof(int32_t) * n);
  return ok();
}

}  // extern "C"

namespace {

// Argument checks of mis_score_labels and mis_score_labels_noalloc (all on
// the host); *need = workspace bytes of the call.
int score_labels_check(const mis_segments *seg, const void *hidden, int32_t hidden_size, const void *lm_head,
                       int32_t vocab, mis_dtype dt, const int32_t *label_ids_h, int32_t num_labels,
                       const float *scores, size_t *need) {
  if (!seg) return fail(MIS_ERR_ARG, "seg is NULL");
  if (!hidden || !lm_head) return fail(MIS_ERR_ARG, "hidden and lm_head must be non-NULL");
  if (!scores && seg->total_items > 0) return fail(MIS_ERR_ARG, "scores is NULL");
  if (!label_ids_h) return fail(MIS_ERR_ARG, "label_ids is NULL");
  int rc = mis_score_workspace_bytes(seg->total_items, vocab, num_labels, hidden_size, dt, need);
  if (rc) return rc;
  for (int32_t i = 0; i < num_labels; ++i)
    if (label_ids_h[i] < 0 || label_ids_h[i] >= vocab)
      return fail(MIS_ERR_LABEL, "label id %d at position %d outside [0, %d)", label_ids_h[i], i, vocab);
  if (dt == MIS_BF16 && hidden_size % 32)
    return fail(MIS_ERR_UNSUPPORTED, "bf16 scoring needs hidden_size %% 32 == 0 (got %d)", hidden_size);
  // a vocabulary tile's LM-head rows are addressed with 32-bit byte offsets
  if (hidden_size > (1 << 22))
    return fail(MIS_ERR_UNSUPPORTED, "hidden_size %d is above the 4194304 the scoring kernels address", hidden_size);
  if (seg->total_items > 0 && !seg->readout_pos) return fail(MIS_ERR_ARG, "seg is not a built segment descriptor");
  return MIS_OK;
}

int score_labels_launch(const mis_segments *seg, const void *hidden, int32_t hidden_size, const void *lm_head,
                        int32_t vocab, mis_dtype dt, const int32_t *label_ids_h, int32_t num_labels,
                        int32_t apply_softmax, float *scores, void *ws, void *stream) {
  mis::LabelArgs la{};
  la.k = num_labels;
  std::memcpy(la.ids, label_ids_h, sizeof(int32_t) * num_labels);
  const mis::ScoreKernel kern = mis::pick_score(seg->total_items, hidden_size, dt, g_score_force, g_score_force_ni);
  hipError_t e = mis::launch_score(seg->readout_pos, seg->total_items, hidden, hidden_size, lm_head, vocab, dt, la,
                                   apply_softmax ? 1 : 0, scores, static_cast<float *>(ws), kern,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "scoring launch");
  return ok();
}

}  // namespace

extern "C" {

int mis_score_labels(const mis_segments *seg, const void *hidden, int32_t hidden_size,
                     const void *lm_head, int32_t vocab, mis_dtype dt, const int32_t *label_ids_h,
                     int32_t num_labels, int32_t apply_softmax, float *scores, void *ws,
                     size_t ws_bytes, void *stream) {
  size_t need;
  int rc = score_labels_check(seg, hidden, hidden_size, lm_head, vocab, dt, label_ids_h, num_labels, scores, &need);
  if (rc) return rc;
  if (!ws) return fail(MIS_ERR_ARG, "ws is NULL");
  if (ws_bytes < need) return fail(MIS_ERR_WORKSPACE, "ws_bytes %zu < required %zu", ws_bytes, need);
  if (seg->total_items == 0) return ok();
  return score_labels_launch(seg, hidden, hidden_size, lm_head, vocab, dt, label_ids_h, num_labels, apply_softmax,
                             scores, ws, stream);
}

int mis_score_labels_noalloc(const mis_segments *seg, const void *hidden, int32_t hidden_size,
                             const void *lm_head, int32_t vocab, mis_dtype dt, const int32_t *label_ids_h,
                             int32_t num_labels, int32_t apply_softmax, float *scores, void *stream) {
  size_t need;
  int rc = score_labels_check(seg, hidden, hidden_size, lm_head, vocab, dt, label_ids_h, num_labels, scores, &need);
  if (rc) return rc;
  // the partials and label logits only (the readout-position region of the
  // workspace serves mis_score_labels_at)
  const size_t nvt = size_t(mis::score_vocab_tiles(vocab));
  const size_t used = score_ws_positions_offset(size_t(std::max(seg->total_items, 1)), nvt, num_labels);
  if (used > size_t(MIS_SCORE_SCRATCH_BYTES))
    return fail(MIS_ERR_WORKSPACE,
                "%d items x %d vocabulary rows x %d labels need %zu bytes of scratch; the library's scratch holds "
                "%zu (mis_score_labels takes a caller workspace of any size)",
                seg->total_items, vocab, num_labels, used, size_t(MIS_SCORE_SCRATCH_BYTES));
  if (seg->total_items == 0) return ok();
  void *ws = nullptr;
  hipError_t e = mis::score_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "device address of the scoring scratch");
  return score_labels_launch(seg, hidden, hidden_size, lm_head, vocab, dt, label_ids_h, num_labels, apply_softmax,
                             scores, ws, stream);
}

int mis_score_labels_at(const int32_t *positions_h, int32_t num_rows, int32_t num_tokens,
                        const void *hidden, int32_t hidden_size, const void *lm_head, int32_t vocab,
                        mis_dtype dt, const int32_t *label_ids_h, int32_t num_labels,
                        int32_t apply_softmax, float *scores, void *ws, size_t ws_bytes, void *stream) {
  if (num_rows < 0 || num_tokens < 1) return fail(MIS_ERR_ARG, "need num_rows >= 0 and num_tokens >= 1");
  if (num_rows > 0 && (!positions_h || !scores)) return fail(MIS_ERR_ARG, "positions and scores must be non-NULL");
  if (!hidden || !lm_head || !ws) return fail(MIS_ERR_ARG, "hidden, lm_head and ws must be non-NULL");
  if (!label_ids_h) return fail(MIS_ERR_ARG, "label_ids is NULL");
  size_t need;
  int rc = mis_score_workspace_bytes(num_rows, vocab, num_labels, hidden_size, dt, &need);
  if (rc) return rc;
  for (int32_t i = 0; i < num_labels; ++i)
    if (label_ids_h[i] < 0 || label_ids_h[i] >= vocab)
      return fail(MIS_ERR_LABEL, "label id %d at position %d outside [0, %d)", label_ids_h[i], i, vocab);
  for (int32_t i = 0; i < num_rows; ++i)
    if (positions_h[i] < 0 || positions_h[i] >= num_tokens)
      return fail(MIS_ERR_ARG, "position %d at index %d outside [0, %d)", positions_h[i], i, num_tokens);
  if (ws_bytes < need) return fail(MIS_ERR_WORKSPACE, "ws_bytes %zu < required %zu", ws_bytes, need);
  if (dt == MIS_BF16 && hidden_size % 32)
    return fail(MIS_ERR_UNSUPPORTED, "bf16 scoring needs hidden_size %% 32 == 0 (got %d)", hidden_size);
  // a vocabulary tile's LM-head rows are addressed with 32-bit byte offsets
  if (hidden_size > (1 << 22))
    return fail(MIS_ERR_UNSUPPORTED, "hidden_size %d is above the 4194304 the scoring kernels address", hidden_size);
  if (num_rows == 0) return ok();
  const size_t off = score_ws_positions_offset(size_t(num_rows), size_t(mis::score_vocab_tiles(vocab)), num_labels);
  int32_t *pos_dev = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(ws) + off);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = stage_ring().upload(pos_dev, positions_h, sizeof(int32_t) * size_t(num_rows), st);
  if (e != hipSuccess) return hip_fail(e, "staging readout positions");
  mis::LabelArgs la{};
  la.k = num_labels;
  std::memcpy(la.ids, label_ids_h, sizeof(int32_t) * num_labels);
  e = mis::launch_score(pos_dev, num_rows, hidden, hidden_size, lm_head, vocab, dt, la, apply_softmax ? 1 : 0,
                        scores, static_cast<float *>(ws),
                        mis::pick_score(num_rows, hidden_size, dt, g_score_force, g_score_force_ni), st);
  if (e != hipSuccess) return hip_fail(e, "scoring launch");
  return ok();
}

int mis_set_kernel_choice(const char *attention, const char *score) {
  mis::AttnForce af;
  if (!attention || !*attention || !std::strcmp(attention, "auto")) af = mis::AttnForce::Auto;
  else if (!std::strcmp(attention, "pipe")) af = mis::AttnForce::Pipe;
  else if (!std::strcmp(attention, "pipe32")) af = mis::AttnForce::Pipe32;
  else if (!std::strcmp(attention, "classic")) af = mis::AttnForce::Classic;
  else if (!std::strcmp(attention, "pipe2")) af = mis::AttnForce::Pipe2;
  else return fail(MIS_ERR_ARG, "unknown attention kernel choice '%s' (auto, pipe, pipe2, pipe32, classic)", attention);
  mis::ScoreForce sf;
  int ni = 0;
  if (!score || !*score || !std::strcmp(score, "auto")) sf = mis::ScoreForce::Auto;
  else if (!std::strcmp(score, "narrow")) sf = mis::ScoreForce::Narrow;
  else if (!std::strcmp(score, "wide")) sf = mis::ScoreForce::Wide;
  else if (!std::strncmp(score, "wide", 4) && score[4] >= '3' && score[4] <= '8' && score[4] != '7' && !score[5]) {
    sf = mis::ScoreForce::Wide;
    ni = score[4] - '0';
  } else if (!std::strcmp(score, "persist")) {
    sf = mis::ScoreForce::Persist;
  } else if (!std::strncmp(score, "persist", 7) && score[7] >= '3' && score[7] <= '5' && !score[8]) {
    sf = mis::ScoreForce::Persist;
    ni = score[7] - '0';
  } else {
    return fail(MIS_ERR_ARG,
                "unknown scoring kernel choice '%s' (auto, narrow, wide, wide3..wide6, wide8, persist, persist3..5)",
                score);
  }
  g_attn_force = af;
  g_score_force = sf;
  g_score_force_ni = ni;
  return ok();
}

const char *mis_attention_kernel_name(const mis_segments *seg, mis_dtype dt, int32_t hq, int32_t hkv,
                                      int32_t head_dim) {
  int32_t bm, bn;
  if (!seg) {
    fail(MIS_ERR_ARG, "seg is NULL");
    return "";
  }
  if (mis_attention_tile_shape(dt, hq, hkv, head_dim, &bm, &bn) != MIS_OK) return "";
  if (dt != MIS_BF16) return "attn_f32_kernel";
  return mis::attention_bf16_name(mis::pick_attention_bf16(*seg, hq, hkv, g_attn_force));
}

const char *mis_score_kernel_name(int32_t num_items, int32_t hidden_size, mis_dtype dt) {
  if (num_items < 0 || hidden_size < 1) {
    fail(MIS_ERR_ARG, "need num_items >= 0 and hidden_size >= 1");
    return "";
  }
  mis::score_kernel_name(mis::pick_score(num_items, hidden_size, dt, g_score_force, g_score_force_ni),
                         g_kernel_name, sizeof(g_kernel_name));
  return g_kernel_name;
}

}  // extern "C"
