// Host-side checks of the C ABI (include/mis.h) in an AddressSanitizer and
// UndefinedBehaviorSanitizer build: every malformed input must come back
// with its status code and an error text, before anything touches a device,
// and a valid call on a host without a GPU must report MIS_ERR_HIP. The GPU
// launchers are stubs (launch_stubs.cpp); nothing here runs device code.
// Prints "ok <n> checks" and returns 0, or names the first failed check.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mis.h"

namespace {

int g_checks = 0;

bool expect(const char *what, int got, int want) {
  ++g_checks;
  if (got == want && (want == MIS_OK) == (mis_last_error()[0] == '\0')) return true;
  std::fprintf(stderr, "FAILED %s: status %d (want %d), error text '%s'\n", what, got, want, mis_last_error());
  return false;
}

bool expect_true(const char *what, bool cond) {
  ++g_checks;
  if (cond) return true;
  std::fprintf(stderr, "FAILED %s\n", what);
  return false;
}

// A fake device address: the checks below fail before it could be used.
void *const kFakeDev = reinterpret_cast<void *>(uintptr_t(0x100000));

mis_segments built_segments(int32_t tokens, int32_t items) {
  mis_segments s{};
  s.num_requests = 1;
  s.total_tokens = tokens;
  s.total_items = items;
  s.block_m = s.block_n = 64;
  s.num_work = (tokens + 63) / 64;
  s.num_visits = s.num_work;
  s.max_seqlen = tokens;
  s.cu_seqlens = s.prefix_lens = s.cu_items = s.cu_tiles = s.item_begin = s.readout_pos = s.item_id = s.pos_id =
      s.work = static_cast<const int32_t *>(kFakeDev);
  s.tile_class = static_cast<const int8_t *>(kFakeDev);
  return s;
}

}  // namespace

int main() {
  bool ok = true;
  size_t bytes = 0;
  const int32_t cu1[] = {0, 100};
  // ---- segment size query
  ok &= expect("segments_bytes valid", mis_segments_bytes(1, cu1, 4, 64, 64, &bytes), MIS_OK);
  ok &= expect("segments_bytes bytes NULL", mis_segments_bytes(1, cu1, 4, 64, 64, nullptr), MIS_ERR_ARG);
  ok &= expect("segments_bytes negative items", mis_segments_bytes(1, cu1, -1, 64, 64, &bytes), MIS_ERR_ARG);
  ok &= expect("segments_bytes block 48x24", mis_segments_bytes(1, cu1, 4, 48, 24, &bytes), MIS_ERR_UNSUPPORTED);
  ok &= expect("segments_bytes block 512", mis_segments_bytes(1, cu1, 4, 512, 64, &bytes), MIS_ERR_UNSUPPORTED);
  const int32_t cu_bad0[] = {1, 100};
  ok &= expect("segments_bytes cu[0] != 0", mis_segments_bytes(1, cu_bad0, 4, 64, 64, &bytes), MIS_ERR_SEGMENTS);
  const int32_t cu_flat[] = {0, 100, 100};
  ok &= expect("segments_bytes empty request", mis_segments_bytes(2, cu_flat, 4, 64, 64, &bytes), MIS_ERR_SEGMENTS);
  ok &= expect("segments_bytes no requests", mis_segments_bytes(0, cu1, 0, 64, 64, &bytes), MIS_ERR_ARG);

  // ---- segment builder metadata checks (request of 100 tokens, prefix 40)
  mis_segments out{};
  const int32_t pl[] = {40}, ci[] = {0, 3};
  auto build = [&](const int32_t *cu, const int32_t *p, const int32_t *c, const int32_t *st, size_t dev_bytes) {
    return mis_build_segments(1, cu, p, c, st, 64, 64, kFakeDev, dev_bytes, &out, nullptr);
  };
  const int32_t st_ok[] = {40, 60, 90};
  const int32_t st_first[] = {41, 60, 90}, st_order[] = {40, 90, 60}, st_out[] = {40, 60, 100};
  ok &= expect("build first item not at the prefix end", build(cu1, pl, ci, st_first, 1 << 20), MIS_ERR_SEGMENTS);
  ok &= expect("build items out of order", build(cu1, pl, ci, st_order, 1 << 20), MIS_ERR_SEGMENTS);
  ok &= expect("build empty last item", build(cu1, pl, ci, st_out, 1 << 20), MIS_ERR_SEGMENTS);
  const int32_t pl_long[] = {101};
  ok &= expect("build prefix longer than the request", build(cu1, pl_long, ci, st_ok, 1 << 20), MIS_ERR_SEGMENTS);
  const int32_t ci_none[] = {0, 0};
  ok &= expect("build no items, prefix != length", build(cu1, pl, ci_none, st_ok, 1 << 20), MIS_ERR_SEGMENTS);
  const int32_t ci_bad[] = {1, 3};
  ok &= expect("build cu_items[0] != 0", build(cu1, pl, ci_bad, st_ok, 1 << 20), MIS_ERR_SEGMENTS);
  ok &= expect("build NULL item starts", build(cu1, pl, ci, nullptr, 1 << 20), MIS_ERR_ARG);
  ok &= expect("build buffer too small", build(cu1, pl, ci, st_ok, 16), MIS_ERR_WORKSPACE);
  ok &= expect("build NULL out",
               mis_build_segments(1, cu1, pl, ci, st_ok, 64, 64, kFakeDev, 1 << 20, nullptr, nullptr), MIS_ERR_ARG);
  ok &= expect("build NULL buffer",
               mis_build_segments(1, cu1, pl, ci, st_ok, 64, 64, nullptr, 1 << 20, &out, nullptr), MIS_ERR_ARG);
  // valid metadata reaches the launch; there is no device
  ok &= expect("build valid, no device (kernel arguments)", build(cu1, pl, ci, st_ok, 1 << 20), MIS_ERR_HIP);
  {
    // a batch too large for kernel arguments stages through pinned memory
    const int32_t n = 2000;
    std::vector<int32_t> cu = {0, 40 + 2 * n}, p = {40}, c = {0, n}, st(n);
    for (int32_t i = 0; i < n; ++i) st[i] = 40 + 2 * i;
    ok &= expect("build valid, no device (pinned staging)", build(cu.data(), p.data(), c.data(), st.data(), 1 << 24),
                 MIS_ERR_HIP);
  }

  // ---- attention
  int32_t bm = 0, bn = 0;
  ok &= expect("tile shape bf16", mis_attention_tile_shape(MIS_BF16, 16, 8, 128, &bm, &bn), MIS_OK);
  ok &= expect("tile shape hq % hkv", mis_attention_tile_shape(MIS_BF16, 12, 8, 128, &bm, &bn), MIS_ERR_ARG);
  ok &= expect("tile shape head_dim 96", mis_attention_tile_shape(MIS_F32, 8, 8, 96, &bm, &bn), MIS_ERR_UNSUPPORTED);
  ok &= expect("tile shape bf16 head_dim 64", mis_attention_tile_shape(MIS_BF16, 8, 8, 64, &bm, &bn),
               MIS_ERR_UNSUPPORTED);
  ok &= expect("tile shape dtype 7", mis_attention_tile_shape(mis_dtype(7), 8, 8, 64, &bm, &bn), MIS_ERR_UNSUPPORTED);
  mis_segments s = built_segments(100, 3);
  void *t = kFakeDev;
  ok &= expect("prefill NULL seg", mis_attention_prefill(nullptr, t, t, t, t, MIS_BF16, 16, 8, 128, 0.f, nullptr),
               MIS_ERR_ARG);
  ok &= expect("prefill NULL o", mis_attention_prefill(&s, t, t, t, nullptr, MIS_BF16, 16, 8, 128, 0.f, nullptr),
               MIS_ERR_ARG);
  ok &= expect("prefill scale NaN", mis_attention_prefill(&s, t, t, t, t, MIS_BF16, 16, 8, 128, NAN, nullptr),
               MIS_ERR_ARG);
  mis_segments s32 = s;
  s32.block_m = s32.block_n = 32;
  ok &= expect("prefill tile shape mismatch",
               mis_attention_prefill(&s32, t, t, t, t, MIS_BF16, 16, 8, 128, 0.f, nullptr), MIS_ERR_UNSUPPORTED);
  mis_segments huge = built_segments(2000000, 3);
  ok &= expect("prefill request beyond 32-bit offsets",
               mis_attention_prefill(&huge, t, t, t, t, MIS_BF16, 64, 8, 128, 0.f, nullptr), MIS_ERR_UNSUPPORTED);
  ok &= expect("prefill valid, no device", mis_attention_prefill(&s, t, t, t, t, MIS_BF16, 16, 8, 128, 0.f, nullptr),
               MIS_ERR_HIP);
  ok &= expect("append valid, no device", mis_attention_append(&s, t, t, t, t, MIS_F32, 4, 4, 64, 0.f, nullptr),
               MIS_ERR_HIP);
  ok &= expect("rope theta 0", mis_apply_rope(&s, t, t, MIS_BF16, 16, 8, 128, 0.f, nullptr), MIS_ERR_ARG);
  ok &= expect("rope theta inf", mis_apply_rope(&s, t, t, MIS_BF16, 16, 8, 128, INFINITY, nullptr), MIS_ERR_ARG);
  ok &= expect("rope head_dim 96", mis_apply_rope(&s, t, t, MIS_BF16, 16, 8, 96, 1e4f, nullptr), MIS_ERR_UNSUPPORTED);
  ok &= expect("rope NULL k", mis_apply_rope(&s, t, nullptr, MIS_BF16, 16, 8, 128, 1e4f, nullptr), MIS_ERR_ARG);
  ok &= expect("rope K only, no device", mis_apply_rope(&s, nullptr, t, MIS_BF16, 16, 8, 128, 1e4f, nullptr),
               MIS_ERR_HIP);
  ok &= expect("rope table bytes", mis_rope_table_bytes(100, 128, &bytes), MIS_OK);
  ok &= expect_true("rope table bytes value", bytes == size_t(100) * 128 * 4);
  ok &= expect("rope table 0 positions", mis_rope_table_bytes(0, 128, &bytes), MIS_ERR_ARG);
  ok &= expect("rope table short buffer", mis_rope_table(100, 128, 1e4f, t, 100 * 128 * 4 - 1, nullptr), MIS_ERR_ARG);
  ok &= expect("rope table, no device", mis_rope_table(100, 128, 1e4f, t, 100 * 128 * 4, nullptr), MIS_ERR_HIP);
  ok &= expect("fused rope NULL table",
               mis_attention_prefill_rope(&s, t, t, t, t, MIS_BF16, 16, 8, 128, 0.f, nullptr, 1000, nullptr),
               MIS_ERR_ARG);
  ok &= expect("fused rope short table",
               mis_attention_prefill_rope(&s, t, t, t, t, MIS_BF16, 16, 8, 128, 0.f, t, s.max_seqlen - 1, nullptr),
               MIS_ERR_ARG);
  ok &= expect("fused rope valid, no device",
               mis_attention_append_rope(&s, t, t, t, t, MIS_BF16, 16, 8, 128, 0.f, t, s.max_seqlen, nullptr),
               MIS_ERR_HIP);

  // ---- scoring
  const int32_t labels[] = {3, 7}, bad_label[] = {3, 1000};
  ok &= expect("workspace K = 0", mis_score_workspace_bytes(3, 1000, 0, 64, MIS_BF16, &bytes), MIS_ERR_LABEL);
  ok &= expect("workspace K = 257", mis_score_workspace_bytes(3, 1000, 257, 64, MIS_BF16, &bytes), MIS_ERR_LABEL);
  ok &= expect("workspace vocab 0", mis_score_workspace_bytes(3, 0, 2, 64, MIS_BF16, &bytes), MIS_ERR_ARG);
  ok &= expect("workspace valid", mis_score_workspace_bytes(3, 1000, 2, 64, MIS_BF16, &bytes), MIS_OK);
  float *sc = static_cast<float *>(kFakeDev);
  ok &= expect("score label outside the vocabulary",
               mis_score_labels(&s, t, 64, t, 1000, MIS_BF16, bad_label, 2, 0, sc, t, bytes, nullptr), MIS_ERR_LABEL);
  ok &= expect("score workspace too small",
               mis_score_labels(&s, t, 64, t, 1000, MIS_BF16, labels, 2, 0, sc, t, bytes - 1, nullptr),
               MIS_ERR_WORKSPACE);
  ok &= expect("score bf16 hidden 48",
               mis_score_labels(&s, t, 48, t, 1000, MIS_BF16, labels, 2, 0, sc, t, 1 << 20, nullptr),
               MIS_ERR_UNSUPPORTED);
  ok &= expect("score NULL scores",
               mis_score_labels(&s, t, 64, t, 1000, MIS_BF16, labels, 2, 0, nullptr, t, bytes, nullptr), MIS_ERR_ARG);
  ok &= expect("score valid, no device",
               mis_score_labels(&s, t, 64, t, 1000, MIS_BF16, labels, 2, 0, sc, t, bytes, nullptr), MIS_ERR_HIP);
  mis_segments many = built_segments(3000, 2000);
  ok &= expect("noalloc beyond its scratch",
               mis_score_labels_noalloc(&many, t, 64, t, 151936, MIS_BF16, labels, 2, 0, sc, nullptr),
               MIS_ERR_WORKSPACE);
  ok &= expect("noalloc valid, no device",
               mis_score_labels_noalloc(&s, t, 64, t, 1000, MIS_BF16, labels, 2, 0, sc, nullptr), MIS_ERR_HIP);
  const int32_t pos_ok[] = {0, 99}, pos_bad[] = {0, 100};
  ok &= expect("score_at position out of range",
               mis_score_labels_at(pos_bad, 2, 100, t, 64, t, 1000, MIS_BF16, labels, 2, 0, sc, t, 1 << 20, nullptr),
               MIS_ERR_ARG);
  ok &= expect("score_at valid, no device",
               mis_score_labels_at(pos_ok, 2, 100, t, 64, t, 1000, MIS_BF16, labels, 2, 0, sc, t, 1 << 20, nullptr),
               MIS_ERR_HIP);

  // ---- kernel choice
  ok &= expect("choice unknown attention", mis_set_kernel_choice("fastest", nullptr), MIS_ERR_ARG);
  ok &= expect("choice unknown score", mis_set_kernel_choice(nullptr, "wide7"), MIS_ERR_ARG);
  ok &= expect("choice valid", mis_set_kernel_choice("pipe32", "wide5"), MIS_OK);
  ok &= expect("choice reset", mis_set_kernel_choice(nullptr, nullptr), MIS_OK);
  ++g_checks;
  if (std::strncmp(mis_version(), "mis-gfx950", 10) != 0) {
    std::fprintf(stderr, "FAILED version string '%s'\n", mis_version());
    ok = false;
  }
  if (!ok) return 1;
  std::printf("ok %d checks\n", g_checks);
  return 0;
}
