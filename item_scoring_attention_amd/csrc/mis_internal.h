// Internal declarations shared by the host ABI (abi.cpp) and the HIP kernel
// sources. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "mis.h"

namespace mis {

// Tile shape of the bf16 MFMA attention kernel: 64 query tokens x 64 keys.
constexpr int kAttnBlockM = 64;
constexpr int kAttnBlockN = 64;

// Vocabulary rows per workgroup of the scoring kernels (one partial
// (max, sum-exp) pair per item and vocabulary tile).
constexpr int kScoreBlockV = 128;

struct LabelArgs {
  int32_t k;
  int32_t ids[MIS_MAX_LABELS];
};

// Builder: per-item begin/readout, per-token item/position ids, per-tile
// classes. item_starts is request-relative (as the caller gave it).
hipError_t launch_segments(const mis_segments &seg, const int32_t *item_starts_dev,
                           hipStream_t stream);

// Metadata small enough to travel in the builder's kernel arguments: the
// staged arrays packed back to back (kInlineWords int32 at most) and, per
// array, its word offset there, its word offset in the segment buffer and
// its length. Array order: cu_seqlens, prefix_lens, cu_items, cu_tiles,
// item_starts, work.
constexpr int kInlineWords = 768;
constexpr int kInlineArrays = 6;
struct InlineMeta {
  int32_t w[kInlineWords];
};
struct InlineLayout {
  int32_t src[kInlineArrays], dst[kInlineArrays], len[kInlineArrays];
};
hipError_t launch_segments_inline(const mis_segments &seg, const InlineLayout &lay, const InlineMeta &meta,
                                  int32_t *stage, hipStream_t stream);

// items_only != 0: rows of query tiles that hold prefix rows only are not
// computed (appending items to a cached prefix).
hipError_t launch_attention_f32(const mis_segments &seg, const float *q, const float *k,
                                const float *v, float *o, int hq, int hkv, int d, float scale,
                                int items_only, hipStream_t stream);

// Compute units of the current device (queried once per device).
int device_cus();

// The bf16 attention kernels and the rule that picks one per call.
enum class AttnKernel : int {
  Pipe4 = 0,    // attn_pipe_kernel<4, 1>: 64 query rows per wave, 4 heads per workgroup
  Pipe2 = 1,    // attn_pipe_kernel<2, 1>: 64 query rows per wave, 2 heads per workgroup
  Pipe32 = 2,   // attn_pipe_kernel<2, 2>: 32 query rows per wave, two waves per SIMD
  Classic2 = 3, // attn_dma_kernel<2, 2>: plain loop, 2 heads x 2 row blocks
  Classic1 = 4, // attn_dma_kernel<2, 1>: plain loop, 1 head x 2 row blocks (odd group sizes)
};
// A caller's forced choice (tests, A/B comparisons); Auto = by shape.
enum class AttnForce : int { Auto = 0, Pipe = 1, Pipe32 = 2, Classic = 3, Pipe2 = 4 };
AttnKernel pick_attention_bf16(const mis_segments &seg, int hq, int hkv, AttnForce force);
const char *attention_bf16_name(AttnKernel k);

// rope_cs: NULL, or the rotary table [positions][d/2] of float (cos, sin)
// pairs; Q is then rotated at the rows' position ids as it is loaded.
hipError_t launch_attention_bf16(const mis_segments &seg, const void *q, const void *k,
                                 const void *v, void *o, int hq, int hkv, int d, float scale,
                                 int items_only, AttnKernel kernel, const float *rope_cs, hipStream_t stream);

// 64 query rows per wave, software-pipelined key-tile loop, `heads` (2 or 4,
// dividing the GQA group) query heads per workgroup, head_dim 128;
// launch_attention_bf16 dispatches to it.
hipError_t launch_attention_bf16_pipe(const mis_segments &seg, const void *q, const void *k,
                                      const void *v, void *o, int hq, int hkv, float scale,
                                      int items_only, int heads, const float *rope_cs, hipStream_t stream);

// The same loop with 32 query rows per wave, two waves per SIMD (even GQA
// group sizes, head_dim 128).
hipError_t launch_attention_bf16_pipe32(const mis_segments &seg, const void *q, const void *k,
                                        const void *v, void *o, int hq, int hkv, float scale,
                                        int items_only, const float *rope_cs, hipStream_t stream);

// Inverse frequencies theta^(-2i/D) of the rotary embedding, i < D/2.
struct RopeFreq {
  double inv[64];
};

// Rotates Q (hq heads; q may be NULL with hq == 0) and K in place at the
// segment position ids.
hipError_t launch_rope(const mis_segments &seg, void *q, void *k, mis_dtype dt, int hq, int hkv, int d,
                       const RopeFreq &freq, hipStream_t stream);
// table [npos][d/2] of float (cos, sin) pairs, the rotation pass's angles.
hipError_t launch_rope_table(float *table, int npos, int d, const RopeFreq &freq, hipStream_t stream);

// Scoring workspace layout: partial maxima [nvt][N], partial sum-exp
// [nvt][N], label logits [N][K] (all float32), then N int32 readout
// positions (used by mis_score_labels_at).
inline int score_vocab_tiles(int vocab) { return (vocab + kScoreBlockV - 1) / kScoreBlockV; }

// Device address, on the current device, of the library's own scoring
// workspace (MIS_SCORE_SCRATCH_BYTES, a static device array in score.hip);
// looked up once per device and kept. Allocates nothing.
hipError_t score_scratch(void **ptr);

// The LM-head kernels and the rule that picks one per call.
enum class ScoreKind : int {
  Narrow = 0,  // score_lds_kernel<NI, NS>: 128 vocabulary rows x 32 NI items (NI 1, 2, 4)
  Wide = 1,    // score_wide_kernel<NI, NS>: 256 vocabulary rows x 32 NI items (NI 3, 4, 5, 6, 8)
  Global = 2,  // score_bf16_kernel<NI>: operands from global memory (H % 64 != 0)
  F32 = 3,     // score_f32_kernel
  Persist = 4, // score_persist_kernel<NI, 3>: the wide tiles, persistent workgroups with loader waves
};
struct ScoreKernel {
  ScoreKind kind;
  int ni;  // item blocks of 32 per workgroup tile
};
// A caller's forced choice: Auto, the narrow tiles, wide tiles with
// force_ni item blocks (0: blocks chosen by shape), or the persistent wide
// tiles (item blocks 3-5). Ignored where the forced kernel does not apply
// (fp32, H % 64 != 0; the persistent tiles need H >= 128 and fall back to
// the wide ones).
enum class ScoreForce : int { Auto = 0, Narrow = 1, Wide = 2, Persist = 3 };
ScoreKernel pick_score(int num_rows, int h, mis_dtype dt, ScoreForce force, int force_ni);
// Writes the kernel's name into buf (at most n bytes).
void score_kernel_name(const ScoreKernel &k, char *buf, size_t n);

// N rows of label scores from the hidden rows at readout_pos[0 .. N-1].
hipError_t launch_score(const int32_t *readout_pos, int num_rows, const void *hidden, int h, const void *lm_head,
                        int vocab, mis_dtype dt, const LabelArgs &labels, int apply_softmax,
                        float *scores, float *ws, const ScoreKernel &kernel, hipStream_t stream);

}  // namespace mis
