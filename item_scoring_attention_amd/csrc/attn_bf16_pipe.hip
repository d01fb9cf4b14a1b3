// bf16 MIS prefill attention on CDNA4 MFMA (gfx950) with a software-pipelined
// key-tile loop: 64 query rows per wave (attn_pipe_kernel<HP, 1>) or 32 rows
// per wave and two waves per SIMD (attn_pipe_kernel<2, 2>).
//
// Computes O = softmax(scale * Q K^T + M) V per query head with the mask M of
// From Generation to Scoring, §4.1, Eq. 4 (a prefix row sees the prefix up to
// itself; an item row sees the whole prefix and its own item up to itself),
// visiting only the key tiles a query tile can see (§4.3: the MIS kernels
// skip fully masked tiles; the SGLang blog lists the same change for its
// FlashInfer kernels).
//
// Why 64 rows per wave: a K or V^T fragment read from LDS then feeds two
// MFMAs (two 32-row query blocks) instead of one. With 32 rows per wave the
// transposing V^T reads alone (ds_read_b64_tr_b16 moves half the bytes of a
// ds_read_b128 per instruction) cap the PV product below the MFMA rate. The
// price is registers: O^T (128) and Q^T (64) live in AGPRs, S, P and the
// fragment rings in VGPRs, one wave per SIMD. The 32-row loop fits two waves
// per SIMD, so one workgroup's start and finish overlap another's loop.
//
// Work decomposition: a workgroup takes one 64-token query tile, one KV head
// and HP of its query heads; with TB = 1 one wave per head owns the 64 rows,
// with TB = 2 two waves per head own 32 rows each. It stages each 64-key K
// and V tile once for all its waves. <4, 1> runs one workgroup per CU, <2, 1>
// and <2, 2> two.
// The KV head varies fastest over blockIdx, so with 8 KV heads each XCD (the
// dispatcher deals workgroups round-robin to the 8 XCDs) serves one KV head
// from its own L2. Query tiles arrive longest first (the builder's work list).
//
// The key-tile loop is one inline-assembly block (attn_loop.inc, written by
// gen_attn_loop.py, which documents the register map and the pipeline). The
// compiler cannot keep this split of AGPR and VGPR state apart by itself: it
// moves the accumulators between the two files on every step.
//
// Layouts (shared with the LDS-direct loads the block issues):
//   LDS: the K stages, then the V stages, 16 KB each, 64 keys x 256-byte
//   rows; chunk c (16 bytes) of K row r sits in slot c ^ (r & 15), of V row
//   r in slot c ^ 4 (r & 3), so the K reads (ds_read_b128, 16
//   consecutive keys at one chunk) and the transposing V reads are free of
//   bank conflicts.
//   MFMA v_mfma_f32_32x32x16_bf16: S^T = K Q^T with the keys on the rows, so a
//   lane owns one query column and P^T leaves the accumulator already in the
//   B-operand layout of O^T += V^T P^T; V^T comes from ds_read_b64_tr_b16 in
//   the key order the accumulator implies (keys {4g..4g+3, 8+4g..8+4g+3} of a
//   16-key step in the eight slots of lane group g).
#include "attn_loop.inc"
#include "gfx950_util.h"
#include "mis_internal.h"
#include "rope_math.h"

namespace mis {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

constexpr int D = 128;
constexpr int BM = kAttnBlockM;  // query tokens per workgroup (and per wave)
constexpr int BN = kAttnBlockN;  // keys per LDS tile
constexpr int TILE = BN * D;     // bf16 elements of one K or V stage
constexpr float kLog2e = 1.4426950408889634f;
static_assert(BM == 64 && BN == 64, "the loop block is written for 64 x 64 tiles");

// Scalars and per-lane values the loop block reads (names as in the block).
struct LoopArgs {
  uint32_t ka[8];   // LDS byte address of this lane's K fragment slot, per 16-dim step
  uint32_t va[4];   // LDS byte address of this lane's V^T read, per 32-dim block
  uint32_t ko[8];   // byte offset of this lane's K chunk in a tile, per LDS-direct load of the wave
  uint32_t vo[8];   // same for V
  int rjt[2];       // last visible key of the lane's two query rows, minus 4g
  int rjb[2];       // first key of the rows' own item (0 for prefix rows), minus 4g
  int rlq;          // prefix length minus 4g
  uint32_t sel;     // A operand of the row-sum MFMAs: bf16 (1, 1) or (0, 0), by lane
  int nvis, a_end, b_start, a_full;
  uint32_t kb_lo, kb_hi, vb_lo, vb_hi;  // this KV head's K and V at the request start
  uint32_t rb64, nrec;                  // 64 token rows in bytes; descriptor range
  uint32_t wlds;                        // LDS address of this wave's first DMA row
  float c;                              // softmax scale * log2(e)
};

// Per-lane offsets of the LDS-direct loads: 4 or 8 loads per wave, tile and operand.
#define MIS_ATTN_KV4                                                                                                \
  [ko0] "v"(x.ko[0]), [ko1] "v"(x.ko[1]), [ko2] "v"(x.ko[2]), [ko3] "v"(x.ko[3]), [vo0] "v"(x.vo[0]),            \
      [vo1] "v"(x.vo[1]), [vo2] "v"(x.vo[2]), [vo3] "v"(x.vo[3])
#define MIS_ATTN_KV8                                                                                                \
  MIS_ATTN_KV4, [ko4] "v"(x.ko[4]), [ko5] "v"(x.ko[5]), [ko6] "v"(x.ko[6]), [ko7] "v"(x.ko[7]),                 \
      [vo4] "v"(x.vo[4]), [vo5] "v"(x.vo[5]), [vo6] "v"(x.vo[6]), [vo7] "v"(x.vo[7])

#define MIS_ATTN_LOOP_OPERANDS(KV)                                                                                  \
  : [o0] "={a[0:31]}"(o0), [o1] "={a[32:63]}"(o1), [o2] "={a[64:95]}"(o2), [o3] "={a[96:127]}"(o3),              \
    [l0] "=v"(l0), [l1] "=v"(l1)                                                                                    \
  : [q0] "{a[128:159]}"(q0), [q1] "{a[160:191]}"(q1), [ka0] "v"(x.ka[0]), [ka1] "v"(x.ka[1]),                    \
    [ka2] "v"(x.ka[2]), [ka3] "v"(x.ka[3]), [ka4] "v"(x.ka[4]), [ka5] "v"(x.ka[5]), [ka6] "v"(x.ka[6]),            \
    [ka7] "v"(x.ka[7]), [va0] "v"(x.va[0]), [va1] "v"(x.va[1]), [va2] "v"(x.va[2]), [va3] "v"(x.va[3]), KV,        \
    [rjt0] "v"(x.rjt[0]), [rjt1] "v"(x.rjt[1]), [rjb0] "v"(x.rjb[0]), [rjb1] "v"(x.rjb[1]), [rlq] "v"(x.rlq),     \
    [sel] "v"(x.sel),                                                                                             \
    [nvis] "s"(x.nvis), [a_end] "s"(x.a_end), [b_start] "s"(x.b_start), [a_full] "s"(x.a_full),                   \
    [kb_lo] "s"(x.kb_lo), [kb_hi] "s"(x.kb_hi), [vb_lo] "s"(x.vb_lo), [vb_hi] "s"(x.vb_hi), [rb64] "s"(x.rb64),    \
    [nrec] "s"(x.nrec), [wlds] "s"(x.wlds), [c] "s"(x.c)                                                          \
  : MIS_ATTN_LOOP_CLOBBERS

#define MIS_ATTN_LOOP_OPERANDS_QB1                                                                                  \
  : [o0] "={a[0:31]}"(o0), [o1] "={a[32:63]}"(o1), [l0] "=v"(l0)                                                   \
  : [q0] "{a[64:95]}"(q0), [ka0] "v"(x.ka[0]), [ka1] "v"(x.ka[1]), [ka2] "v"(x.ka[2]), [ka3] "v"(x.ka[3]),         \
    [ka4] "v"(x.ka[4]), [ka5] "v"(x.ka[5]), [ka6] "v"(x.ka[6]), [ka7] "v"(x.ka[7]), [va0] "v"(x.va[0]),            \
    [va1] "v"(x.va[1]), [va2] "v"(x.va[2]), [va3] "v"(x.va[3]), MIS_ATTN_KV4, [rjt0] "v"(x.rjt[0]),               \
    [rjb0] "v"(x.rjb[0]), [rlq] "v"(x.rlq), [sel] "v"(x.sel), [nvis] "s"(x.nvis), [a_end] "s"(x.a_end),          \
    [b_start] "s"(x.b_start),                                                                                     \
    [a_full] "s"(x.a_full), [kb_lo] "s"(x.kb_lo), [kb_hi] "s"(x.kb_hi), [vb_lo] "s"(x.vb_lo),                     \
    [vb_hi] "s"(x.vb_hi), [rb64] "s"(x.rb64), [nrec] "s"(x.nrec), [wlds] "s"(x.wlds), [c] "s"(x.c)                \
  : MIS_ATTN_LOOP_CLOBBERS_QB1

// The ring's first loads (a block of their own, issued with the kernel's own
// loads); the loop block then finds them landed.
#define MIS_ATTN_PROLOGUE_OPERANDS(KV)                                                                              \
  ::KV, [nvis] "s"(x.nvis), [a_end] "s"(x.a_end), [b_start] "s"(x.b_start), [kb_lo] "s"(x.kb_lo),                 \
    [kb_hi] "s"(x.kb_hi), [vb_lo] "s"(x.vb_lo), [vb_hi] "s"(x.vb_hi), [rb64] "s"(x.rb64), [nrec] "s"(x.nrec),     \
    [wlds] "s"(x.wlds)                                                                                            \
  : MIS_ATTN_PROLOGUE_CLOBBERS

// Runs the whole key-tile loop; O^T (unnormalised) and the row sums of the
// lane's two query rows come back. DPW = LDS-direct loads per wave, tile and operand (16 / HP).
template <int DPW>
__device__ __forceinline__ void attn_loop(const LoopArgs &x, const f32x32 &q0, const f32x32 &q1, f32x32 &o0,
                                          f32x32 &o1, f32x32 &o2, f32x32 &o3, float &l0, float &l1) {
  static_assert(DPW == 4 || DPW == 8, "loop block generated for 2 or 4 heads per workgroup");
  // The block writes M0 (the LDS address of its loads). Clang warns that a
  // reserved register is listed as clobbered; the compiler sets M0 itself
  // before each of its own uses, and none follows the block.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (DPW == 4)
    asm volatile(MIS_ATTN_LOOP_TEXT_DPW4 MIS_ATTN_LOOP_OPERANDS(MIS_ATTN_KV4));
  else
    asm volatile(MIS_ATTN_LOOP_TEXT_DPW8 MIS_ATTN_LOOP_OPERANDS(MIS_ATTN_KV8));
#pragma clang diagnostic pop
}

// The same loop for 32 query rows per wave (one query block): four waves
// load a tile, two K/V stages, and the wave fits in 256 registers.
__device__ __forceinline__ void attn_loop_qb1(const LoopArgs &x, const f32x32 &q0, f32x32 &o0, f32x32 &o1,
                                              float &l0) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(MIS_ATTN_LOOP_TEXT_QB1 MIS_ATTN_LOOP_OPERANDS_QB1);
#pragma clang diagnostic pop
}

// HP heads x TB row blocks per workgroup, one wave each: TB = 1 gives a wave
// 64 query rows (two 32-row query blocks, one wave per SIMD), TB = 2 gives it
// 32 rows (two waves per SIMD). K/V stages of the ring: four when one
// workgroup holds the CU (HP = 4, TB = 1: 128 KB of LDS), two when two
// workgroups share it (64 KB each).
template <int HP, int TB>
constexpr int kStages = HP == 4 && TB == 1 ? 4 : 2;

template <int HP, int TB>
__global__ __launch_bounds__(64 * HP * TB, TB) void attn_pipe_kernel(
    const int32_t *__restrict__ work, const int32_t *__restrict__ cu_seqlens,
    const int32_t *__restrict__ prefix_lens, const int32_t *__restrict__ cu_tiles,
    const int8_t *__restrict__ tile_class, const int32_t *__restrict__ pos_id, const __bf16 *__restrict__ q,
    const __bf16 *__restrict__ k, const __bf16 *__restrict__ v, __bf16 *__restrict__ o, int hq,
    int hkv, float c, int items_only, const float *__restrict__ rope_cs) {
  constexpr int NW = HP * TB;                // waves
  constexpr int QB = 2 / TB;                 // 32-row query blocks per wave
  constexpr int ROWS_PER_WAVE = BN / NW;     // tile rows each wave loads
  constexpr int STAGES = kStages<HP, TB>;
  static_assert(NW == 2 || NW == 4, "the loop blocks are generated for 8 or 4 loads per wave and tile");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[2 * STAGES * TILE];  // K stages, then V stages

  const int gsz = hq / hkv;
  const int groups = gsz / HP;
  const int kvh = blockIdx.x % hkv;
  const int rest = blockIdx.x / hkv;
  const int hc = rest % groups;
  const int w = rest / groups;

  const int r = work[4 * w + 0];
  const int qt = work[4 * w + 1];
  const int a_end = work[4 * w + 2];  // prefix key tiles [0, a_end)
  const int b_lo = work[4 * w + 3];   // first key tile of the own-item range
  const int base = cu_seqlens[r];
  const int Tr = cu_seqlens[r + 1] - base;
  const int lq = prefix_lens[r];
  // Appending items to a cached prefix: a query tile that holds prefix rows
  // only has nothing to compute (the whole workgroup leaves together).
  if (items_only && qt * BM + BM <= lq) return;
  const int nkt = (Tr + BN - 1) / BN;
  const int j1 = min(Tr, qt * BM + BM);
  const int b_hi = (j1 + BN - 1) / BN;
  const int b_start = max(b_lo, a_end);
  const int n_visit = a_end + (b_hi - b_start);
  const int cls_base = cu_tiles[r] + qt * nkt;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int ql = lane & 31;
  const int hp = wave / TB;
  const int tb = wave % TB;  // row block: rows 32 tb .. of the query tile (TB = 2)
  const int head = kvh * gsz + hc * HP + hp;
  const int row0 = qt * BM + 32 * tb;  // first query row of the wave

  const int64_t q_stride = int64_t(hq) * D;
  const int64_t kv_stride = int64_t(hkv) * D;
  const uint32_t kv_row_bytes = uint32_t(kv_stride) * 2u;

  // The V stages start as zeros: rows past the request end are not written
  // by the loads, and the first PV step multiplies a zero P with the last
  // stage. Done first, so the ring's first loads can go out with the kernel's
  // own (below) once every wave's stores are in LDS.
  for (int i = tid; i < STAGES * TILE / 8; i += 64 * NW)
    *reinterpret_cast<uint4 *>(&smem[STAGES * TILE + i * 8]) = make_uint4(0, 0, 0, 0);

  LoopArgs x;
  x.nvis = n_visit;
  x.a_end = a_end;
  x.b_start = b_start;
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t vlds0 = lds0 + uint32_t(STAGES * TILE * 2);  // start of the V stages
  // K fragment of 16-dim step kk: key ql (+32 for the second key block), chunk 2 kk + g.
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) x.ka[kk] = lds0 + uint32_t(ql) * 256u + 16u * uint32_t((2 * kk + g) ^ (ql & 15));
  // V^T reads: in a 16-lane group G, lanes 4e..4e+3 read key 4 (G / 2) + e (and
  // eight rows further), dims 32 db + 16 (G % 2) + 4 (lane % 4); the transpose
  // hands lane i of the group dim 32 db + 16 (G % 2) + i of four keys.
  {
    const int G = lane >> 4, e = (lane >> 2) & 3, qd = lane & 3;
    const int key = 4 * (G >> 1) + e;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = 4 * db + 2 * (G & 1) + (qd >> 1);
      x.va[db] = vlds0 + uint32_t(key) * 256u + 16u * uint32_t(chunk ^ (4 * (key & 3))) + 8u * uint32_t(qd & 1);
    }
  }
  // LDS-direct loads: instruction i of a wave covers tile rows ROWS_PER_WAVE *
  // wave + 4 i + lane / 16, LDS slot lane % 16, so the lane fetches global
  // chunk slot ^ swizzle(row) (ROWS_PER_WAVE is a multiple of 16, so the K
  // swizzle depends on i % 4 and lane / 16 only). The whole offset of the
  // row inside the tile sits in the per-lane offset: the buffer range check
  // covers that offset but not the scalar one, and rows past the request's
  // end must fail it.
  const uint32_t wrow = uint32_t(ROWS_PER_WAVE * wave);
  {
    const int rl = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t row = wrow + uint32_t(4 * i + rl);
      x.ko[i] = row * kv_row_bytes + 16u * uint32_t(slot ^ ((4 * i + rl) & 15));
      x.vo[i] = row * kv_row_bytes + 16u * uint32_t(slot ^ (4 * (rl & 3)));
    }
  }
  const uint64_t kb = reinterpret_cast<uint64_t>(k + int64_t(base) * kv_stride + int64_t(kvh) * D);
  const uint64_t vb = reinterpret_cast<uint64_t>(v + int64_t(base) * kv_stride + int64_t(kvh) * D);
  x.kb_lo = uint32_t(kb);
  x.kb_hi = uint32_t(kb >> 32);
  x.vb_lo = uint32_t(vb);
  x.vb_hi = uint32_t(vb >> 32);
  x.rb64 = 64u * kv_row_bytes;
  // A tile descriptor starting at key k0 covers nrec - k0 * row bytes: up to
  // this head's last key of the request, so rows past the end read nothing.
  x.nrec = uint32_t(Tr) * kv_row_bytes - uint32_t(kvh) * D * 2u;
  x.wlds = lds0 + wrow * 256u;
  x.c = c;
  x.rlq = lq - 4 * g;
  // Row sums on v_mfma_f32_16x16x32_bf16 with P^T as the B operand: lane
  // l's A values select the k-groups (lanes / 16) of the same parity as its
  // output rows' group, so each lane's accumulator holds its own query's
  // sum: A[m][k] = 1 where (k / 8) % 2 == (m / 4) % 2, and lane l holds
  // A[l % 16][8 (l / 16) ..].
  x.sel = (((lane >> 4) ^ (lane >> 2)) & 1) == 0 ? 0x3f803f80u : 0u;

  // Every wave's zero stores are in LDS before any load lands there (an LDS
  // wait and a barrier; no fence, which would wait for vector memory too).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // The kernel's own loads, issued together, their results used only after
  // the ring's first loads are out too (one round trip for all of them).
  // Q^T operands of the wave's query blocks; rows past the request end read as zeros.
  f32x32 qv[QB];
  {
    const uint32_t q_bytes = uint32_t(Tr) * uint32_t(q_stride) * 2u - uint32_t(head) * D * 2u;
    const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(q + int64_t(base) * q_stride + int64_t(head) * D), 0, q_bytes, kRsrcWord3);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t qo = uint32_t(row0 + 32 * qb + ql) * uint32_t(q_stride) * 2u + 16u * g;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const f32x4 f = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qrsrc, qo + 32u * kk, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[qb][4 * kk + e] = f[e];
      }
    }
  }
  // classes of visits lane + 64 u, issued with the kernel's own loads so
  // that their latency is paid once (lanes past the last visit read visit
  // 0's tile); tiles with more visits scan the rest after the ring's start
  auto visit_tile = [&](int idx) { return idx < a_end ? idx : b_start + (idx - a_end); };
  constexpr int KCU = 8;
  int tcs[KCU];
#pragma unroll
  for (int u = 0; u < KCU; ++u) {
    const int idx = lane + 64 * u;
    tcs[u] = 2;
    if (u == 0 || 64 * u < n_visit)
      tcs[u] = tile_class[cls_base + (idx < n_visit ? visit_tile(idx) : visit_tile(0))];
  }
  // position ids of the lane's query rows (rows past the request end read the last row)
  int pos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) pos[qb] = pos_id[base + min(row0 + 32 * qb + ql, Tr - 1)];

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (QB == 1)
    asm volatile(MIS_ATTN_PROLOGUE_TEXT_QB1 MIS_ATTN_PROLOGUE_OPERANDS(MIS_ATTN_KV4));
  else if constexpr (BN / HP / 4 == 4)
    asm volatile(MIS_ATTN_PROLOGUE_TEXT_DPW4 MIS_ATTN_PROLOGUE_OPERANDS(MIS_ATTN_KV4));
  else
    asm volatile(MIS_ATTN_PROLOGUE_TEXT_DPW8 MIS_ATTN_PROLOGUE_OPERANDS(MIS_ATTN_KV8));
#pragma clang diagnostic pop

  // Visits before a_full are fully visible tiles (class 2) that end inside
  // the request; the mask runs on every visit from a_full on.
  {
    int first = n_visit;
#pragma unroll
    for (int u = 0; u < KCU; ++u) {
      const int idx = lane + 64 * u;
      if (idx < n_visit) {
        const int kt = visit_tile(idx);
        if ((tcs[u] != 2) | (kt * BN + BN > Tr)) first = min(first, idx);
      }
    }
    for (int i0 = 64 * KCU; i0 < n_visit; i0 += 64) {
      const int idx = i0 + lane;
      if (idx < n_visit) {
        const int kt = visit_tile(idx);
        if ((tile_class[cls_base + kt] != 2) | (kt * BN + BN > Tr)) first = min(first, idx);
      }
    }
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) first = min(first, __shfl_xor(first, s));
    x.a_full = __builtin_amdgcn_readfirstlane(first);
  }

  // Mask bounds of the lane's query rows (j = row0 + query block * 32 + lane % 32);
  // the lane's keys in a sub-tile are key0 + 8 (a / 4) + a % 4 + 4 g.
  x.rjt[1] = x.rjb[1] = 0;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int j = row0 + 32 * qb + ql;
    // an item row at offset d of its item has position id lq + d (the
    // reused positions), so its item starts at row j - d
    const int jb = (j < Tr && j >= lq) ? j - (pos[qb] - lq) : 0;
    x.rjt[qb] = min(j, Tr - 1) - 4 * g;
    x.rjb[qb] = jb - 4 * g;
  }

  // Q rotated here when the caller passes the rotary table (cos, sin of
  // every position and pair, the rotation pass's values): lane half g holds
  // dims 16 kk + 8 g .. + 7 of both halves of its head row (kk and kk + 4),
  // so every pair (i, i + 64) is in the lane's own registers.
  if (rope_cs) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float4 *tp = reinterpret_cast<const float4 *>(rope_cs + int64_t(pos[qb]) * D);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        float cs[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 t = tp[8 * kk + 4 * g + u];
          cs[4 * u] = t.x, cs[4 * u + 1] = t.y, cs[4 * u + 2] = t.z, cs[4 * u + 3] = t.w;
        }
        f32x4 flo, fhi;
#pragma unroll
        for (int e = 0; e < 4; ++e) flo[e] = qv[qb][4 * kk + e], fhi[e] = qv[qb][4 * (kk + 4) + e];
        bf16x8 lo = __builtin_bit_cast(bf16x8, flo), hi = __builtin_bit_cast(bf16x8, fhi);
        rope_rotate8(lo, hi, cs);
        flo = __builtin_bit_cast(f32x4, lo);
        fhi = __builtin_bit_cast(f32x4, hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[qb][4 * kk + e] = flo[e], qv[qb][4 * (kk + 4) + e] = fhi[e];
      }
    }
  }

  f32x32 o0, o1, o2, o3;
  float l0, l1 = 1.f;
  if constexpr (QB == 2)
    attn_loop<BN / HP / 4>(x, qv[0], qv[QB - 1], o0, o1, o2, o3, l0, l1);
  else
    attn_loop_qb1(x, qv[0], o0, o1, l0);

  // O^T accumulator element a of lane l: dim 8 (a / 4) + 4 g + a % 4 of the
  // 32-dim block, query row l % 32 of the block. l0 and l1 are the full row
  // sums of the lane's query rows.
  const float inv0 = 1.0f / l0;
  const float inv1 = 1.0f / l1;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int j = row0 + 32 * qb + ql;
    if (j >= Tr) continue;
    const float inv = qb ? inv1 : inv0;
    __bf16 *op = o + int64_t(base + j) * q_stride + int64_t(head) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const f32x32 &ob = qb ? (db < 2 ? o2 : o3) : (db < 2 ? o0 : o1);
      const int off = 16 * (db & 1);
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = __bf16(ob[off + 4 * a4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * a4 + 4 * g) = ov;
      }
    }
  }
}

template <int HP, int TB>
hipError_t launch_pipe(const mis_segments &seg, const void *q, const void *k, const void *v, void *o, int hq,
                       int hkv, float c, int items_only, const float *rope_cs, hipStream_t st) {
  const int64_t blocks = int64_t(seg.num_work) * hq / HP;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  attn_pipe_kernel<HP, TB><<<dim3(unsigned(blocks)), 64 * HP * TB, 0, st>>>(
      seg.work, seg.cu_seqlens, seg.prefix_lens, seg.cu_tiles, seg.tile_class, seg.pos_id,
      static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k), static_cast<const __bf16 *>(v),
      static_cast<__bf16 *>(o), hq, hkv, c, items_only, rope_cs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16_pipe(const mis_segments &seg, const void *q, const void *k, const void *v, void *o,
                                      int hq, int hkv, float scale, int items_only, int heads, const float *rope_cs,
                                      hipStream_t st) {
  const int gsz = hq / hkv;
  if (gsz % heads != 0 || (heads != 2 && heads != 4)) return hipErrorInvalidValue;
  const float c = scale * kLog2e;
  // 4 heads per workgroup share each staged K/V tile among 4 waves (one
  // workgroup per CU, a 4-stage ring); 2 heads run two workgroups per CU.
  if (heads == 4) return launch_pipe<4, 1>(seg, q, k, v, o, hq, hkv, c, items_only, rope_cs, st);
  return launch_pipe<2, 1>(seg, q, k, v, o, hq, hkv, c, items_only, rope_cs, st);
}

hipError_t launch_attention_bf16_pipe32(const mis_segments &seg, const void *q, const void *k, const void *v,
                                        void *o, int hq, int hkv, float scale, int items_only, const float *rope_cs,
                                        hipStream_t st) {
  const int gsz = hq / hkv;
  if (gsz % 2 != 0) return hipErrorInvalidValue;
  // 2 heads x 2 row blocks of 32 per workgroup, two workgroups per CU.
  return launch_pipe<2, 2>(seg, q, k, v, o, hq, hkv, scale * kLog2e, items_only, rope_cs, st);
}

}  // namespace mis
