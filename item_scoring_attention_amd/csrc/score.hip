// Label scoring: readout gather -> item x vocabulary LM-head contraction ->
// split-vocabulary logsumexp -> label log-probs.
//
// From Generation to Scoring, §3.3 (Eq. 2): the score comes from the
// next-token logits at the item's last token. The JEV post ("Why a Decision
// Workload Deserves a Scoring Interface") keeps the full-vocabulary
// projection and normalisation even when only a few label columns are
// returned, and the Score API returns one row per item in label order, or a
// softmax over the labels with apply_softmax.
//
// Pass 1 (one workgroup per 128 vocabulary rows x an item tile): gather the
// readout hidden rows, contract them with the LM-head rows on MFMA (fp32
// accumulation), and reduce each item's logits over the tile to a partial
// (max, sum exp(z - max)) with wavefront reductions. Label logits are copied
// out in fp32 by the lane that holds them. Full logits never reach memory.
// Pass 2 (one wave per item): merge the partials exactly,
// lse = M + log(sum_c s_c * exp(m_c - M)), and write z_label - lse (or the
// softmax over the label logits).
#include <algorithm>
#include <cstdio>
#include <mutex>

#include "gfx950_util.h"
#include "mis_internal.h"

namespace mis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int BV = kScoreBlockV;

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ------------------------------------------- bf16 MFMA, any H % 32 == 0
// Operands straight from global memory (used when H is not a multiple of 64).
// 4 waves: wv = wave & 1 picks 64 vocabulary rows, wn = wave >> 1 picks
// 32*NI items. Workgroup tile: 128 rows x 64*NI items.
template <int NI>
__global__ __launch_bounds__(256) void score_bf16_kernel(
    const __bf16 *__restrict__ hidden, const __bf16 *__restrict__ w, int H, int V, int N,
    const int32_t *__restrict__ readout_pos, LabelArgs labels, float *__restrict__ pmax,
    float *__restrict__ psum, float *__restrict__ plab, int nvt) {
  constexpr int BI = 64 * NI;
  __shared__ float red[2][2][NI][32];  // [wv][wn][ni][item column] cross-wave exchange

  const int vt = blockIdx.x;
  const int v0 = vt * BV;
  const int n0 = blockIdx.y * BI;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, ql = lane & 31;
  const int wv = wave & 1, wn = wave >> 1;

  const __bf16 *arow[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int vr = min(v0 + 64 * wv + 32 * mi + ql, V - 1);
    arow[mi] = w + int64_t(vr) * H + 8 * g;
  }
  const __bf16 *brow[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const int n = min(n0 + 32 * (NI * wn + ni) + ql, N - 1);
    brow[ni] = hidden + int64_t(readout_pos[n]) * H + 8 * g;
  }

  f32x16 acc[2][NI];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[mi][ni][a] = 0.f;

  for (int h = 0; h < H; h += 32) {
    bf16x8 af[2][2], bf[NI][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi][s] = *reinterpret_cast<const bf16x8 *>(arow[mi] + h + 16 * s);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bf[ni][s] = *reinterpret_cast<const bf16x8 *>(brow[ni] + h + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][s], bf[ni][s], acc[mi][ni], 0, 0, 0);
  }

  // Element a of acc[mi][ni] is logit z[vocab row][item], vocab row =
  // v0 + 64*wv + 32*mi + 8*(a/4) + 4*g + a%4, item = n0 + 32*(NI*wn + ni) + ql.
  auto row_of = [&](int mi, int a) { return v0 + 64 * wv + 32 * mi + 8 * (a >> 2) + 4 * g + (a & 3); };

  float m[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    float x = -INFINITY;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        if (row_of(mi, a) < V) x = fmaxf(x, acc[mi][ni][a]);
    x = fmaxf(x, __shfl_xor(x, 32));
    if (g == 0) red[wv][wn][ni][ql] = x;
  }
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) m[ni] = fmaxf(red[0][wn][ni][ql], red[1][wn][ni][ql]);
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    float s = 0.f;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        if (row_of(mi, a) < V) s += fast_exp(acc[mi][ni][a] - m[ni]);
    s += __shfl_xor(s, 32);
    if (g == 0) red[wv][wn][ni][ql] = s;
  }
  __syncthreads();
  if (wv == 0 && g == 0) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = n0 + 32 * (NI * wn + ni) + ql;
      if (n < N) {
        pmax[int64_t(vt) * N + n] = m[ni];
        psum[int64_t(vt) * N + n] = red[0][wn][ni][ql] + red[1][wn][ni][ql];
      }
    }
  }

  // label logits held by this wave
  for (int kx = 0; kx < labels.k; ++kx) {
    const int ro = labels.ids[kx] - v0 - 64 * wv;
    if (ro < 0 || ro >= 64) continue;
    const int mi = ro >> 5, rr = ro & 31;
    if (((rr >> 2) & 1) != g) continue;
    const int at = 4 * (rr >> 3) + (rr & 3);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      float z = 0.f;
#pragma unroll
      for (int a = 0; a < 16; ++a) z = (a == at) ? (mi ? acc[1][ni][a] : acc[0][ni][a]) : z;
      const int n = n0 + 32 * (NI * wn + ni) + ql;
      if (n < N) plab[int64_t(n) * labels.k + kx] = z;
    }
  }
}

// ------------------------------------------ bf16 LDS-staged (H % 64 == 0)
// Workgroup tile: 128 vocabulary rows x 32*NI items (4 waves x 32 rows, each
// wave all the tile's items). With N <= 64 the kernel is a stream: every
// LM-head row is read once and feeds at most two MFMAs per 16 hidden dims.
// With more items the item tiles of one vocabulary tile run on one XCD and
// re-read its W tile from L2; the tile then feeds NI MFMAs per fragment read.
// The hidden dimension is walked in 64-dim chunks. Both operands of a chunk (128 W rows x 64 dims and the
// gathered readout rows, items x 64 dims) go to an NS-deep LDS ring by
// LDS-direct loads: 8 lanes cover one 128-byte line, so every load
// instruction reads 8 whole lines. Chunk c + NS - 1 is issued while chunk c
// is contracted. Past the last chunk the loads are still issued (W at an
// out-of-range buffer offset, which returns zeros without a memory access;
// X re-reading chunk 0) into a slot nobody reads, which keeps the loop free
// of branches and every wait count constant.
// LDS layout of a staged chunk: 128 bytes per row (W row or item), 16-byte
// piece p of row r in slot p ^ ((r >> 1) & 7), so the 16 rows that 16 lanes
// of one ds_read_b128 touch spread over all 64 banks.
// K-slot order inside a chunk: k-step s of half-wave g covers dims
// 32*g + 8*s .. +8 for both operands (any order works if A and B agree).
template <int NI, int NS>
__global__ __launch_bounds__(256) void score_lds_kernel(
    const __bf16 *__restrict__ hidden, const __bf16 *__restrict__ w, int H, int V, int N,
    const int32_t *__restrict__ readout_pos, LabelArgs labels, float *__restrict__ pmax,
    float *__restrict__ psum, float *__restrict__ plab, int nvt, int nit) {
  static_assert(NI == 1 || NI == 2 || NI == 4, "1, 2 or 4 item blocks of 32");
  constexpr int NIT = 32 * NI;                 // items in the tile
  constexpr int WCH = BV * 64;                 // bf16 elements of a staged W chunk
  constexpr int XCH = NIT * 64;                // ... and of a staged X chunk
  constexpr int PER_CHUNK = BV / 32 + NI;      // vector-memory ops per wave per chunk
  // One LDS object for the ring and the epilogue's exchange: with several
  // __shared__ arrays the compiler tags each with an alias scope and makes
  // every LDS read wait for the newest LDS-direct load into the same array.
  struct Smem {
    __bf16 w[NS][WCH];
    __bf16 x[NS][XCH];
    float red[4][NI][32];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto &ws_ = sm.w;
  auto &xs = sm.x;
  auto &red = sm.red;

  // Workgroup b runs on XCD b % 8 (round-robin dispatch). The nit item
  // tiles of one vocabulary tile get consecutive workgroups of the same XCD,
  // so its L2 serves the W tile to all of them.
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int vt = 8 * (jx / nit) + xcd;
  const int n0 = (jx % nit) * NIT;
  if (vt >= nvt) return;  // padding of the vocabulary tile count to a multiple of 8
  const int v0 = vt * BV;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, ql = lane & 31;
  const int piece = lane & 7;

  // W rows v0 .. v0 + 127 (rows past V read as zero). Instruction i of this
  // wave stages rows 32*wave + 8*i .. +8 (lane >> 3 picks the row).
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16 *>(w + int64_t(v0) * H), 0, uint32_t(min(BV, V - v0)) * uint32_t(H) * 2u,
      kRsrcWord3);
  uint32_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    woff[i] = uint32_t(r) * uint32_t(H) * 2u + 16u * uint32_t(piece ^ ((r >> 1) & 7));
  }
  // Readout rows: instruction i of this wave stages items 32*i + 8*wave .. +8.
  const __bf16 *xsrc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = 32 * i + 8 * wave + (lane >> 3);
    xsrc[i] = hidden + int64_t(readout_pos[min(n0 + n, N - 1)]) * H + 8 * (piece ^ ((n >> 1) & 7));
  }

  f32x16 acc[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[ni][a] = 0.f;

  const int nch = H / 64;
  auto issue = [&](int c, int slot) {
    const bool real = c < nch;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_load16(wrs, &ws_[slot][(32 * wave + 8 * i) * 64], real ? woff[i] + 128u * uint32_t(c) : 0x80000000u);
#pragma unroll
    for (int i = 0; i < NI; ++i) lds_load16(xsrc[i] + (real ? 64 * c : 0), &xs[slot][(32 * i + 8 * wave) * 64]);
  };

  // LDS read offsets (elements) of this lane's fragments for k-step s.
  const int wr = 32 * wave + ql;
  int wrd[4], xrd[NI][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    wrd[st] = wr * 64 + 8 * ((4 * g + st) ^ ((wr >> 1) & 7));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = 32 * ni + ql;
      xrd[ni][st] = n * 64 + 8 * ((4 * g + st) ^ ((n >> 1) & 7));
    }
  }

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p, p);
  int slot = 0;
  for (int c = 0; c < nch; ++c) {
    // chunk c landed: this wave's loads (NS - 2 chunks were issued after
    // it), then everyone's; the slot chunk c - 1 used is free again.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * PER_CHUNK));
    barrier_no_fence();
    issue(c + NS - 1, slot == 0 ? NS - 1 : slot - 1);
    const __bf16 *wb = ws_[slot];
    const __bf16 *xb = xs[slot];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8 af = *reinterpret_cast<const bf16x8 *>(wb + wrd[st]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const bf16x8 bfr = *reinterpret_cast<const bf16x8 *>(xb + xrd[ni][st]);
        acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[ni], 0, 0, 0);
      }
    }
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the trailing loads land before the workgroup ends

  // epilogue: element a of acc[ni] is z[row v0 + 32*wave + 8*(a/4) + 4*g + a%4][item n0 + 32*ni + ql]
  auto row_of = [&](int a) { return v0 + 32 * wave + 8 * (a >> 2) + 4 * g + (a & 3); };
  float m[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    float x = -INFINITY;
#pragma unroll
    for (int a = 0; a < 16; ++a)
      if (row_of(a) < V) x = fmaxf(x, acc[ni][a]);
    x = fmaxf(x, __shfl_xor(x, 32));
    if (g == 0) red[wave][ni][ql] = x;
  }
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    m[ni] = fmaxf(fmaxf(red[0][ni][ql], red[1][ni][ql]), fmaxf(red[2][ni][ql], red[3][ni][ql]));
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    float sum = 0.f;
#pragma unroll
    for (int a = 0; a < 16; ++a)
      if (row_of(a) < V) sum += fast_exp(acc[ni][a] - m[ni]);
    sum += __shfl_xor(sum, 32);
    if (g == 0) red[wave][ni][ql] = sum;
  }
  __syncthreads();
  if (wave == 0 && g == 0) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = n0 + 32 * ni + ql;
      if (n < N) {
        pmax[int64_t(vt) * N + n] = m[ni];
        psum[int64_t(vt) * N + n] = red[0][ni][ql] + red[1][ni][ql] + red[2][ni][ql] + red[3][ni][ql];
      }
    }
  }
  for (int kx = 0; kx < labels.k; ++kx) {
    const int ro = labels.ids[kx] - v0 - 32 * wave;
    if (ro < 0 || ro >= 32) continue;
    if (((ro >> 2) & 1) != g) continue;
    const int at = 4 * (ro >> 3) + (ro & 3);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      float z = 0.f;
#pragma unroll
      for (int a = 0; a < 16; ++a) z = (a == at) ? acc[ni][a] : z;
      const int n = n0 + 32 * ni + ql;
      if (n < N) plab[int64_t(n) * labels.k + kx] = z;
    }
  }
}

// Epilogue of the 256-row tiles: element a of acc[mi][ni] of wave w, lane
// (g, ql) is z[row v0 + 64w + 32mi + 8(a/4) + 4g + a%4][item n0 + 32ni + ql].
// Per item: (max, sum exp) over the tile's rows below V, through the 4-wave
// exchange red; label logits copied out exactly by the lane that holds them.
template <int NI>
__device__ __forceinline__ void wide_epilogue(const f32x16 (&acc)[2][NI], float (&red)[4][NI][32], int v0, int vt,
                                              int n0, int V, int N, const LabelArgs &labels, float *pmax,
                                              float *psum, float *plab) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, ql = lane & 31;
  auto row_of = [&](int mi, int a) { return v0 + 64 * wave + 32 * mi + 8 * (a >> 2) + 4 * g + (a & 3); };
  float m[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    float x = -INFINITY;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        if (row_of(mi, a) < V) x = fmaxf(x, acc[mi][ni][a]);
    x = fmaxf(x, __shfl_xor(x, 32));
    if (g == 0) red[wave][ni][ql] = x;
  }
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    m[ni] = fmaxf(fmaxf(red[0][ni][ql], red[1][ni][ql]), fmaxf(red[2][ni][ql], red[3][ni][ql]));
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    float sum = 0.f;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        if (row_of(mi, a) < V) sum += fast_exp(acc[mi][ni][a] - m[ni]);
    sum += __shfl_xor(sum, 32);
    if (g == 0) red[wave][ni][ql] = sum;
  }
  __syncthreads();
  if (wave == 0 && g == 0) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = n0 + 32 * ni + ql;
      if (n < N) {
        pmax[int64_t(vt) * N + n] = m[ni];
        psum[int64_t(vt) * N + n] = red[0][ni][ql] + red[1][ni][ql] + red[2][ni][ql] + red[3][ni][ql];
      }
    }
  }
  for (int kx = 0; kx < labels.k; ++kx) {
    const int ro = labels.ids[kx] - v0 - 64 * wave;
    if (ro < 0 || ro >= 64) continue;
    const int mi = ro >> 5, rr = ro & 31;
    if (((rr >> 2) & 1) != g) continue;
    const int at = 4 * (rr >> 3) + (rr & 3);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      float z = 0.f;
#pragma unroll
      for (int a = 0; a < 16; ++a) z = (a == at) ? (mi ? acc[1][ni][a] : acc[0][ni][a]) : z;
      const int n = n0 + 32 * ni + ql;
      if (n < N) plab[int64_t(n) * labels.k + kx] = z;
    }
  }
}

// ------------------------------- bf16 LDS-staged, wide tiles (H % 64 == 0)
// For many items the contraction is MFMA-bound, and with 32 vocabulary rows
// per wave the fragment reads (one W fragment and NI readout fragments per
// NI MFMAs, every readout fragment read by all four waves) outrun the LDS.
// Here a wave owns 64 vocabulary rows, so a readout fragment feeds two MFMAs:
// workgroup tile 256 rows x 32*NI items, one workgroup per CU, NS-deep ring
// of 64-dim chunks. Staging, swizzle and the epilogue follow score_lds_kernel.
template <int NI, int NS>
__global__ __launch_bounds__(256, 1) void score_wide_kernel(
    const __bf16 *__restrict__ hidden, const __bf16 *__restrict__ w, int H, int V, int N,
    const int32_t *__restrict__ readout_pos, LabelArgs labels, float *__restrict__ pmax,
    float *__restrict__ psum, float *__restrict__ plab, int nvt, int nit) {
  constexpr int BVW = 256;                     // vocabulary rows of the tile
  constexpr int NIT = 32 * NI;                 // items in the tile
  constexpr int WCH = BVW * 64;                // bf16 elements of a staged W chunk
  constexpr int XCH = NIT * 64;                // ... and of a staged X chunk
  constexpr int PER_CHUNK = BVW / 32 + NI;     // vector-memory ops per wave per chunk
  struct Smem {
    __bf16 w[NS][WCH];
    __bf16 x[NS][XCH];
    float red[4][NI][32];
  };
  static_assert(sizeof(Smem) <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto &ws_ = sm.w;
  auto &xs = sm.x;
  auto &red = sm.red;

  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int vt = 8 * (jx / nit) + xcd;
  const int n0 = (jx % nit) * NIT;
  if (vt >= nvt) return;
  const int v0 = vt * BVW;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, ql = lane & 31;
  const int piece = lane & 7;

  // W rows v0 .. v0 + 255 (rows past V read as zero). Instruction i of this
  // wave stages rows 64*wave + 8*i .. +8.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16 *>(w + int64_t(v0) * H), 0, uint32_t(min(BVW, V - v0)) * uint32_t(H) * 2u,
      kRsrcWord3);
  uint32_t woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 64 * wave + 8 * i + (lane >> 3);
    woff[i] = uint32_t(r) * uint32_t(H) * 2u + 16u * uint32_t(piece ^ ((r >> 1) & 7));
  }
  // Readout rows: instruction i of this wave stages items 32*i + 8*wave .. +8.
  const __bf16 *xsrc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = 32 * i + 8 * wave + (lane >> 3);
    xsrc[i] = hidden + int64_t(readout_pos[min(n0 + n, N - 1)]) * H + 8 * (piece ^ ((n >> 1) & 7));
  }

  f32x16 acc[2][NI];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[mi][ni][a] = 0.f;

  const int nch = H / 64;
  auto issue = [&](int c, int slot) {
    const bool real = c < nch;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      lds_load16(wrs, &ws_[slot][(64 * wave + 8 * i) * 64], real ? woff[i] + 128u * uint32_t(c) : 0x80000000u);
#pragma unroll
    for (int i = 0; i < NI; ++i) lds_load16(xsrc[i] + (real ? 64 * c : 0), &xs[slot][(32 * i + 8 * wave) * 64]);
  };

  // LDS read offsets (elements) of this lane's fragments for k-step st.
  int wrd[2][4], xrd[NI][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int wr = 64 * wave + 32 * mi + ql;
      wrd[mi][st] = wr * 64 + 8 * ((4 * g + st) ^ ((wr >> 1) & 7));
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = 32 * ni + ql;
      xrd[ni][st] = n * 64 + 8 * ((4 * g + st) ^ ((n >> 1) & 7));
    }
  }

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p, p);
  int slot = 0;
  for (int c = 0; c < nch; ++c) {
    // chunk c landed: this wave's loads (NS - 2 chunks were issued after
    // it), then everyone's; the slot chunk c - 1 used is free again.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * PER_CHUNK));
    barrier_no_fence();
    const __bf16 *wb = ws_[slot];
    const __bf16 *xb = xs[slot];
    bf16x8 af[4][2], bfr[4][NI];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) af[st][mi] = *reinterpret_cast<const bf16x8 *>(wb + wrd[mi][st]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[st][ni] = *reinterpret_cast<const bf16x8 *>(xb + xrd[ni][st]);
    }
    issue(c + NS - 1, slot == 0 ? NS - 1 : slot - 1);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[st][mi], bfr[st][ni], acc[mi][ni], 0, 0, 0);
    // Issue order: the fragments of k-steps 0 and 1, then the MFMAs with the
    // other fragment reads after the first step's, and the LDS-direct loads
    // of a later chunk one after each MFMA: a wave issues in order, so a run
    // of loads would hold the matrix cores back.
    constexpr int RD = 2 + NI, MF = 2 * NI, LD = PER_CHUNK;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RD, 0);
#pragma unroll
    for (int i = 0; i < 4 * MF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < LD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (i == MF - 1 || i == 2 * MF - 1) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
    }
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the trailing loads land before the workgroup ends
  wide_epilogue<NI>(acc, red, v0, vt, n0, V, N, labels, pmax, psum, plab);
}

// ---------------- bf16, wide tiles, persistent workgroups with loader waves
// The 256-row x 32*NI-item tiles and LDS layout of score_wide_kernel, with
// two changes. (1) Each workgroup loops over its share of the tiles (one
// workgroup per CU), so the first chunks of its next tile are staged while
// it finishes the current one: the per-tile start (readout positions, the
// ring's first loads) leaves the critical path. (2) Waves 4-7 only stage
// chunks into the LDS ring and waves 0-3 only read fragments and issue
// MFMAs (one of each per SIMD), so no load instruction waits in front of an
// MFMA. The loaders' vector-memory operations are all loads, so their counts
// complete in order; the compute waves' epilogue stores never mix with them.
template <int NI, int NS>
__global__ __launch_bounds__(512, 1) void score_persist_kernel(
    const __bf16 *__restrict__ hidden, const __bf16 *__restrict__ w, int H, int V, int N,
    const int32_t *__restrict__ readout_pos, LabelArgs labels, float *__restrict__ pmax,
    float *__restrict__ psum, float *__restrict__ plab, int nvt, int nit) {
  constexpr int BVW = 256;                  // vocabulary rows of a tile
  constexpr int NIT = 32 * NI;              // items of a tile
  constexpr int WCH = BVW * 64;             // bf16 elements of a staged W chunk
  constexpr int XCH = NIT * 64;             // ... and of a staged readout chunk
  constexpr int PER_CHUNK = BVW / 32 + NI;  // loads per loader wave and chunk
  struct Smem {
    __bf16 w[NS][WCH];
    __bf16 x[NS][XCH];
    float red[4][NI][32];
  };
  static_assert(sizeof(Smem) <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto &ws_ = sm.w;
  auto &xs = sm.x;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cw = wave & 3;  // compute waves 0-3, loader waves 4-7 (one of each per SIMD)
  const int lane = tid & 63;
  const int g = lane >> 5, ql = lane & 31;
  const int piece = lane & 7;
  const int nch = H / 64;
  // Tile k of this workgroup: jx = blockIdx / 8 + k * gridDim / 8 (gridDim is
  // a multiple of 8, so all its tiles are on its XCD), vocabulary tile
  // 8 (jx / nit) + XCD, item tile jx % nit: the item tiles of one vocabulary
  // tile run on one XCD at about the same time and share its L2.
  const int xcd = blockIdx.x & 7, j0 = blockIdx.x >> 3, J = gridDim.x >> 3;
  const int vts = (nvt - xcd + 7) / 8;  // vocabulary tiles of this XCD
  const int ntile = max(0, (vts * nit - j0 + J - 1) / J);
  if (ntile == 0) return;
  auto tile_vt = [&](int k) { return 8 * ((j0 + k * J) / nit) + xcd; };
  auto tile_n0 = [&](int k) { return ((j0 + k * J) % nit) * NIT; };

  if (wave >= 4) {
    // ---- loader: chunk q of the workgroup's sequence (tile q / nch, chunk
    // q % nch) goes to ring slot q % NS, NS - 1 chunks ahead of its use.
    uint32_t woff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 64 * cw + 8 * i + (lane >> 3);
      woff[i] = uint32_t(r) * uint32_t(H) * 2u + 16u * uint32_t(piece ^ ((r >> 1) & 7));
    }
    // first W row of a tile (V past the last tile: its loads read nothing)
    auto w_row0 = [&](int k) { return __builtin_amdgcn_readfirstlane(k < ntile ? tile_vt(k) * BVW : V); };
    // rows past V, and tiles past the last, read nothing (zero-length range);
    // built from wave-uniform values where it is used, so it stays in scalar registers
    auto w_rsrc = [&](int v0) {
      const uint32_t rows = __builtin_amdgcn_readfirstlane(uint32_t(max(0, min(BVW, V - v0))));
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16 *>(w + int64_t(min(v0, V - 1)) * H), 0,
                                               rows * uint32_t(H) * 2u, kRsrcWord3);
    };
    // readout positions of a tile's items (tiles past the last: item 0)
    auto positions = [&](int k, int (&pos)[NI]) {
      const int n0 = k < ntile ? tile_n0(k) : 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) pos[i] = readout_pos[min(n0 + 32 * i + 8 * cw + (lane >> 3), N - 1)];
    };
    auto rows = [&](const int (&pos)[NI], const __bf16 *(&src)[NI]) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = 32 * i + 8 * cw + (lane >> 3);
        src[i] = hidden + int64_t(pos[i]) * H + 8 * (piece ^ ((n >> 1) & 7));
      }
    };
    int wv0 = w_row0(0), wv0_next = w_row0(1);
    const __bf16 *xsrc[NI];
    int pos_next[NI];
    {
      int pos0[NI];
      positions(0, pos0);
      rows(pos0, xsrc);
      positions(1, pos_next);
    }
    auto issue = [&](int c, int slot) {
      const __amdgpu_buffer_rsrc_t wrs = w_rsrc(wv0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        lds_load16(wrs, &ws_[slot][(64 * cw + 8 * i) * 64], woff[i] + 128u * uint32_t(c));
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_load16(xsrc[i] + 64 * c, &xs[slot][(32 * i + 8 * cw) * 64]);
    };
    // the sequence's first NS - 1 chunks (all in tile 0: nch >= NS - 1)
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) issue(p, p);
    int ik = 0, ic = NS - 1, islot = NS - 1;  // next chunk to issue: tile ik, chunk ic, ring slot islot
    for (int k = 0; k < ntile; ++k) {
      for (int c = 0; c < nch; ++c) {
        // chunk (k, c) landed: this wave's loads of it (NS - 2 chunks' loads,
        // and at most one tile's readout positions, were issued after them)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * PER_CHUNK));
        barrier_no_fence();
        if (ic == nch) {  // the issue point enters the next tile
          ic = 0;
          ++ik;
          wv0 = wv0_next;
          wv0_next = w_row0(ik + 1);
          rows(pos_next, xsrc);
          positions(ik + 1, pos_next);
        }
        issue(ic, islot);  // into the slot chunk (k, c) - 1 used
        ++ic;
        islot = islot + 1 == NS ? 0 : islot + 1;
      }
      // the compute waves' epilogue barriers
      barrier_no_fence();
      barrier_no_fence();
      barrier_no_fence();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the trailing loads land before the workgroup ends
    return;
  }

  // ---- compute waves: fragments of chunk q from ring slot q % NS
  int wrd[2][4], xrd[NI][4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int wr = 64 * cw + 32 * mi + ql;
      wrd[mi][st] = wr * 64 + 8 * ((4 * g + st) ^ ((wr >> 1) & 7));
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = 32 * ni + ql;
      xrd[ni][st] = n * 64 + 8 * ((4 * g + st) ^ ((n >> 1) & 7));
    }
  }
  int slot = 0;
  for (int k = 0; k < ntile; ++k) {
    f32x16 acc[2][NI];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int a = 0; a < 16; ++a) acc[mi][ni][a] = 0.f;
    for (int c = 0; c < nch; ++c) {
      barrier_no_fence();
      const __bf16 *wb = ws_[slot];
      const __bf16 *xb = xs[slot];
      bf16x8 af[4][2], bfr[4][NI];
      auto rd = [&](int st) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) af[st][mi] = *reinterpret_cast<const bf16x8 *>(wb + wrd[mi][st]);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bfr[st][ni] = *reinterpret_cast<const bf16x8 *>(xb + xrd[ni][st]);
      };
      auto mm = [&](int st) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[st][mi], bfr[st][ni], acc[mi][ni], 0, 0, 0);
      };
      // k-steps in order, each a fenced group: the fragments of k-steps 0 and
      // 1 first, then k-step st's MFMAs with the reads of k-step st + 2
      constexpr int RD = 2 + NI, MF = 2 * NI;
      rd(0);
      rd(1);
      __builtin_amdgcn_sched_barrier(0);
      rd(2);
      mm(0);
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      rd(3);
      mm(1);
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mm(2);
      mm(3);
      __builtin_amdgcn_sched_barrier(0);
      slot = slot + 1 == NS ? 0 : slot + 1;
    }
    const int vt = tile_vt(k);
    wide_epilogue<NI>(acc, sm.red, vt * BVW, vt, tile_n0(k), V, N, labels, pmax, psum, plab);
  }
}

// ---------------------------------------------------------------- fp32
// One workgroup per (128 vocabulary rows, item); one thread per row.
__global__ __launch_bounds__(BV) void score_f32_kernel(
    const float *__restrict__ hidden, const float *__restrict__ w, int H, int V, int N,
    const int32_t *__restrict__ readout_pos, LabelArgs labels, float *__restrict__ pmax,
    float *__restrict__ psum, float *__restrict__ plab, int nvt) {
  __shared__ float red[BV / 64];
  const int vt = blockIdx.x, n = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vr = vt * BV + tid;
  const bool ok = vr < V;
  const float *x = hidden + int64_t(readout_pos[n]) * H;
  const float *wr = w + int64_t(ok ? vr : 0) * H;
  float z = 0.f;
  for (int h = 0; h < H; ++h) z = fmaf(wr[h], x[h], z);

  float mx = ok ? z : -INFINITY;
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < BV / 64; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  float s = ok ? expf(z - m) : 0.f;
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int i = 0; i < BV / 64; ++i) t += red[i];
    pmax[int64_t(vt) * N + n] = m;
    psum[int64_t(vt) * N + n] = t;
  }
  if (ok)
    for (int kx = 0; kx < labels.k; ++kx)
      if (labels.ids[kx] == vr) plab[int64_t(n) * labels.k + kx] = z;
}

// ---------------------------------------------------------------- combine
// One 256-thread workgroup per item.
__device__ __forceinline__ float block_max(float x, float *sh) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  __syncthreads();
  return x;
}

__device__ __forceinline__ float block_sum(float x, float *sh) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  x = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return x;
}

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ pmax,
                                                      const float *__restrict__ psum,
                                                      const float *__restrict__ plab, int nvt, int N, int K,
                                                      int apply_softmax, float *__restrict__ out) {
  __shared__ float sh[4];
  const int n = blockIdx.x, tid = threadIdx.x;
  // partials are vocabulary-tile major: tile c of item n at c * N + n
  const float *pm = pmax + n;
  const float *ps = psum + n;
  const float *zl = plab + int64_t(n) * K;
  float *o = out + int64_t(n) * K;
  if (apply_softmax) {
    float mx = -INFINITY;
    for (int kx = tid; kx < K; kx += 256) mx = fmaxf(mx, zl[kx]);
    mx = block_max(mx, sh);
    float s = 0.f;
    for (int kx = tid; kx < K; kx += 256) s += expf(zl[kx] - mx);
    s = block_sum(s, sh);
    for (int kx = tid; kx < K; kx += 256) o[kx] = expf(zl[kx] - mx) / s;
    return;
  }
  float M = -INFINITY;
  for (int c = tid; c < nvt; c += 256) M = fmaxf(M, pm[int64_t(c) * N]);
  M = block_max(M, sh);
  float s = 0.f;
  for (int c = tid; c < nvt; c += 256) s += ps[int64_t(c) * N] * expf(pm[int64_t(c) * N] - M);
  s = block_sum(s, sh);
  const float lse = M + logf(s);
  for (int kx = tid; kx < K; kx += 256) o[kx] = zl[kx] - lse;
}

}  // namespace

// The workspace of mis_score_labels_noalloc: partial maxima, partial sums
// and label logits, as in a caller's workspace. Every GPU the library runs
// on holds its own copy until the process ends. Host code never passes the
// name itself to a kernel (on the host it is only a stand-in for the
// symbol): score_scratch looks up the device address once per device.
static __device__ __align__(256) unsigned char scratch[MIS_SCORE_SCRATCH_BYTES];

hipError_t score_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

ScoreKernel pick_score(int N, int H, mis_dtype dt, ScoreForce force, int force_ni) {
  if (dt != MIS_BF16) return {ScoreKind::F32, 1};
  if (H % 64 != 0) return {ScoreKind::Global, N <= 64 ? 1 : N <= 128 ? 2 : 4};
  // Up to 64 items stream W through the narrow tiles (every LM-head row read
  // once). More items are MFMA-bound: the persistent workgroups with loader
  // waves (item blocks 3-5, the fewest padded items, then the widest tile),
  // or the wide tiles when forced or H < 128.
  if ((force == ScoreForce::Persist || (force == ScoreForce::Auto && N > 64)) && H >= 128) {
    int ni = force_ni;
    if (ni != 3 && ni != 4 && ni != 5) {
      ni = 3;
      for (int c : {4, 5}) {
        const int pc = (N + 32 * c - 1) / (32 * c) * 32 * c, pb = (N + 32 * ni - 1) / (32 * ni) * 32 * ni;
        if (pc <= pb) ni = c;
      }
    }
    return {ScoreKind::Persist, ni};
  }
  const bool wide = force == ScoreForce::Wide || force == ScoreForce::Persist || (force == ScoreForce::Auto && N > 64);
  if (!wide) return {ScoreKind::Narrow, N <= 32 ? 1 : N <= 64 ? 2 : 4};
  int ni = force_ni;
  if (ni != 3 && ni != 4 && ni != 5 && ni != 6 && ni != 8) {
    // item blocks per tile: the fewest padded items, then the widest tile
    ni = 3;
    for (int c : {4, 5, 6, 8}) {
      const int pc = (N + 32 * c - 1) / (32 * c) * 32 * c, pb = (N + 32 * ni - 1) / (32 * ni) * 32 * ni;
      if (pc <= pb) ni = c;
    }
  }
  return {ScoreKind::Wide, ni};
}

// LDS ring depth of each tile shape: 3 stages while W streams once (one
// workgroup per CU for the wide tiles up to 5 item blocks), 2 when two
// workgroups share a CU or the readout tile is large.
static int score_stages(const ScoreKernel &k) {
  if (k.kind == ScoreKind::Narrow) return k.ni == 4 ? 2 : 3;
  if (k.kind == ScoreKind::Wide) return k.ni <= 5 ? 3 : 2;
  return 0;
}

void score_kernel_name(const ScoreKernel &k, char *buf, size_t n) {
  switch (k.kind) {
    case ScoreKind::Narrow: snprintf(buf, n, "score_lds_kernel<%d, %d>", k.ni, score_stages(k)); return;
    case ScoreKind::Wide: snprintf(buf, n, "score_wide_kernel<%d, %d>", k.ni, score_stages(k)); return;
    case ScoreKind::Persist: snprintf(buf, n, "score_persist_kernel<%d, 3>", k.ni); return;
    case ScoreKind::Global: snprintf(buf, n, "score_bf16_kernel<%d>", k.ni); return;
    case ScoreKind::F32: snprintf(buf, n, "score_f32_kernel"); return;
  }
  if (n) buf[0] = 0;
}

hipError_t launch_score(const int32_t *readout_pos, int N, const void *hidden, int H, const void *lm_head,
                        int V, mis_dtype dt, const LabelArgs &labels, int apply_softmax,
                        float *scores, float *ws, const ScoreKernel &kern, hipStream_t st) {
  const int nvt = score_vocab_tiles(V);
  int nvt_used = nvt;  // vocabulary tiles of the kernel that runs (the workspace fits the most)
  const size_t part = ((sizeof(float) * size_t(N) * nvt + 255) / 256) * 256;
  float *pmax = ws;
  float *psum = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + part);
  float *plab = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + 2 * part);
  const __bf16 *hp = static_cast<const __bf16 *>(hidden);
  const __bf16 *wp = static_cast<const __bf16 *>(lm_head);
  const int ni = kern.ni;
  switch (kern.kind) {
    case ScoreKind::Wide: {
      const int nvw = (V + 255) / 256;
      const int nit = (N + 32 * ni - 1) / (32 * ni);
      const unsigned grid = unsigned((nvw + 7) / 8 * 8 * nit);
#define MIS_WIDE(NI, NS)                                                                                  \
  score_wide_kernel<NI, NS><<<grid, 256, 0, st>>>(hp, wp, H, V, N, readout_pos, labels, pmax, psum, plab, \
                                                  nvw, nit)
      switch (ni) {
        case 3: MIS_WIDE(3, 3); break;
        case 4: MIS_WIDE(4, 3); break;
        case 5: MIS_WIDE(5, 3); break;
        case 6: MIS_WIDE(6, 2); break;
        case 8: MIS_WIDE(8, 2); break;
        default: return hipErrorInvalidValue;
      }
#undef MIS_WIDE
      nvt_used = nvw;
      break;
    }
    case ScoreKind::Persist: {
      if (H < 128) return hipErrorInvalidValue;  // the ring's first two chunks are in the first tile
      const int nvw = (V + 255) / 256;
      const int nit = (N + 32 * ni - 1) / (32 * ni);
      const int tiles8 = (nvw + 7) / 8 * 8 * nit;  // tile slots over the 8 XCDs
      const unsigned grid = unsigned(std::max(8, std::min(device_cus() / 8 * 8, tiles8)));
#define MIS_PERSIST(NI) \
  score_persist_kernel<NI, 3><<<grid, 512, 0, st>>>(hp, wp, H, V, N, readout_pos, labels, pmax, psum, plab, nvw, nit)
      switch (ni) {
        case 3: MIS_PERSIST(3); break;
        case 4: MIS_PERSIST(4); break;
        case 5: MIS_PERSIST(5); break;
        default: return hipErrorInvalidValue;
      }
#undef MIS_PERSIST
      nvt_used = nvw;
      break;
    }
    case ScoreKind::Narrow: {
      const int nit = (N + 32 * ni - 1) / (32 * ni);
      const unsigned grid = unsigned((nvt + 7) / 8 * 8 * nit);
      if (ni == 1)
        score_lds_kernel<1, 3><<<grid, 256, 0, st>>>(hp, wp, H, V, N, readout_pos, labels, pmax, psum,
                                                     plab, nvt, nit);
      else if (ni == 2)
        score_lds_kernel<2, 3><<<grid, 256, 0, st>>>(hp, wp, H, V, N, readout_pos, labels, pmax, psum,
                                                     plab, nvt, nit);
      else
        score_lds_kernel<4, 2><<<grid, 256, 0, st>>>(hp, wp, H, V, N, readout_pos, labels, pmax, psum,
                                                     plab, nvt, nit);
      break;
    }
    case ScoreKind::Global:
      if (ni == 1)
        score_bf16_kernel<1><<<dim3(nvt, (N + 63) / 64), 256, 0, st>>>(hp, wp, H, V, N, readout_pos, labels,
                                                                      pmax, psum, plab, nvt);
      else if (ni == 2)
        score_bf16_kernel<2><<<dim3(nvt, (N + 127) / 128), 256, 0, st>>>(hp, wp, H, V, N, readout_pos, labels,
                                                                        pmax, psum, plab, nvt);
      else
        score_bf16_kernel<4><<<dim3(nvt, (N + 255) / 256), 256, 0, st>>>(hp, wp, H, V, N, readout_pos, labels,
                                                                        pmax, psum, plab, nvt);
      break;
    case ScoreKind::F32:
      score_f32_kernel<<<dim3(nvt, N), BV, 0, st>>>(static_cast<const float *>(hidden),
                                                    static_cast<const float *>(lm_head), H, V, N, readout_pos,
                                                    labels, pmax, psum, plab, nvt);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_kernel<<<N, 256, 0, st>>>(pmax, psum, plab, nvt_used, N, labels.k, apply_softmax, scores);
  return hipGetLastError();
}

}  // namespace mis
