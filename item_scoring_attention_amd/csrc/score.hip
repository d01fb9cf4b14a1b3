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
#include "mis_internal.h"

namespace mis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int BV = kScoreBlockV;

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ---------------------------------------------------------------- bf16 MFMA
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

#pragma unroll 2
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
        pmax[int64_t(n) * nvt + vt] = m[ni];
        psum[int64_t(n) * nvt + vt] = red[0][wn][ni][ql] + red[1][wn][ni][ql];
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

// ------------------------------------------------- bf16 streaming (N <= 64)
// HBM-bound regime: every LM-head row is read once and feeds at most two
// MFMAs per 16 hidden dims, so the kernel is a stream. 4 waves x 32 rows =
// 128 vocabulary rows per workgroup. Each lane streams 64 contiguous bytes of
// its row per 64-dim chunk, prefetched two chunks ahead; the gathered readout
// rows of the chunk sit in LDS (double-buffered, shared by the 4 waves).
// K-slot order inside a chunk: k-step s of half-wave g covers dims
// 32*g + 8*s .. +8 for both operands (any order works if A and B agree).
template <int NI>
__global__ __launch_bounds__(256) void score_stream_kernel(
    const __bf16 *__restrict__ hidden, const __bf16 *__restrict__ w, int H, int V, int N,
    const int32_t *__restrict__ readout_pos, LabelArgs labels, float *__restrict__ pmax,
    float *__restrict__ psum, float *__restrict__ plab, int nvt) {
  constexpr int XP = 64 + 8;  // LDS row pitch (bf16) of a staged chunk: 144 B
  constexpr int NIT = 32 * NI;  // items in the tile
  __shared__ __attribute__((aligned(16))) __bf16 xs[2][NIT * XP];
  __shared__ float red[4][NI][32];

  const int vt = blockIdx.x;
  const int v0 = vt * BV;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, ql = lane & 31;
  const int row = v0 + 32 * wave + ql;
  const __bf16 *wrow = w + int64_t(min(row, V - 1)) * H + 32 * g;

  // staging of the gathered rows: thread -> (item xi + 32*i, 16-byte chunk xc of the 64 dims)
  const int xi = tid >> 3, xc = tid & 7;
  static_assert(NI == 1 || NI == 2, "one or two item blocks");
  const __bf16 *xrow0 = hidden + int64_t(readout_pos[min(xi, N - 1)]) * H + 8 * xc;
  const __bf16 *xrow1 = hidden + int64_t(readout_pos[min(xi + 32, N - 1)]) * H + 8 * xc;

  f32x16 acc[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int a = 0; a < 16; ++a) acc[ni][a] = 0.f;

  const int nch = H / 64;
  bf16x8 wb0[4], wb1[4], wb2[4];  // prefetch ring of three chunks
  auto load_w = [&](int c, bf16x8 (&dst)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[s] = *reinterpret_cast<const bf16x8 *>(wrow + 64 * c + 8 * s);
  };
  uint4 xreg0 = make_uint4(0, 0, 0, 0), xreg1 = make_uint4(0, 0, 0, 0);
  auto load_x = [&](int c) {
    xreg0 = *reinterpret_cast<const uint4 *>(xrow0 + 64 * c);
    if (NI > 1) xreg1 = *reinterpret_cast<const uint4 *>(xrow1 + 64 * c);
  };
  auto store_x = [&](int buf) {
    *reinterpret_cast<uint4 *>(&xs[buf][xi * XP + 8 * xc]) = xreg0;
    if (NI > 1) *reinterpret_cast<uint4 *>(&xs[buf][(xi + 32) * XP + 8 * xc]) = xreg1;
  };
  // chunk c: prefetch chunk c + 2 into `pre`, contract chunk c from `cur`
  auto step = [&](int c, bf16x8 (&cur)[4], bf16x8 (&pre)[4]) {
    if (c + 2 < nch) load_w(c + 2, pre);
    if (c + 1 < nch) load_x(c + 1);
    const __bf16 *xb = xs[c & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const bf16x8 bfr = *reinterpret_cast<const bf16x8 *>(xb + (32 * ni + ql) * XP + 32 * g + 8 * s);
        acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[s], bfr, acc[ni], 0, 0, 0);
      }
    if (c + 1 < nch) store_x((c + 1) & 1);
    __syncthreads();
  };

  load_w(0, wb0);
  if (nch > 1) load_w(1, wb1);
  load_x(0);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 3) {
    step(c, wb0, wb2);
    if (c + 1 < nch) step(c + 1, wb1, wb0);
    if (c + 2 < nch) step(c + 2, wb2, wb1);
  }

  // epilogue: element a of acc[ni] is z[row v0 + 32*wave + 8*(a/4) + 4*g + a%4][item 32*ni + ql]
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
      const int n = 32 * ni + ql;
      if (n < N) {
        pmax[int64_t(n) * nvt + vt] = m[ni];
        psum[int64_t(n) * nvt + vt] = red[0][ni][ql] + red[1][ni][ql] + red[2][ni][ql] + red[3][ni][ql];
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
      const int n = 32 * ni + ql;
      if (n < N) plab[int64_t(n) * labels.k + kx] = z;
    }
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
    pmax[int64_t(n) * nvt + vt] = m;
    psum[int64_t(n) * nvt + vt] = t;
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
                                                      const float *__restrict__ plab, int nvt, int K,
                                                      int apply_softmax, float *__restrict__ out) {
  __shared__ float sh[4];
  const int n = blockIdx.x, tid = threadIdx.x;
  const float *pm = pmax + int64_t(n) * nvt;
  const float *ps = psum + int64_t(n) * nvt;
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
  for (int c = tid; c < nvt; c += 256) M = fmaxf(M, pm[c]);
  M = block_max(M, sh);
  float s = 0.f;
  for (int c = tid; c < nvt; c += 256) s += ps[c] * expf(pm[c] - M);
  s = block_sum(s, sh);
  const float lse = M + logf(s);
  for (int kx = tid; kx < K; kx += 256) o[kx] = zl[kx] - lse;
}

}  // namespace

hipError_t launch_score(const mis_segments &seg, const void *hidden, int H, const void *lm_head,
                        int V, mis_dtype dt, const LabelArgs &labels, int apply_softmax,
                        float *scores, float *ws, hipStream_t st) {
  const int N = seg.total_items;
  const int nvt = score_vocab_tiles(V);
  const size_t part = ((sizeof(float) * size_t(N) * nvt + 255) / 256) * 256;
  float *pmax = ws;
  float *psum = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + part);
  float *plab = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + 2 * part);
  if (dt == MIS_BF16) {
    const __bf16 *hp = static_cast<const __bf16 *>(hidden);
    const __bf16 *wp = static_cast<const __bf16 *>(lm_head);
    if (N <= 32 && H % 64 == 0) {
      score_stream_kernel<1><<<nvt, 256, 0, st>>>(hp, wp, H, V, N, seg.readout_pos, labels, pmax,
                                                 psum, plab, nvt);
    } else if (N <= 64 && H % 64 == 0) {
      score_stream_kernel<2><<<nvt, 256, 0, st>>>(hp, wp, H, V, N, seg.readout_pos, labels, pmax,
                                                 psum, plab, nvt);
    } else if (N <= 64) {
      score_bf16_kernel<1><<<dim3(nvt, (N + 63) / 64), 256, 0, st>>>(
          hp, wp, H, V, N, seg.readout_pos, labels, pmax, psum, plab, nvt);
    } else if (N <= 128) {
      score_bf16_kernel<2><<<dim3(nvt, (N + 127) / 128), 256, 0, st>>>(
          hp, wp, H, V, N, seg.readout_pos, labels, pmax, psum, plab, nvt);
    } else {
      score_bf16_kernel<4><<<dim3(nvt, (N + 255) / 256), 256, 0, st>>>(
          hp, wp, H, V, N, seg.readout_pos, labels, pmax, psum, plab, nvt);
    }
  } else {
    score_f32_kernel<<<dim3(nvt, N), BV, 0, st>>>(static_cast<const float *>(hidden),
                                                  static_cast<const float *>(lm_head), H, V, N,
                                                  seg.readout_pos, labels, pmax, psum, plab, nvt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_kernel<<<N, 256, 0, st>>>(pmax, psum, plab, nvt, labels.k, apply_softmax, scores);
  return hipGetLastError();
}

}  // namespace mis
