// fp32 MIS prefill attention (From Generation to Scoring, §4.1, Eq. 4).
//
// Correctness-grade path for fp32 workloads: one thread per (query token,
// query head) walks only the keys its row may see, i.e. the prefix keys up to
// the row and, for item rows, the keys of its own item up to the row. Keys of
// other items are never read. Online softmax in fp32.
#include "mis_internal.h"

namespace mis {
namespace {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    int B, int T, int hq, int hkv, float scale, const int32_t *__restrict__ cu_seqlens,
    const int32_t *__restrict__ prefix_lens, const int32_t *__restrict__ item_id,
    const int32_t *__restrict__ item_begin, const float *__restrict__ q,
    const float *__restrict__ k, const float *__restrict__ v, float *__restrict__ o, int items_only) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  if (t >= T) return;
  // request of token t
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_seqlens[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int32_t base = cu_seqlens[lo];
  const int32_t lq = prefix_lens[lo];
  const int32_t u = t - base;
  if (items_only && u < lq) return;  // appending items to a cached prefix: prefix rows are not recomputed
  const int g = (h * hkv) / hq;
  const int64_t kv_stride = int64_t(hkv) * D;

  float qr[D];
  const float *qp = q + (int64_t(t) * hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = qp[d] * scale;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  auto visit = [&](int32_t k_lo, int32_t k_hi) {  // request-local [k_lo, k_hi)
    for (int32_t kk = k_lo; kk < k_hi; ++kk) {
      const float *kp = k + (int64_t(base + kk)) * kv_stride + int64_t(g) * D;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], kp[d], s);
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new);  // 0 on the first key (m = -inf)
      const float p = expf(s - m_new);
      l = l * alpha + p;
      const float *vp = v + (int64_t(base + kk)) * kv_stride + int64_t(g) * D;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vp[d], acc[d] * alpha);
      m = m_new;
    }
  };
  if (u < lq) {
    visit(0, u + 1);
  } else {
    visit(0, lq);
    visit(item_begin[item_id[t]] - base, u + 1);
  }
  const float inv = 1.f / l;
  float *op = o + (int64_t(t) * hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
}

}  // namespace

hipError_t launch_attention_f32(const mis_segments &seg, const float *q, const float *k,
                                const float *v, float *o, int hq, int hkv, int d, float scale,
                                int items_only, hipStream_t st) {
  const dim3 grid((seg.total_tokens + 63) / 64, hq);
  if (d == 64) {
    attn_f32_kernel<64><<<grid, 64, 0, st>>>(seg.num_requests, seg.total_tokens, hq, hkv, scale,
                                             seg.cu_seqlens, seg.prefix_lens, seg.item_id,
                                             seg.item_begin, q, k, v, o, items_only);
  } else if (d == 128) {
    attn_f32_kernel<128><<<grid, 64, 0, st>>>(seg.num_requests, seg.total_tokens, hq, hkv, scale,
                                              seg.cu_seqlens, seg.prefix_lens, seg.item_id,
                                              seg.item_begin, q, k, v, o, items_only);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mis
