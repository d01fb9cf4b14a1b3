// Rotary position embedding of Q and K, in place, at the segment position ids.
//
// From Generation to Scoring, §4.1 (position-id rule): prefix token u sits at
// position u and the token at offset d inside any item at Lq + d, so every
// item is rotated as if it followed the prefix alone. The rotation is the
// usual rotary embedding: dims i and i + D/2 form a pair turned by
// pos * theta^(-2i/D).
//
// One thread owns 8 consecutive pairs of one token in up to 4 of its head rows
// (query heads first, then KV heads; KV heads only when Q is rotated inside
// the attention call): it computes the 8 angles (product and reduction modulo
// 2*pi in fp64, then sin/cos in fp32), issues all its loads, then rotates and
// stores. A head row is a 2*D-byte contiguous run read by D/16 threads.
// HBM-bound: every rotated byte is read and written once.
//
// The cos/sin table (rope_table_kernel) holds the same angles for positions
// 0 .. P-1, for the attention kernels that rotate Q while loading it.
#include "mis_internal.h"
#include "rope_math.h"

namespace mis {
namespace {

constexpr int kPairsPerThread = 8;

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
  }
  static __device__ __forceinline__ void store(float *p, const float (&x)[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
};
template <>
struct Vec8<__bf16> {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ void load(const __bf16 *p, float (&x)[8]) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = float(v[e]);
  }
  static __device__ __forceinline__ void store(__bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __bf16(x[e]);  // round to nearest even
    *reinterpret_cast<bf16x8 *>(p) = v;
  }
};

constexpr int kHeadsPerThread = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(const int32_t *__restrict__ pos_id, T *__restrict__ q,
                                                   T *__restrict__ k, int ntok, int hq, int hkv,
                                                   RopeFreq freq) {
  constexpr int HALF = D / 2;
  constexpr int NCH = HALF / kPairsPerThread;  // threads per head row
  const int heads = hq + hkv;
  const int nhb = (heads + kHeadsPerThread - 1) / kHeadsPerThread;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int ch = int(idx % NCH);
  const int64_t rest = idx / NCH;
  const int hb = int(rest % nhb);
  const int64_t t = rest / nhb;
  if (t >= ntok) return;
  const int i0 = ch * kPairsPerThread;
  const double pos = double(pos_id[t]);
  float cs[kPairsPerThread], sn[kPairsPerThread];
#pragma unroll
  for (int e = 0; e < kPairsPerThread; ++e) rope_cos_sin(pos, freq.inv[i0 + e], cs[e], sn[e]);
  T *rows[kHeadsPerThread];
  float a[kHeadsPerThread][8], b[kHeadsPerThread][8];
#pragma unroll
  for (int u = 0; u < kHeadsPerThread; ++u) {
    const int h = min(hb * kHeadsPerThread + u, heads - 1);  // a short last block repeats its last row
    rows[u] = h < hq ? q + (t * hq + h) * D : k + (t * hkv + (h - hq)) * D;
    Vec8<T>::load(rows[u] + i0, a[u]);
    Vec8<T>::load(rows[u] + HALF + i0, b[u]);
  }
#pragma unroll
  for (int u = 0; u < kHeadsPerThread; ++u) {
    if (hb * kHeadsPerThread + u >= heads) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(a[u][e], b[u][e], cs[e], sn[e]);
    Vec8<T>::store(rows[u] + i0, a[u]);
    Vec8<T>::store(rows[u] + HALF + i0, b[u]);
  }
}

// table[p][i] = (cos, sin) of the angle of pair i at position p, p < npos.
template <int D>
__global__ __launch_bounds__(256) void rope_table_kernel(float2 *__restrict__ table, int npos, RopeFreq freq) {
  constexpr int HALF = D / 2;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(npos) * HALF) return;
  float c, s;
  rope_cos_sin(double(idx / HALF), freq.inv[idx % HALF], c, s);
  table[idx] = make_float2(c, s);
}

template <typename T, int D>
hipError_t launch(const mis_segments &seg, T *q, T *k, int hq, int hkv, const RopeFreq &f, hipStream_t st) {
  constexpr int NCH = D / 2 / kPairsPerThread;
  const int64_t threads = int64_t(seg.total_tokens) * ((hq + hkv + kHeadsPerThread - 1) / kHeadsPerThread) * NCH;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  rope_kernel<T, D><<<unsigned(blocks), 256, 0, st>>>(seg.pos_id, q, k, seg.total_tokens, hq, hkv, f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_table(float *table, int npos, int d, const RopeFreq &f, hipStream_t st) {
  const int64_t blocks = (int64_t(npos) * (d / 2) + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  float2 *t = reinterpret_cast<float2 *>(table);
  if (d == 128) rope_table_kernel<128><<<unsigned(blocks), 256, 0, st>>>(t, npos, f);
  else rope_table_kernel<64><<<unsigned(blocks), 256, 0, st>>>(t, npos, f);
  return hipGetLastError();
}

hipError_t launch_rope(const mis_segments &seg, void *q, void *k, mis_dtype dt, int hq, int hkv, int d,
                       const RopeFreq &f, hipStream_t st) {
  if (dt == MIS_BF16) {
    if (d == 128) return launch<__bf16, 128>(seg, static_cast<__bf16 *>(q), static_cast<__bf16 *>(k), hq, hkv, f, st);
    return launch<__bf16, 64>(seg, static_cast<__bf16 *>(q), static_cast<__bf16 *>(k), hq, hkv, f, st);
  }
  if (d == 128) return launch<float, 128>(seg, static_cast<float *>(q), static_cast<float *>(k), hq, hkv, f, st);
  return launch<float, 64>(seg, static_cast<float *>(q), static_cast<float *>(k), hq, hkv, f, st);
}

}  // namespace mis
