// Measurement probe (not part of the MIS ABI): the bf16 MFMA rate this GPU
// sustains, for pricing the attention kernel against a measured peak beside
// the published one. Built into libmis_probe.so; only the benchmark loads it.
//
// Every wave issues v_mfma_f32_32x32x16_bf16 back to back on eight
// independent accumulators (more than the pipe's dependent-issue distance),
// one wave per SIMD, no memory traffic in the loop. The operands are
// non-zero (zero operands run at a higher clock than real data); the random
// mode also changes them from one MFMA to the next, as real data does, which
// draws more power and lowers the clock the part holds.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;

// Uniform bits -> roughly N(0, 1) (sum of four uniforms, centred and scaled).
__device__ __forceinline__ float gauss(uint32_t h) {
  const float u = float(h & 255) + float((h >> 8) & 255) + float((h >> 16) & 255) + float(h >> 24);
  return (u - 510.f) * (1.f / 147.8f);
}

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  return x ^ (x >> 16);
}

// mode 0: small operands that repeat on every MFMA (few bits toggle);
// mode 1: N(0, 1)-like bf16 operands, different for each of the eight chains,
// so consecutive MFMAs switch operands as they do on real data.
__global__ __launch_bounds__(256, 1) void mfma_peak_kernel(float *__restrict__ sink, int iters, int mode) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (mode == 0) {
        a[c][e] = __bf16(float(((lane * 7 + e * 3) & 15) - 7) * 0.001f);
        b[c][e] = __bf16(float(((lane * 5 + e * 11) & 15) - 8) * 0.001f);
      } else {
        const uint32_t s = (blockIdx.x * 256u + threadIdx.x) * 131u + uint32_t(c * 8 + e);
        a[c][e] = __bf16(gauss(mix(2u * s + 1u)));
        b[c][e] = __bf16(gauss(mix(2u * s + 2u)));
      }
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  // keeps the loop alive; the value itself is never used
  if (s == 12345.678f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

// Launches `blocks` workgroups of 4 waves, each wave `iters` x 8 MFMAs of
// 32 x 32 x 16 (32768 FLOP each), on `stream`, with the operands of `mode`
// (0: small and repeating, 1: random N(0, 1)-like). sink: device
// float[blocks] (written only in a case that does not occur). Returns a
// hipError_t code.
int mis_probe_mfma_bf16(int blocks, int iters, int mode, float *sink, void *stream) {
  if (blocks < 1 || iters < 1 || !sink || (mode != 0 && mode != 1)) return int(hipErrorInvalidValue);
  mfma_peak_kernel<<<dim3(unsigned(blocks)), 256, 0, static_cast<hipStream_t>(stream)>>>(sink, iters, mode);
  return int(hipGetLastError());
}

// FLOPs one launch of mis_probe_mfma_bf16 performs.
double mis_probe_mfma_bf16_flops(int blocks, int iters) {
  return double(blocks) * 4.0 * double(iters) * kChains * 32.0 * 32.0 * 16.0 * 2.0;
}

}  // extern "C"
