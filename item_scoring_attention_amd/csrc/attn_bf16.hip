// bf16 MIS prefill attention on CDNA4 MFMA (gfx950).
//
// Computes O = softmax(scale * Q K^T + M) V per query head with the mask M of
// From Generation to Scoring, §4.1, Eq. 4: a prefix row sees the prefix up to
// itself; an item row sees the whole prefix and its own item up to itself.
// Flash-style online softmax: key tiles are streamed through LDS and key
// tiles that hold only other items' tokens are never visited (the paper's
// §4.3 remark that the MIS kernels skip fully masked tiles; the SGLang blog's
// list of FlashInfer changes).
//
// Work decomposition
//   workgroup = (query tile of 64 tokens, KV head, group of HG query heads of
//   that KV head); 2*HG waves, wave = 32 query tokens x 1 query head. The
//   workgroup order puts the KV head in the fastest-varying position, so with
//   8 KV heads every XCD (workgroups are dealt round-robin to the 8 XCDs)
//   serves one KV head and its K/V stay in that XCD's L2. Query tiles arrive
//   longest first from the builder's work list.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64)
//   S^T = K Q^T: A = K rows (keys) from LDS, B = Q^T (queries) held in
//   registers for the whole kernel. Accumulator element a of lane l is
//   S^T[key 8*(a/4) + 4*(l/32) + a%4][query l%32], so every lane owns one
//   query column: the row max needs one exchange with lane l^32 and the row
//   sum none until the end.
//   O^T += V^T P^T: B = P^T comes straight from the S^T accumulator (rounded
//   to bf16); its 8 slots per lane hold keys {4g..4g+3, 8+4g..8+4g+3} of a
//   16-key step (g = l/32). A = V^T is stored in LDS with the same key order
//   inside every 16-key group (4-key groups 1 and 2 swapped), so a lane reads
//   its 8 keys with one 16-byte load. The two operands only need to agree on
//   which key sits in which slot.
//
// Softmax in the exp2 domain with the scale folded into one FMA per score.
// The running maximum is only raised when it grows by more than 2^8 (a
// stale maximum keeps every p <= 256 and is exact because O and the row sum
// share it); the O rescale is skipped when no lane of the wave raised it.
#include "mis_internal.h"

namespace mis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int BM = kAttnBlockM;      // query tokens per workgroup
constexpr int BN = kAttnBlockN;      // keys per LDS tile
constexpr int K_LD = D + 8;          // K tile row pitch (bf16), 272 B: conflict-free 16 B reads
constexpr int VT_LD = BN + 8;        // V^T tile row pitch (bf16), 144 B
constexpr int K_TILE = BN * K_LD;    // bf16 elements
constexpr int VT_TILE = D * VT_LD;
constexpr int STAGE = K_TILE + VT_TILE;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 of the largest allowed p
// Fourth descriptor word of a raw (stride 0) buffer resource on CDNA: 32-bit
// data format, so offsets are in bytes and out-of-range reads return zero.
constexpr int kRsrcWord3 = 0x00020000;

static_assert(BN == 64 && BM == 64, "kernel written for 64 x 64 tiles");

__device__ constexpr bf16x2 kOnes2 = {__bf16(1.0f), __bf16(1.0f)};

// Column of key kk (0..BN-1) in a V^T row: 4-key groups 1 and 2 of every
// 16-key group swap places.
__device__ __forceinline__ int vt_col(int kk) {
  const int sub = (kk >> 2) & 3;
  const int sub2 = (sub == 1) ? 2 : (sub == 2 ? 1 : sub);
  return (kk & ~15) | (sub2 << 2) | (kk & 3);
}

template <int HG>
__global__ __launch_bounds__(128 * HG, 2) void attn_bf16_kernel(
    const int32_t *__restrict__ work, const int32_t *__restrict__ cu_seqlens,
    const int32_t *__restrict__ prefix_lens, const int32_t *__restrict__ cu_tiles,
    const int8_t *__restrict__ tile_class, const int32_t *__restrict__ item_id,
    const int32_t *__restrict__ item_begin, const __bf16 *__restrict__ q,
    const __bf16 *__restrict__ k, const __bf16 *__restrict__ v, __bf16 *__restrict__ o, int hq,
    int hkv, float c /* softmax scale * log2(e) */) {
  constexpr int NT = 128 * HG;  // threads
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

  const int groups = (hq / hkv) / HG;  // head groups per KV head
  const int kvh = blockIdx.x % hkv;
  const int rest = blockIdx.x / hkv;
  const int hc = rest % groups;
  const int w = rest / groups;

  const int r = work[4 * w + 0];
  const int qt = work[4 * w + 1];
  const int a_end = work[4 * w + 2];
  const int b_lo = work[4 * w + 3];
  const int base = cu_seqlens[r];
  const int Tr = cu_seqlens[r + 1] - base;
  const int lq = prefix_lens[r];
  const int nkt = (Tr + BN - 1) / BN;
  const int j1 = min(Tr, qt * BM + BM);
  const int b_hi = (j1 + BN - 1) / BN;
  const int b_start = max(b_lo, a_end);
  const int n_visit = a_end + (b_hi - b_start);
  const int cls_base = cu_tiles[r] + qt * nkt;  // tile_class index of key tile 0
  const int32_t *cls_words = reinterpret_cast<const int32_t *>(tile_class);  // 256-byte aligned

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63;
  const int g = lane >> 5;   // half-wave
  const int ql = lane & 31;  // query column owned by this lane
  const int tb = wave & 1;   // 32-token sub-block
  const int hh = wave >> 1;  // head within the workgroup
  const int head = kvh * (hq / hkv) + hc * HG + hh;
  const int j = qt * BM + tb * 32 + ql;  // request-local query row
  const bool row_ok = j < Tr;
  // Start of the row's own item (request-local); prefix rows never need it.
  const int jb = (row_ok && j >= lq) ? item_begin[item_id[base + j]] - base : 0;

  const int64_t q_stride = int64_t(hq) * D;
  const int64_t kv_stride = int64_t(hkv) * D;

  // Q^T operand: 8 k-steps of 16 head dims, 8 consecutive dims per lane.
  // Rows past the request end read as zeros (their outputs are not stored).
  bf16x8 qf[8];
  {
    const uint32_t q_bytes = uint32_t(Tr) * uint32_t(q_stride) * 2u - uint32_t(head) * D * 2u;
    const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(q + int64_t(base) * q_stride + int64_t(head) * D), 0, q_bytes, kRsrcWord3);
    const uint32_t qo = uint32_t(j) * uint32_t(q_stride) * 2u + 16u * g;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrsrc, qo + 32u * kk, 0, 0));
  }

  // Global -> register staging of one K/V tile through raw buffer loads: the
  // resources span exactly this request's rows of this KV head, so rows at or
  // beyond the request end read as zeros without a branch.
  // K: 64 rows x 16 chunks of 8 dims = 1024 chunks; thread covers chunks tid + NT*i.
  // V: 16 groups of 4 keys x 16 groups of 8 dims = 256 blocks; thread covers tid + NT*i.
  constexpr int KCH = (BN * D / 8) / NT;
  constexpr int VBL = 256 / NT;
  uint4 kreg[KCH];
  uint4 vreg[VBL][4];
  const uint32_t kv_row_bytes = uint32_t(kv_stride) * 2u;
  const __bf16 *kreq = k + int64_t(base) * kv_stride + int64_t(kvh) * D;
  const __bf16 *vreq = v + int64_t(base) * kv_stride + int64_t(kvh) * D;
  uint32_t koff[KCH], voff[VBL];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int ch = tid + NT * i;
    koff[i] = uint32_t(ch >> 4) * kv_row_bytes + uint32_t(ch & 15) * 16u;
  }
#pragma unroll
  for (int i = 0; i < VBL; ++i) {
    const int blk = tid + NT * i;
    voff[i] = uint32_t(4 * (blk & 15)) * kv_row_bytes + uint32_t(blk >> 4) * 16u;
  }

  auto tile_of = [&](int idx) { return idx < a_end ? idx : b_start + (idx - a_end); };

  // The buffer range check covers only the per-lane offset, so each tile gets
  // its own descriptor starting at its first key and ending at the request's
  // last key of this KV head (k0 < Tr for every visited tile).
  auto load_tile = [&](int kt) {
    const int k0 = kt * BN;
    const uint32_t nbytes = uint32_t(Tr - k0) * kv_row_bytes - uint32_t(kvh) * D * 2u;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(kreq + int64_t(k0) * kv_stride), 0, nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(vreq + int64_t(k0) * kv_stride), 0, nbytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < KCH; ++i)
      kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, koff[i], 0, 0));
#pragma unroll
    for (int i = 0; i < VBL; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        vreg[i][rr] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[i] + uint32_t(rr) * kv_row_bytes, 0, 0));
  };

  auto store_tile = [&](int buf) {
    __bf16 *ks = smem + buf * STAGE;
    __bf16 *vs = ks + K_TILE;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + NT * i;
      const int row = ch >> 4, col = (ch & 15) * 8;
      *reinterpret_cast<uint4 *>(ks + row * K_LD + col) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VBL; ++i) {
      const int blk = tid + NT * i;
      const int kg = blk & 15, dg = blk >> 4;
      const int col = vt_col(4 * kg);
      // transpose 4 keys x 8 dims -> 8 dims x 4 keys (two bf16 per 32-bit word)
      const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&vreg[i][0]);
      const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&vreg[i][1]);
      const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&vreg[i][2]);
      const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&vreg[i][3]);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        uint2 lo, hi;
        lo.x = (r0[wd] & 0xffffu) | (r1[wd] << 16);
        lo.y = (r2[wd] & 0xffffu) | (r3[wd] << 16);
        hi.x = (r0[wd] >> 16) | (r1[wd] & 0xffff0000u);
        hi.y = (r2[wd] >> 16) | (r3[wd] & 0xffff0000u);
        *reinterpret_cast<uint2 *>(vs + (8 * dg + 2 * wd) * VT_LD + col) = lo;
        *reinterpret_cast<uint2 *>(vs + (8 * dg + 2 * wd + 1) * VT_LD + col) = hi;
      }
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 16; ++a) oacc[db][a] = 0.f;
  float ms = -1e30f;  // running maximum in the scaled (log2) domain
  float lsum = 0.f;   // this lane's share of the row sum

  // Every query tile sees at least its diagonal key tile, so n_visit >= 1.
  load_tile(tile_of(0));
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < n_visit; ++it) {
    const int kt = tile_of(it);
    const int buf = it & 1;
    const bool has_next = it + 1 < n_visit;
    if (has_next) load_tile(tile_of(it + 1));

    const __bf16 *ks = smem + buf * STAGE;
    const __bf16 *vs = ks + K_TILE;

    // S^T for the two 32-key blocks of the tile
    f32x16 sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int a = 0; a < 16; ++a) sacc[b][a] = 0.f;
      const __bf16 *kr = ks + (32 * b + ql) * K_LD + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 af = *reinterpret_cast<const bf16x8 *>(kr + 16 * kk);
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], sacc[b], 0, 0, 0);
      }
    }

    // mask (partly visible tiles and the request's last key tile only)
    const int ci = cls_base + kt;
    const int cls = (cls_words[ci >> 2] >> (8 * (ci & 3))) & 0xff;
    const bool need_mask = (cls != 2) || (kt * BN + BN > Tr);
    if (need_mask) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = kt * BN + 32 * b + 8 * (a >> 2) + 4 * g + (a & 3);
          const bool vis = key <= j && (key < lq || key >= jb);
          sacc[b][a] = vis ? sacc[b][a] : -INFINITY;
        }
    }

    // online softmax
    float mx = sacc[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[b][a]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mcand = mx * c;
    const bool upd = mcand > ms + kRescaleThreshold;
    if (__any(upd)) {
      const float alpha = upd ? __builtin_amdgcn_exp2f(ms - mcand) : 1.0f;
      ms = upd ? mcand : ms;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a = 0; a < 16; ++a) oacc[db][a] *= alpha;
    }
    bf16x8 pf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int a = 0; a < 16; ++a)
        pf[2 * b + (a >> 3)][a & 7] = __bf16(__builtin_amdgcn_exp2f(fmaf(sacc[b][a], c, -ms)));
    // row sum of the bf16-rounded P (the values the PV product uses), two per dot2
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        bf16x2 pp = {pf[x][2 * y], pf[x][2 * y + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, lsum, false);
      }

    // O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
    for (int ksx = 0; ksx < 4; ++ksx) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8 *>(vs + (32 * db + ql) * VT_LD + 16 * ksx + 8 * g);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ksx], oacc[db], 0, 0, 0);
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // normalise and store: lane owns query j, dims 32*db + 8*(a/4) + 4*g + 0..3
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.0f / ltot;
  if (row_ok) {
    __bf16 *op = o + int64_t(base + j) * q_stride + int64_t(head) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = __bf16(oacc[db][4 * a4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * a4 + 4 * g) = ov;
      }
  }
}

}  // namespace

hipError_t launch_attention_bf16(const mis_segments &seg, const void *q, const void *k,
                                 const void *v, void *o, int hq, int hkv, int d, float scale,
                                 hipStream_t st) {
  if (d != D) return hipErrorInvalidValue;
  const int gsz = hq / hkv;
  const float c = scale * kLog2e;
  const __bf16 *qp = static_cast<const __bf16 *>(q);
  const __bf16 *kp = static_cast<const __bf16 *>(k);
  const __bf16 *vp = static_cast<const __bf16 *>(v);
  __bf16 *op = static_cast<__bf16 *>(o);
  if (gsz % 2 == 0) {
    const int64_t blocks = int64_t(seg.num_work) * hkv * (gsz / 2);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    attn_bf16_kernel<2><<<dim3(unsigned(blocks)), 256, 0, st>>>(
        seg.work, seg.cu_seqlens, seg.prefix_lens, seg.cu_tiles, seg.tile_class, seg.item_id,
        seg.item_begin, qp, kp, vp, op, hq, hkv, c);
  } else {
    const int64_t blocks = int64_t(seg.num_work) * hkv * gsz;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    attn_bf16_kernel<1><<<dim3(unsigned(blocks)), 128, 0, st>>>(
        seg.work, seg.cu_seqlens, seg.prefix_lens, seg.cu_tiles, seg.tile_class, seg.item_id,
        seg.item_begin, qp, kp, vp, op, hq, hkv, c);
  }
  return hipGetLastError();
}

}  // namespace mis
