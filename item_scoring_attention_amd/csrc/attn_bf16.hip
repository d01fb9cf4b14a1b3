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

// LDS-direct buffer load of 16 bytes per lane: lane l's bytes land at lds + 16*l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds, 16, voff,
                                           0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Two transposing 8-byte LDS reads (see the head-pair kernel's comment) joined
// into one 8-key MFMA operand.
__device__ __forceinline__ bf16x8 ds_read_vt(const char *p_lo, const char *p_hi) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p_lo);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p_hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// DMA kernel. A wave owns 32 query tokens of HPW query heads (1 or 2) that
// share a KV head; a workgroup is TB token blocks x HP wave columns, so it
// covers BM = 32*TB tokens and HP*HPW query heads. With HPW = 2 every K or V
// fragment read from LDS feeds two MFMAs (half the LDS traffic per FLOP) but
// the wave needs the whole register file (one wave per SIMD); with HPW = 1 a
// wave fits in half of it, two waves share each SIMD, and one wave's softmax
// runs while the other's MFMAs execute.
//
// K and V tiles (64 keys x 128 dims, 16 KB each) go from HBM to LDS by buffer
// loads with the LDS-direct form: a wave instruction writes 1 KB of LDS
// contiguously (lane l at +16*l), so the layout is chosen by which global
// 16-byte chunk each lane fetches. Both tiles are row-major [key][dim] with
// 256-byte rows and an XOR swizzle of the 16-byte chunk index:
//   K: chunk c of key r sits in slot c ^ (r & 15): the 16 consecutive keys
//      that 16 lanes of one ds_read_b128 read at the same chunk land in 16
//      different slots (all 64 banks);
//   V: chunk c of key r sits in slot c ^ 4*(r & 3): the 4 keys x 4 chunks
//      that 32 lanes of one ds_read_b64_tr_b16 read land in 16 different
//      slots.
// V^T fragments come from ds_read_b64_tr_b16: inside a 16-lane group, lanes
// 4e..4e+3 read dims d0..d0+15 of key k0+e and lane i receives dim d0+i of
// keys k0..k0+3. Two such reads give a lane the 8 keys {4g..4g+3,
// 8+4g..8+4g+3} of a 16-key step that the S^T accumulator hands to P^T.
template <int TB, int HP, int HPW>
__global__ __launch_bounds__(64 * TB * HP, HPW == 1 ? 2 : 1) void attn_dma_kernel(
    const int32_t *__restrict__ work, const int32_t *__restrict__ cu_seqlens,
    const int32_t *__restrict__ prefix_lens, const int32_t *__restrict__ cu_tiles,
    const int8_t *__restrict__ tile_class, const int32_t *__restrict__ item_id,
    const int32_t *__restrict__ item_begin, const __bf16 *__restrict__ q,
    const __bf16 *__restrict__ k, const __bf16 *__restrict__ v, __bf16 *__restrict__ o, int hq,
    int hkv, float c /* softmax scale * log2(e) */) {
  static_assert(HPW == 1 || HPW == 2, "one or two heads per wave");
  constexpr int NW = TB * HP;             // waves
  constexpr int BMT = 32 * TB;            // query tokens per workgroup
  constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
  constexpr int ROWS_PER_WAVE = BN / NW;  // DMA rows per wave and tile
  constexpr int DMA_PER_WAVE = ROWS_PER_WAVE / 4;
  static_assert(BN % (4 * NW) == 0, "DMA split");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[2][2][TILE];  // [stage][K, V]

  const int gsz = hq / hkv;
  const int groups = gsz / (HP * HPW);
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
  const int j1 = min(Tr, qt * BMT + BMT);
  const int b_hi = (j1 + BN - 1) / BN;
  const int b_start = max(b_lo, a_end);
  const int n_visit = a_end + (b_hi - b_start);
  const int cls_base = cu_tiles[r] + qt * nkt;
  const int32_t *cls_words = reinterpret_cast<const int32_t *>(tile_class);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int ql = lane & 31;
  const int tb = wave % TB;
  const int hp = wave / TB;
  const int head0 = kvh * gsz + hc * HP * HPW + HPW * hp;  // heads head0 .. head0 + HPW - 1
  const int j = qt * BMT + tb * 32 + ql;
  const bool row_ok = j < Tr;
  const int jb = (row_ok && j >= lq) ? item_begin[item_id[base + j]] - base : 0;

  const int64_t q_stride = int64_t(hq) * D;
  const int64_t kv_stride = int64_t(hkv) * D;
  const uint32_t kv_row_bytes = uint32_t(kv_stride) * 2u;

  // zero both V stages once: rows past the request end may be left unwritten
  // by the DMA and must not hold NaN (0 * NaN in the PV product)
  for (int i = tid; i < 2 * TILE / 8; i += 64 * NW) {
    const int st = i / (TILE / 8), off = i % (TILE / 8);
    *reinterpret_cast<uint4 *>(&smem[st][1][off * 8]) = make_uint4(0, 0, 0, 0);
  }

  // Q^T operands
  bf16x8 qf[HPW][8];
  {
    const uint32_t q_bytes = uint32_t(Tr) * uint32_t(q_stride) * 2u - uint32_t(head0) * D * 2u;
    const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(q + int64_t(base) * q_stride + int64_t(head0) * D), 0, q_bytes, kRsrcWord3);
    const uint32_t qo = uint32_t(j) * uint32_t(q_stride) * 2u + 16u * g;
#pragma unroll
    for (int h = 0; h < HPW; ++h)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        qf[h][kk] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrsrc, qo + 32u * kk + uint32_t(h) * D * 2u, 0, 0));
  }

  // DMA lane mapping: instruction i of this wave covers tile rows
  // ROWS_PER_WAVE*wave + 4*i + (lane >> 4), LDS slot lane & 15.
  uint32_t koff[DMA_PER_WAVE], voff[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int row = ROWS_PER_WAVE * wave + 4 * i + (lane >> 4);
    const int slot = lane & 15;
    koff[i] = uint32_t(row) * kv_row_bytes + 16u * uint32_t(slot ^ (row & 15));
    voff[i] = uint32_t(row) * kv_row_bytes + 16u * uint32_t(slot ^ (4 * (row & 3)));
  }
  const __bf16 *kreq = k + int64_t(base) * kv_stride + int64_t(kvh) * D;
  const __bf16 *vreq = v + int64_t(base) * kv_stride + int64_t(kvh) * D;
  auto tile_of = [&](int idx) { return idx < a_end ? idx : b_start + (idx - a_end); };
  // Each tile gets descriptors that start at its first key and end at the
  // request's last key of this KV head, so rows past the end read as zero.
  auto issue_tile = [&](int kt, int stage) {
    const int k0 = kt * BN;
    const uint32_t nbytes = uint32_t(Tr - k0) * kv_row_bytes - uint32_t(kvh) * D * 2u;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(kreq + int64_t(k0) * kv_stride), 0, nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(vreq + int64_t(k0) * kv_stride), 0, nbytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      dma16(krs, &smem[stage][0][(ROWS_PER_WAVE * wave + 4 * i) * D], koff[i]);
      dma16(vrs, &smem[stage][1][(ROWS_PER_WAVE * wave + 4 * i) * D], voff[i]);
    }
  };

  // LDS read addresses (bytes within a tile).
  // K: lane reads key 32*b + ql, chunk 2*kk + g -> slot (2*kk + g) ^ (ql & 15).
  uint32_t kaddr[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kaddr[kk] = uint32_t(ql) * 256u + 16u * uint32_t((2 * kk + g) ^ (ql & 15));
  // V: 16-lane group G, e = (lane >> 2) & 3, qd = lane & 3: key 4*(G >> 1) + e (+16*ks, +8),
  // dims 32*db + 16*(G & 1) + 4*qd -> chunk 4*db + 2*(G & 1) + (qd >> 1), half (qd & 1).
  uint32_t vaddr[4];
  {
    const int G = lane >> 4, e = (lane >> 2) & 3, qd = lane & 3;
    const int key = 4 * (G >> 1) + e;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = 4 * db + 2 * (G & 1) + (qd >> 1);
      vaddr[db] = uint32_t(key) * 256u + 16u * uint32_t(chunk ^ (4 * (key & 3))) + 8u * uint32_t(qd & 1);
    }
  }

  f32x16 oacc[HPW][4];
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 16; ++a) oacc[h][db][a] = 0.f;
  float ms[HPW], ls[HPW];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    ms[h] = -1e30f;
    ls[h] = 0.f;
  }

  __syncthreads();  // V zero fill done before any DMA lands
  issue_tile(tile_of(0), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < n_visit; ++it) {
    const int kt = tile_of(it);
    const int stage = it & 1;
    if (it + 1 < n_visit) issue_tile(tile_of(it + 1), stage ^ 1);
    const char *kb = reinterpret_cast<const char *>(smem[stage][0]);
    const char *vb = reinterpret_cast<const char *>(smem[stage][1]);

    // S^T = K Q^T over both 32-key blocks; each K fragment feeds HPW MFMAs
    f32x16 sacc[HPW][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int h = 0; h < HPW; ++h)
#pragma unroll
        for (int a = 0; a < 16; ++a) sacc[h][b][a] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kb + kaddr[kk] + 32 * 256 * b);
#pragma unroll
        for (int h = 0; h < HPW; ++h)
          sacc[h][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[h][kk], sacc[h][b], 0, 0, 0);
      }
    }

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
#pragma unroll
          for (int h = 0; h < HPW; ++h) sacc[h][b][a] = vis ? sacc[h][b][a] : -INFINITY;
        }
    }

    // online softmax per head -> P^T operands
    bf16x8 pf[HPW][4];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      float mx = sacc[h][0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[h][b][a]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mcand = mx * c;
      const bool upd = mcand > ms[h] + kRescaleThreshold;
      if (__any(upd)) {
        const float alpha = upd ? __builtin_amdgcn_exp2f(ms[h] - mcand) : 1.0f;
        ms[h] = upd ? mcand : ms[h];
        ls[h] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int a = 0; a < 16; ++a) oacc[h][db][a] *= alpha;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 16; ++a)
          pf[h][2 * b + (a >> 3)][a & 7] = __bf16(__builtin_amdgcn_exp2f(fmaf(sacc[h][b][a], c, -ms[h])));
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          bf16x2 pp = {pf[h][x][2 * y], pf[h][x][2 * y + 1]};
          ls[h] = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls[h], false);
        }
    }

    // O^T += V^T P^T; each V fragment feeds HPW MFMAs
#pragma unroll
    for (int ksx = 0; ksx < 4; ++ksx) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = ds_read_vt(vb + vaddr[db] + ksx * 16 * 256, vb + vaddr[db] + ksx * 16 * 256 + 8 * 256);
#pragma unroll
        for (int h = 0; h < HPW; ++h)
          oacc[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[h][ksx], oacc[h][db], 0, 0, 0);
      }
    }

    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA for the next tile has landed
    __syncthreads();                // ... and every wave's, and nobody reads this stage any more
  }

  if (row_ok) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float inv = 1.0f / (ls[h] + __shfl_xor(ls[h], 32));
      __bf16 *op = o + int64_t(base + j) * q_stride + int64_t(head0 + h) * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = __bf16(oacc[h][db][4 * a4 + e] * inv);
          *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * a4 + 4 * g) = ov;
        }
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
  int64_t blocks;
  if (gsz % 2 == 0) {  // 2 token blocks x 2 heads, one head per wave, two waves per SIMD
    blocks = int64_t(seg.num_work) * hkv * (gsz / 2);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    attn_dma_kernel<2, 2, 1><<<dim3(unsigned(blocks)), 256, 0, st>>>(
        seg.work, seg.cu_seqlens, seg.prefix_lens, seg.cu_tiles, seg.tile_class, seg.item_id,
        seg.item_begin, qp, kp, vp, op, hq, hkv, c);
  } else {  // odd group size: 2 token blocks x 1 head
    blocks = int64_t(seg.num_work) * hkv * gsz;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    attn_dma_kernel<2, 1, 1><<<dim3(unsigned(blocks)), 128, 0, st>>>(
        seg.work, seg.cu_seqlens, seg.prefix_lens, seg.cu_tiles, seg.tile_class, seg.item_id,
        seg.item_begin, qp, kp, vp, op, hq, hkv, c);
  }
  return hipGetLastError();
}

}  // namespace mis
