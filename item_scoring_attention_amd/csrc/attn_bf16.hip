// bf16 MIS prefill attention on CDNA4 MFMA (gfx950).
//
// Computes O = softmax(scale * Q K^T + M) V per query head with the mask M of
// From Generation to Scoring, §4.1, Eq. 4: a prefix row sees the prefix up to
// itself; an item row sees the whole prefix and its own item up to itself.
// Flash-style online softmax: key tiles are streamed through LDS and key
// tiles that hold only other items' tokens are never visited (From Generation to Scoring,
// §4.3: the remark that the MIS kernels skip fully masked tiles; the SGLang blog's
// list of FlashInfer changes).
//
// Work decomposition
//   A workgroup takes one 64-token query tile, one KV head and HP query heads
//   of that KV head: TB = 2 token blocks x HP heads, one wave per (32 query
//   tokens, head). A wave needs ~180 VGPRs, so two waves share each SIMD and
//   one wave's softmax runs beside the other's MFMAs: HP = 2 runs two
//   workgroups per CU, HP = 4 (GQA groups of 4 or more, enough work) one
//   workgroup of 8 waves that shares each staged K/V tile among 4 heads, and
//   HP = 1 serves odd group sizes. The workgroup order
//   puts the KV head in the fastest-varying position, so with 8 KV heads
//   every XCD (workgroups are dealt round-robin to the 8 XCDs) serves one KV
//   head and its K/V stay in that XCD's L2. Query tiles arrive longest first
//   from the builder's work list.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64)
//   S^T = K Q^T: A = K rows (keys) from LDS, B = Q^T (queries) held in
//   registers for the whole kernel. Accumulator element a of lane l is
//   S^T[key 8*(a/4) + 4*(l/32) + a%4][query l%32], so every lane owns one
//   query column: the row max needs one exchange with lane l^32 and the row
//   sum none until the end.
//   O^T += V^T P^T: B = P^T comes straight from the S^T accumulator (rounded
//   to bf16); its 8 slots per lane hold keys {4g..4g+3, 8+4g..8+4g+3} of a
//   16-key step (g = l/32). A = V^T holds the same keys in the same slots
//   (ds_read_b64_tr_b16, below); the two operands only need to agree on which
//   key sits in which slot.
//
// K and V tiles (64 keys x 128 dims, 16 KB each) go from HBM to LDS by buffer
// loads in the LDS-direct form, double-buffered: tile i+1 is requested when
// tile i's iteration starts. A wave instruction writes 1 KB of LDS
// contiguously (lane l at +16*l), so the layout is chosen by which global
// 16-byte chunk each lane fetches. Both tiles are row-major [key][dim] with
// 256-byte rows and an XOR swizzle of the 16-byte chunk:
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
// The compiler makes its first transposing read wait for every outstanding
// LDS-direct load, which would stall PV on the next tile's transfer; the
// reads are therefore issued through inline asm with explicit waits.
//
// Softmax in the exp2 domain with the scale folded into one FMA per score.
// The running maximum is only raised when it grows by more than 2^8 (a
// stale maximum keeps every p <= 256 and is exact because O and the row sum
// share it); the O rescale is skipped when no lane of the wave raised it.
// Row sums add the bf16-rounded P (the values the PV product uses), two per
// v_dot2_f32_bf16.
#include <atomic>
#include <utility>

#include "gfx950_util.h"
#include "mis_internal.h"
#include "rope_math.h"

namespace mis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int BM = kAttnBlockM;  // query tokens per workgroup
constexpr int BN = kAttnBlockN;  // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 of the largest allowed p

static_assert(BN == 64 && BM == 64, "kernel written for 64 x 64 tiles");

__device__ constexpr bf16x2 kOnes2 = {__bf16(1.0f), __bf16(1.0f)};

// The two transposing 8-byte reads of one V^T fragment: keys k0..k0+3 at
// addr + OFF, keys k0+8..k0+11 eight rows (2048 bytes) further. The results
// are not ready when the asm ends: vt_wait<N> must come before any use.
template <int OFF>
__device__ __forceinline__ void vt_read(uint32_t addr, s16x4 &lo, s16x4 &hi) {
  static_assert(OFF >= 0 && OFF + 2048 < 65536, "DS offset field");
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=&v"(lo), "=v"(hi)
               : "v"(addr), "n"(OFF), "n"(OFF + 2048)
               : "memory");
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, so that I can feed
// template arguments (immediate offsets and wait counts).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait until at most N LDS operations of this wave are outstanding. LDS
// operations complete in order, so the reads issued before the last N have
// landed. The fragment registers are tied to the wait, so the compiler can
// neither read nor move them before it.
template <int N>
__device__ __forceinline__ bf16x8 vt_wait(s16x4 &lo, s16x4 &hi) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(lo), "+v"(hi) : "n"(N));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 16-byte K fragment read (ds_read_b128 at addr + OFF) through inline
// asm; like vt_read, the result is valid only after a frag_wait.
template <int OFF>
__device__ __forceinline__ void k_read(uint32_t addr, bf16x8 &f) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "n"(OFF) : "memory");
}

template <int N>
__device__ __forceinline__ void lgkm_wait(bf16x8 &f) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f) : "n"(N));
}

// Fragment reads run KD fragments ahead of the MFMAs that use them.
constexpr int KD = 4;

// S^T (64 keys x 32 queries, two accumulators) of the K tile at LDS byte
// offset KOFF. Fragment f covers dims 16*(f/2) .. +16 of key block f%2; the
// lane reads key 32*(f%2) + l%32 at the swizzled address kaddr[f/2]
// (absolute LDS address of that slot in a tile at offset 0).
template <int KOFF>
__device__ __forceinline__ void qk_tile(const uint32_t (&kaddr)[8], const bf16x8 (&qf)[8], f32x16 (&sacc)[2]) {
  bf16x8 kf[KD + 1];
  auto kread = [&](auto fc) {
    constexpr int f = decltype(fc)::value;
    k_read<KOFF + (f & 1) * 32 * 256>(kaddr[f >> 1], kf[f % (KD + 1)]);
  };
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int a = 0; a < 16; ++a) sacc[b][a] = 0.f;
  static_for<KD>(kread);
  static_for<16>([&](auto fc) {
    constexpr int f = decltype(fc)::value;
    if constexpr (f + KD < 16) kread(std::integral_constant<int, f + KD>{});
    lgkm_wait<(15 - f < KD ? 15 - f : KD)>(kf[f % (KD + 1)]);
    sacc[f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[f % (KD + 1)], qf[f >> 1], sacc[f & 1], 0, 0, 0);
  });
}

// O^T += V^T P^T over the V tile at LDS byte offset VOFF: 16 steps, ks =
// step/4 picks 16 keys (4096 bytes further each), db = step%4 picks 32 dims
// (vaddr[db]: absolute LDS address in a tile at offset 0).
template <int VOFF>
__device__ __forceinline__ void pv_tile(const uint32_t (&vaddr)[4], const bf16x8 (&pf)[4], f32x16 (&oacc)[4]) {
  s16x4 lo[KD + 1], hi[KD + 1];
  auto vread = [&](auto sc) {
    constexpr int step = decltype(sc)::value;
    vt_read<VOFF + (step >> 2) * 16 * 256>(vaddr[step & 3], lo[step % (KD + 1)], hi[step % (KD + 1)]);
  };
  static_for<KD>(vread);
  static_for<16>([&](auto sc) {
    constexpr int step = decltype(sc)::value;
    if constexpr (step + KD < 16) vread(std::integral_constant<int, step + KD>{});
    const bf16x8 vf = vt_wait<2 * (15 - step < KD ? 15 - step : KD)>(lo[step % (KD + 1)], hi[step % (KD + 1)]);
    oacc[step & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[step >> 2], oacc[step & 3], 0, 0, 0);
  });
}

// Eq. 4 mask of key tile kt for this lane's query row j (prefix keys up to
// j; for an item row also its own item's keys from jb on); out-of-range and
// invisible cells become -inf.
__device__ __forceinline__ void mask_tile(f32x16 (&sacc)[2], int kt, int g, int j, int lq, int jb) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int key = kt * BN + 32 * b + 8 * (a >> 2) + 4 * g + (a & 3);
      const bool vis = key <= j && (key < lq || key >= jb);
      sacc[b][a] = vis ? sacc[b][a] : -INFINITY;
    }
}

// Online softmax of one S^T tile (exp2 domain, c = scale * log2 e): raises
// the running maximum ms lazily, rescales O and the two partial row sums when
// it does, and leaves P^T (bf16) in pf. Max and sums use independent chains.
__device__ __forceinline__ void softmax_tile(const f32x16 (&sacc)[2], float c, float &ms, float (&ls)[2],
                                             f32x16 (&oacc)[4], bf16x8 (&pf)[4]) {
  float m2[2];  // one chain of three-input maxima per key block
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    m2[b] = fmaxf(fmaxf(sacc[b][0], sacc[b][1]), sacc[b][2]);
#pragma unroll
    for (int a = 3; a < 15; a += 2) m2[b] = fmaxf(fmaxf(m2[b], sacc[b][a]), sacc[b][a + 1]);
    m2[b] = fmaxf(m2[b], sacc[b][15]);
  }
  float mx = fmaxf(m2[0], m2[1]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mcand = mx * c;
  const bool upd = mcand > ms + kRescaleThreshold;
  if (__any(upd)) {
    const float alpha = upd ? __builtin_amdgcn_exp2f(ms - mcand) : 1.0f;
    ms = upd ? mcand : ms;
    ls[0] *= alpha;
    ls[1] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 16; ++a) oacc[db][a] *= alpha;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int a = 0; a < 16; ++a)
      pf[2 * b + (a >> 3)][a & 7] = __bf16(__builtin_amdgcn_exp2f(fmaf(sacc[b][a], c, -ms)));
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      bf16x2 pp = {pf[x][2 * y], pf[x][2 * y + 1]};
      ls[y & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls[y & 1], false);
    }
}

// Two workgroups per CU (the 64 KB of K/V stages allow no more): two waves
// per SIMD with 2 heads, one with a single head.
template <int TB, int HP>
__global__ __launch_bounds__(64 * TB * HP, HP == 2 ? 2 : 1) void attn_dma_kernel(
    const int32_t *__restrict__ work, const int32_t *__restrict__ cu_seqlens,
    const int32_t *__restrict__ prefix_lens, const int32_t *__restrict__ cu_tiles,
    const int8_t *__restrict__ tile_class, const int32_t *__restrict__ pos_id, const __bf16 *__restrict__ q,
    const __bf16 *__restrict__ k, const __bf16 *__restrict__ v, __bf16 *__restrict__ o, int hq,
    int hkv, float c /* softmax scale * log2(e) */, int items_only, const float *__restrict__ rope_cs) {
  constexpr int NW = TB * HP;             // waves
  constexpr int BMT = 32 * TB;            // query tokens per workgroup
  constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
  constexpr int ROWS_PER_WAVE = BN / NW;  // DMA rows per wave and tile
  constexpr int DMA_PER_WAVE = ROWS_PER_WAVE / 4;
  static_assert(BN % (4 * NW) == 0, "DMA split");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[2][2][TILE];  // [stage][K, V]

  const int gsz = hq / hkv;
  const int groups = gsz / HP;
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
  // Appending items to a cached prefix: a query tile that holds prefix rows
  // only has nothing to compute (the whole workgroup leaves together).
  if (items_only && qt * BMT + BMT <= lq) return;
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
  const int head = kvh * gsz + hc * HP + hp;
  const int j = qt * BMT + tb * 32 + ql;
  const bool row_ok = j < Tr;
  // an item row at offset d of its item has position id lq + d (the reused
  // positions), so its item starts at row j - d
  const int jb = (row_ok && j >= lq) ? j - (pos_id[base + j] - lq) : 0;

  const int64_t q_stride = int64_t(hq) * D;
  const int64_t kv_stride = int64_t(hkv) * D;
  const uint32_t kv_row_bytes = uint32_t(kv_stride) * 2u;

  // Zero both V stages once: rows past the request end may be left unwritten
  // by the DMA and must not hold NaN (0 * NaN in the PV product).
  for (int i = tid; i < 2 * TILE / 8; i += 64 * NW) {
    const int st = i / (TILE / 8), off = i % (TILE / 8);
    *reinterpret_cast<uint4 *>(&smem[st][1][off * 8]) = make_uint4(0, 0, 0, 0);
  }

  // Q^T operands; rows past the request end read as zeros (never stored).
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
  // Q rotated here when the caller passes the rotary table (cos, sin of every
  // position and pair): qf[kk] and qf[kk + 4] hold the two halves of the
  // lane's pairs 16 kk + 8 g .. + 7. Rows past the request end are zeros.
  if (rope_cs) {
    const float4 *tp = reinterpret_cast<const float4 *>(rope_cs + int64_t(row_ok ? pos_id[base + j] : 0) * D);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float cs[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 t = tp[8 * kk + 4 * g + u];
        cs[4 * u] = t.x, cs[4 * u + 1] = t.y, cs[4 * u + 2] = t.z, cs[4 * u + 3] = t.w;
      }
      rope_rotate8(qf[kk], qf[kk + 4], cs);
    }
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
  // LDS read addresses (bytes within a tile).
  // K: lane reads key 32*b + ql, chunk 2*kk + g -> slot (2*kk + g) ^ (ql & 15).
  uint32_t kaddr[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    kaddr[kk] = lds_addr(smem) + uint32_t(ql) * 256u + 16u * uint32_t((2 * kk + g) ^ (ql & 15));
  // V: 16-lane group G, e = (lane >> 2) & 3, qd = lane & 3: key 4*(G >> 1) + e (+16*ks, +8),
  // dims 32*db + 16*(G & 1) + 4*qd -> chunk 4*db + 2*(G & 1) + (qd >> 1), half (qd & 1).
  uint32_t vaddr[4];
  {
    const int G = lane >> 4, e = (lane >> 2) & 3, qd = lane & 3;
    const int key = 4 * (G >> 1) + e;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = 4 * db + 2 * (G & 1) + (qd >> 1);
      vaddr[db] = lds_addr(smem) + uint32_t(key) * 256u + 16u * uint32_t(chunk ^ (4 * (key & 3))) +
                  8u * uint32_t(qd & 1);
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 16; ++a) oacc[db][a] = 0.f;
  float ms = -1e30f, ls[2] = {0.f, 0.f};

  // Each tile gets descriptors that start at its first key and end at the
  // request's last key of this KV head, so rows past the end read as zero
  // (the range check covers only the per-lane offset).
  auto issue_tile = [&](int kt, int stage) {
    const int k0 = kt * BN;
    const uint32_t nbytes = uint32_t(Tr - k0) * kv_row_bytes - uint32_t(kvh) * D * 2u;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(kreq + int64_t(k0) * kv_stride), 0, nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(vreq + int64_t(k0) * kv_stride), 0, nbytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      lds_load16(krs, &smem[stage][0][(ROWS_PER_WAVE * wave + 4 * i) * D], koff[i]);
      lds_load16(vrs, &smem[stage][1][(ROWS_PER_WAVE * wave + 4 * i) * D], voff[i]);
    }
  };

  __syncthreads();  // V zero fill done before any DMA lands
  issue_tile(tile_of(0), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Visit `it` uses stage S = it % 2 (a template argument, so every LDS
  // address is a fixed per-lane register plus an immediate offset).
  constexpr int STAGE_BYTES = 2 * TILE * 2;  // K + V
  auto visit = [&](int it, auto sc) {
    constexpr int S = decltype(sc)::value;
    const int kt = tile_of(it);
    if (it + 1 < n_visit) issue_tile(tile_of(it + 1), S ^ 1);
    f32x16 sacc[2];
    qk_tile<S * STAGE_BYTES>(kaddr, qf, sacc);
    const int ci = cls_base + kt;
    const int cls = (cls_words[ci >> 2] >> (8 * (ci & 3))) & 0xff;
    if ((cls != 2) || (kt * BN + BN > Tr)) mask_tile(sacc, kt, g, j, lq, jb);
    bf16x8 pf[4];
    softmax_tile(sacc, c, ms, ls, oacc, pf);
    pv_tile<S * STAGE_BYTES + TILE * 2>(vaddr, pf, oacc);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA for the next tile has landed
    __syncthreads();                // ... and every wave's, and nobody reads this stage any more
  };
  for (int it = 0; it < n_visit; it += 2) {
    visit(it, std::integral_constant<int, 0>{});
    if (it + 1 < n_visit) visit(it + 1, std::integral_constant<int, 1>{});
  }

  if (row_ok) {
    const float lsum = ls[0] + ls[1];
    const float inv = 1.0f / (lsum + __shfl_xor(lsum, 32));
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

template <int TB, int HP>
hipError_t launch_variant(const mis_segments &seg, const __bf16 *qp, const __bf16 *kp, const __bf16 *vp,
                          __bf16 *op, int hq, int hkv, float c, int items_only, const float *rope_cs, hipStream_t st) {
  const int64_t blocks = int64_t(seg.num_work) * hq / HP;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  attn_dma_kernel<TB, HP><<<dim3(unsigned(blocks)), 64 * TB * HP, 0, st>>>(
      seg.work, seg.cu_seqlens, seg.prefix_lens, seg.cu_tiles, seg.tile_class, seg.pos_id, qp, kp, vp, op,
      hq, hkv, c, items_only, rope_cs);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (queried once per device).
int device_cus() {
  // per device, queried once; threads that race here store the same value
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

AttnKernel pick_attention_bf16(const mis_segments &seg, int hq, int hkv, AttnForce force) {
  const int gsz = hq / hkv;
  // The pipelined loops are generated for even GQA group sizes; odd ones
  // (MHA included) always take this file's plain loop with one head.
  if (gsz % 2 != 0) return AttnKernel::Classic1;
  switch (force) {
    case AttnForce::Pipe: return gsz % 4 == 0 ? AttnKernel::Pipe4 : AttnKernel::Pipe2;
    case AttnForce::Pipe2: return AttnKernel::Pipe2;
    case AttnForce::Pipe32: return AttnKernel::Pipe32;
    case AttnForce::Classic: return AttnKernel::Classic2;
    case AttnForce::Auto: break;
  }
  // The loop with 64 query rows per wave reads half the LDS per MFMA of the
  // 32-row loop, but runs one wave per SIMD, so it cannot hide the fixed
  // cost of starting a query tile behind another workgroup. Measured on the
  // workloads here: GQA groups of 4 or more take it with 4 heads per
  // workgroup when query tiles visit 48 key tiles or more on average and
  // every CU gets at least 8 such workgroups (the long-prefix batch); groups
  // of 2 (or 6, 10, ...) take it with 2 heads per workgroup from 20 visits
  // per query tile on (2048- to 8192-token prefixes with 64 items: 3-7%
  // faster; shorter prefixes and the profile-labeling batch: 4-8% slower).
  // Other shapes take the 32-row loop, two waves per SIMD.
  const int64_t visits = seg.num_visits, tiles = seg.num_work;
  if (gsz % 4 == 0 && visits >= 48 * tiles && tiles * (hq / 4) >= 8 * int64_t(device_cus()))
    return AttnKernel::Pipe4;
  if (gsz % 4 == 2 && visits >= 20 * tiles) return AttnKernel::Pipe2;
  return AttnKernel::Pipe32;
}

const char *attention_bf16_name(AttnKernel k) {
  switch (k) {
    case AttnKernel::Pipe4: return "attn_pipe_kernel<4, 1>";
    case AttnKernel::Pipe2: return "attn_pipe_kernel<2, 1>";
    case AttnKernel::Pipe32: return "attn_pipe_kernel<2, 2>";
    case AttnKernel::Classic2: return "attn_dma_kernel<2, 2>";
    case AttnKernel::Classic1: return "attn_dma_kernel<2, 1>";
  }
  return "";
}

hipError_t launch_attention_bf16(const mis_segments &seg, const void *q, const void *k,
                                 const void *v, void *o, int hq, int hkv, int d, float scale,
                                 int items_only, AttnKernel kernel, const float *rope_cs, hipStream_t st) {
  if (d != D) return hipErrorInvalidValue;
  const float c = scale * kLog2e;
  const __bf16 *qp = static_cast<const __bf16 *>(q);
  const __bf16 *kp = static_cast<const __bf16 *>(k);
  const __bf16 *vp = static_cast<const __bf16 *>(v);
  __bf16 *op = static_cast<__bf16 *>(o);
  switch (kernel) {
    case AttnKernel::Pipe4:
      return launch_attention_bf16_pipe(seg, q, k, v, o, hq, hkv, scale, items_only, 4, rope_cs, st);
    case AttnKernel::Pipe2:
      return launch_attention_bf16_pipe(seg, q, k, v, o, hq, hkv, scale, items_only, 2, rope_cs, st);
    case AttnKernel::Pipe32:
      return launch_attention_bf16_pipe32(seg, q, k, v, o, hq, hkv, scale, items_only, rope_cs, st);
    case AttnKernel::Classic2: return launch_variant<2, 2>(seg, qp, kp, vp, op, hq, hkv, c, items_only, rope_cs, st);
    case AttnKernel::Classic1: return launch_variant<2, 1>(seg, qp, kp, vp, op, hq, hkv, c, items_only, rope_cs, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mis
