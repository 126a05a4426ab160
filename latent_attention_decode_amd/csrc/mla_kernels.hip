// HIP kernels (gfx950) for single-token multi-head latent attention decode.
//
// Split-K flash-decoding, as in the split kernels of amd-mixed-mla
// submissions 727205 "v25: LEAN" (`mla_s1`) and 599694 "overhead
// elimination" (`_flash_fp8_split_s1`): one 256-thread workgroup per planned
// work item, i.e. a token range of one sequence, streamed in tiles with an
// online softmax.  A workgroup whose item is the whole sequence writes the
// bf16 output; otherwise it writes a normalised partial plus its log-sum-exp.
// An empty sequence's item writes zeros.
//
//   mla_stage1_fp8    fp8 cache (mla_stage1_fp8.hip): 128-token tiles moved
//                     HBM -> LDS by cache-to-LDS loads; both contractions on
//                     fp8 / MX matrix instructions straight on the cached codes.
//   mla_stage1_mxfp4  MXFP4 cache (mla_stage1_mxfp4.hip): the same streaming,
//                     scores on the e2m1 codes with their e8m0 block scales,
//                     V converted to e4m3 per tile for P.V.
//   mla_stage1        (this file) bf16 cache, and MXFP4 whose scale rows are
//                     not 2-byte aligned: 64-token tiles, both contractions
//                     on v_mfma_f32_16x16x32_bf16.  A contiguous bf16 cache
//                     streams into a ring of two LDS buffers by cache-to-LDS
//                     loads (one workgroup per CU); a paged one, and MXFP4
//                     (decoded to bf16 exactly on the way into LDS), are
//                     staged through registers (two workgroups per CU).
//   mla_merge         (this file) per (sequence, quarter of the columns) of
//                     the split sequences, the log-sum-exp weighted merge of
//                     the partials (727205 `mla_rd`; 700955 "locked baseline
//                     dispatch" `reduce_lse_v71`; 599694 `_flash_fp8_split_s2`).
//
// In mla_stage1 wave w scores a quarter of the tile's tokens against the 16
// heads (S^T[token, head] = K Q^T) and accumulates output columns
// 128w..128w+127 over all of the tile's tokens (O^T[dim, head] += V^T P^T,
// V^T through the gfx950 transposing LDS reads); the softmax runs in the log2
// domain with a lazy maximum shared by the four waves, which only moves (and
// O and the sums are rescaled) when a tile maximum passes it by more than 8,
// bounding every weight by 2^8 and keeping the result exact.  Contractions
// over the 576 columns run in a permuted column order (any order common to
// both operands is valid).  Everything accumulates in fp32.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

// ---------------------------------------------------------------------------
// format traits
// ---------------------------------------------------------------------------
template <int F> struct Traits;
template <> struct Traits<kBf16> {  // streamed by cache-to-LDS loads (DmaRing)
  static constexpr int kRowBytes = 1152;
  static constexpr int kLdsPitch = 1168;  // bf16 elements + 16 B
};
template <> struct Traits<kMxfp4> {
  static constexpr int kRowBytes = 288;   // e2m1 nibbles; scales live apart
  static constexpr int kLdsPitch = 1168;  // decoded to bf16 in LDS
  static constexpr int kBuffers = 1;
  static constexpr bool kPrefetch = true;
};

constexpr int kTileTokens = kTile * 2;  // 64 tokens per workgroup iteration

template <int F> struct Tile {
  static constexpr int kChunksPerRow = Traits<F>::kRowBytes / 16;
  static constexpr int kChunkTotal = kTileTokens * kChunksPerRow;
  // 16-B loads per thread (the MXFP4 tile, 1152 chunks, leaves the last one
  // to half of the threads)
  static constexpr int kChunks = (kChunkTotal + kStage1Threads - 1) / kStage1Threads;
  // Each group of 16 rows sits 64 B further on than the one before, which
  // spreads the transposing V reads (rows of two 16-row groups together)
  // over the banks.
  static constexpr int kBytes = kTileTokens * Traits<F>::kLdsPitch + (kTileTokens / 16) * 64;
  __host__ __device__ static constexpr int row_offset(int r) {
    return r * Traits<F>::kLdsPitch + (r >> 4) * 64;
  }
};

// bytes one LDS row holds: the bf16 row (stored, or decoded from MXFP4)
template <int F> constexpr int kLdsRowBytes = 2 * kQkDim;

template <int F> constexpr bool rows_disjoint() {
  for (int r = 0; r + 1 < kTileTokens; ++r)
    if (Tile<F>::row_offset(r) + kLdsRowBytes<F> > Tile<F>::row_offset(r + 1)) return false;
  return Tile<F>::row_offset(kTileTokens - 1) + kLdsRowBytes<F> <= Tile<F>::kBytes;
}
static_assert(rows_disjoint<kBf16>() && rows_disjoint<kMxfp4>(), "LDS tile rows overlap");

static_assert(Tile<kBf16>::kChunks == 18 && Tile<kMxfp4>::kChunks == 5, "tile chunking");

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

// 8 e2m1 nibbles (low nibble first) times 2^(e-127) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Token (within a 32-token P.V step) of element e (0..7) of lane group g.
// Elements 0..3 are the score registers of lane group g of the wave that
// scored the step's first 16 tokens (tokens 4g..4g+3), elements 4..7 those
// of the wave that scored the next 16 (16+4g..16+4g+3).
__device__ __forceinline__ int pv_token(int g, int e) {
  return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4);
}

// ---------------------------------------------------------------------------
// tile loads: global -> registers (one tile ahead) -> LDS
// ---------------------------------------------------------------------------
template <int F, bool PAGED>
struct TileRegs {
  static constexpr int kN = Tile<F>::kChunks;
  static constexpr int kCPR = Tile<F>::kChunksPerRow;
  static constexpr int kRB = Traits<F>::kRowBytes;
  static constexpr int kStepRows = kStage1Threads / kCPR;  // whole rows per 256 chunks
  static constexpr int kStepCols = kStage1Threads % kCPR;
  u32x4 d[kN];
  uint32_t s[F == kMxfp4 ? kN : 1];

  __device__ static bool chunk_live(int j, int tid) {
    return Tile<F>::kChunkTotal % kStage1Threads == 0 ||
           j * kStage1Threads + tid < Tile<F>::kChunkTotal;
  }

  // Issue the loads of the tile starting at logical token `tok0`.  Rows past
  // `tok_last` are replaced by row `tok_last`, so every load is in bounds and
  // every LDS row holds finite data (masked later by index).
  __device__ __forceinline__ void issue(const Stage1Args& a, int64_t seq_base, int tok0,
                                        int tok_last, int tid) {
    if (!PAGED && F != kMxfp4 && tok0 + kTileTokens - 1 <= tok_last) {
      // the whole tile is one contiguous block: thread-contiguous 16-B loads
      const uint8_t* base = a.kv + (seq_base + tok0) * kRB + tid * 16;
#pragma unroll
      for (int j = 0; j < kN; ++j)
        d[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + j * (16 * kStage1Threads)));
      return;
    }
    uint32_t my_row = 0;  // physical row of tile row (tid & 63), paged only
    if (PAGED) {
      const int tok = min(tok0 + (tid & 63), tok_last);
      const int pmask = (1 << a.page_shift) - 1;
      const uint32_t page = (uint32_t)a.page_indices[seq_base + (tok >> a.page_shift)];
      my_row = (page << a.page_shift) + (uint32_t)(tok & pmask);
    }
    int r = tid / kCPR, cc = tid % kCPR;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      if (chunk_live(j, tid)) {
        uint32_t row;
        if (PAGED)
          row = (uint32_t)__shfl((int)my_row, r, 64);
        else
          row = (uint32_t)(seq_base + min(tok0 + r, tok_last));
        d[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.kv + (int64_t)row * kRB + cc * 16));
        if constexpr (F == kMxfp4) s[j] = a.kv_mx_scales[(int64_t)row * a.scale_stride + cc];
      }
      cc += kStepCols;
      r += kStepRows;
      if (cc >= kCPR) { cc -= kCPR; r += 1; }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds_tile, int tid) const {
    int r = tid / kCPR, cc = tid % kCPR;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      if (chunk_live(j, tid)) {
        uint8_t* row = lds_tile + Tile<F>::row_offset(r);
        if constexpr (F == kMxfp4) {
          // chunk cc of a row = the 32 elements of scale block cc
          const float scale = __uint_as_float(s[j] << 23);
          bf16x8* dst = reinterpret_cast<bf16x8*>(row + cc * 64);
          dst[0] = fp4x8_to_bf16(d[j][0], scale);
          dst[1] = fp4x8_to_bf16(d[j][1], scale);
          dst[2] = fp4x8_to_bf16(d[j][2], scale);
          dst[3] = fp4x8_to_bf16(d[j][3], scale);
        } else {
          *reinterpret_cast<u32x4*>(row + cc * 16) = d[j];
        }
      }
      cc += kStepCols;
      r += kStepRows;
      if (cc >= kCPR) { cc -= kCPR; r += 1; }
    }
  }
};

// ---------------------------------------------------------------------------
// stage 1
// ---------------------------------------------------------------------------
// LDS: the tile buffers, and apart from them (a separate object, so that the
// compiler sees these accesses cannot alias the cache-to-LDS loads in flight)
// the bf16 P^T fragments of the four waves, the per-wave tile maxima and sums,
// and (paged fp8) the page ids of the item.
template <int F>
struct Stage1Tiles {
  uint8_t tile[Traits<F>::kBuffers][Tile<F>::kBytes];
};
// The contiguous bf16 cache streams into a ring of two tile buffers by
// cache-to-LDS loads (one workgroup per CU), in the same padded row layout:
// the 74 loads of 1 KB fill the buffer slot by slot, a slot in a row's data
// taking its 16 bytes of the row and a padding slot a harmless copy of the
// row's first 16.
constexpr int kDmaLoads = 74;                 // 1 KB loads per tile buffer
constexpr int kDmaTileBytes = kDmaLoads * 1024;
static_assert(kDmaTileBytes >= Tile<kBf16>::kBytes, "a DMA buffer holds a padded bf16 tile");
struct DmaRing {
  uint8_t tile[2][kDmaTileBytes];
};
// Tile row and 16-byte chunk whose data belongs at byte o of a padded bf16
// tile (chunk 0 of the row for a padding slot; the last row past the end).
// With s = o / 16: a group of 16 rows spans 16 * 73 + 4 = 1172 slots (73 per
// row, the last of them padding, then 4 more), so the row is 16 (s / 1172) +
// (s % 1172) / 73 and the chunk (s % 1172) % 73.
__device__ __forceinline__ void dma_slot_source(int o, int& r, int& c) {
  constexpr int kRowSlots = Traits<kBf16>::kLdsPitch / 16;  // 73
  constexpr int kGroupSlots = 16 * kRowSlots + 4;           // 1172
  const int s = o >> 4;
  const int grp = s / kGroupSlots;
  const int in = s - grp * kGroupSlots;
  const int rr = in / kRowSlots;
  r = min(16 * grp + min(rr, 15), kTileTokens - 1);
  c = in - rr * kRowSlots;
  if (rr > 15 || c >= 2 * kQkDim / 16 || 16 * grp + rr >= kTileTokens) c = 0;  // padding
}

template <int F, bool PAGED>
struct Stage1Lds {
  uint2 p[kWaves][64];               // 4 bf16 probabilities per lane
  f32x4 tmax[kWaves][kNumHeads];     // [wave][head][lane group] tile maxima
  float lsum[kWaves][kNumHeads];
  int32_t pages[F == kBf16 && PAGED ? kItemPagesBf16 : 1];  // paged bf16: page ids of the item
};

// One 64-token tile held in `cur`: scores, shared lazy max, P.V.  Ends after
// the P.V reads were issued; the caller orders what follows.
template <int F, bool PAGED>
__device__ __forceinline__ void attend_tile(Stage1Lds<F, PAGED>& sh, const uint8_t* cur, const bf16x8 (&qf)[18],
                                            f32x4 (&o)[8], float& m_ref, float& l_part,
                                            int tok0, int tok_last, float xscale, int wave,
                                            int lane, int k_off, int v_off_lo, int v_off_hi) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
  // ---- scores S^T for tokens 16*wave .. +15 of the tile ----
  // four independent accumulation chains over the 18 k-steps
  f32x4 sacc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) sacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const uint8_t* kr = cur + k_off;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const bf16x8* p = reinterpret_cast<const bf16x8*>(kr + 128 * j);
      const bf16x8 kl = p[0];
      const bf16x8 kh = p[1];
      const int c = 2 * (j & 1);
      sacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qf[2 * j], sacc[c], 0, 0, 0);
      sacc[c + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qf[2 * j + 1], sacc[c + 1], 0, 0, 0);
    }
  }
  float x[4];
  float tmax = kNegInf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = ((sacc[0][i] + sacc[1][i]) + (sacc[2][i] + sacc[3][i])) * xscale;
    if (tok0 + 16 * wave + 4 * g + i > tok_last) x[i] = kNegInf;
    tmax = fmaxf(tmax, x[i]);
  }
  reinterpret_cast<float*>(&sh.tmax[wave][r16])[g] = tmax;
  float p[4];
  {
    const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mr);
    sh.p[wave][lane] = uint2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  }
  lds_barrier();  // scores, maxima and P of all waves are in LDS

  // ---- lazy rescale: only when a tile max passes m_ref + 8 ----
  float tile_max = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const f32x4 t = sh.tmax[w][r16];
    tile_max = fmaxf(tile_max, fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
  }
  if (__ballot(tile_max > m_ref + kLazyRescale) != 0) {  // same outcome in every wave
    const float m_new = fmaxf(m_ref, tile_max);
    const float alpha = (m_new == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
    for (int v = 0; v < 8; ++v) o[v] *= alpha;
    l_part *= alpha;
    m_ref = m_new;
    const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mr);
    lds_barrier();  // everyone has read the old P
    sh.p[wave][lane] = uint2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    lds_barrier();
  }
  l_part += (p[0] + p[1]) + (p[2] + p[3]);

  // ---- O^T[dims of this wave] += V^T P^T over the 64 tokens ----
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const uint2 p_lo = sh.p[2 * kk][lane];
    const uint2 p_hi = sh.p[2 * kk + 1][lane];
    const bf16x8 pt = __builtin_bit_cast(bf16x8, u32x4{p_lo.x, p_lo.y, p_hi.x, p_hi.y});
    const uint8_t* vb = cur + kk * Tile<F>::row_offset(32);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off_lo + 32 * v));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off_hi + 32 * v));
      const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
      const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
      const bf16x8 va = bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
      o[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pt, o[v], 0, 0, 0);
    }
  }
}

template <int F>
using Stage1Buffers = typename std::conditional<F == kBf16, DmaRing, Stage1Tiles<F>>::type;

// One work item: tokens [tok_begin, tok_end) of one sequence.
template <int F, bool PAGED>
__device__ __forceinline__ void stage1_item(const Stage1Args& a, const WorkItem& item, Stage1Buffers<F>& tiles,
                                            Stage1Lds<F, PAGED>& sh) {
  constexpr bool kDma = F == kBf16;
  const int tid = threadIdx.x;
  if (item.slot == WorkItem::kEmpty) {  // empty sequence: its output is zero
    uint4* dst = reinterpret_cast<uint4*>(a.out + (int64_t)item.batch * kNumHeads * kVDim);
#pragma unroll
    for (int k = 0; k < (kNumHeads * kVDim * 2 / 16) / kStage1Threads; ++k)
      dst[tid + kStage1Threads * k] = uint4{0u, 0u, 0u, 0u};
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63;
  const int r16 = lane & 15;  // MFMA row/column index of this lane
  const int g = lane >> 4;    // MFMA k-group of this lane
  const int b = item.batch;
  const int tok_last = item.tok_end - 1;
  const int ntiles = (item.tok_end - item.tok_begin + kTileTokens - 1) / kTileTokens;
  const int64_t seq_base = item.kv_base;  // kv_indptr[b]: first row, or first page slot

  const float xscale = a.score_scale;

  // Query as the B operand of S^T = K Q^T: lane (head r16, group g) holds,
  // for k-step 2j+h, q[head][64j + 16g + 8h .. +8].
  bf16x8 qf[18];
  {
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
        a.q + ((int64_t)b * kNumHeads + r16) * kQkDim + 16 * g);
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      qf[2 * j] = qrow[8 * j];
      qf[2 * j + 1] = qrow[8 * j + 1];
    }
  }

  // This wave's output: dims 128*wave + 16v + 4g + i of head r16.
  f32x4 o[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // running max (log2 units) of head r16, same in all waves
  float l_part = 0.f;     // this lane's share of the running sum

  // per-lane LDS offsets inside a tile buffer
  const int k_off = Tile<F>::row_offset(16 * wave + r16) + 32 * g;
  const int dv0 = 128 * wave;  // first output column of this wave
  // ds_read_b64_tr_b16: lane quad (4e..4e+3) names row e of a 4 x 16-element
  // block (4 elements each); lane i receives element i of each of the 4 rows.
  const int v_off_lo = Tile<F>::row_offset(pv_token(g, r16 >> 2)) + (r16 & 3) * 8 + 2 * dv0;
  const int v_off_hi = Tile<F>::row_offset(pv_token(g, 4 + (r16 >> 2))) + (r16 & 3) * 8 + 2 * dv0;

  if constexpr (kDma) {
    // ---- cache-to-LDS ring of two buffers ----
    // This wave's loads of a tile: 19 (waves 0, 1) or 18 (waves 2, 3), load
    // j being number l0 + j of the tile's 74, at LDS 1024 (l0 + j).
    const int nl = wave < 2 ? 19 : 18;
    const int l0 = wave < 2 ? 19 * wave : 38 + 18 * (wave - 2);
    int srow[19], scol[19];
#pragma unroll
    for (int j = 0; j < 19; ++j) dma_slot_source(1024 * (l0 + min(j, nl - 1)) + 16 * lane, srow[j], scol[j]);
    int page0 = 0;
    if constexpr (PAGED) {
      // the item's page ids into LDS by four-byte cache-to-LDS loads, all in
      // flight together (lanes past the last page repeat it)
      page0 = item.tok_begin >> a.page_shift;
      const int npages = min(((item.tok_end - 1) >> a.page_shift) - page0 + 1, kItemPagesBf16);
      const int32_t* psrc = a.page_indices + seq_base + page0;
      const uint32_t pm0 = lds_u32(&sh.pages[0]);
      for (int j = wave; 64 * j < npages; j += kWaves) dma_u32(psrc + min(64 * j + lane, npages - 1), pm0 + 256 * j);
    }
    // The query (and the page ids) land before the first tiles are issued:
    // issued together with the first tiles of every CU, the query would
    // queue behind them at the memory and land last.
    wait_loads<0>();
    if constexpr (PAGED) lds_barrier();
    auto issue = [&](int n) {  // tile n into buffer n % 2
      const int tok0 = item.tok_begin + n * kTileTokens;
      const int lim = tok_last - tok0;
      const uint32_t m0 = lds_u32(&tiles.tile[n & 1][0]) + 1024 * l0;
      const uint8_t* src[19];
#pragma unroll
      for (int j = 0; j < 19; ++j) {
        int64_t row;
        if constexpr (PAGED) {
          const int tok = tok0 + min(srow[j], lim);
          const uint32_t page = (uint32_t)sh.pages[(tok >> a.page_shift) - page0];
          row = (int64_t)((page << a.page_shift) + (uint32_t)(tok & ((1 << a.page_shift) - 1)));
        } else {
          row = seq_base + tok0 + min(srow[j], lim);
        }
        src[j] = a.kv + row * (2 * kQkDim) + 16 * scol[j] - (j < 18 ? 1024 * (j & 3) : 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) dma_group<4>(src + 4 * q, m0 + 4096 * q);
      dma_group<2>(src + 16, m0 + 4096 * 4);
      if (nl == 19) dma_one(src[18], m0 + 1024 * 18);
    };
    issue(0);
    if (ntiles > 1) issue(1);
    for (int n = 0; n < ntiles; ++n) {
      const int tok0 = item.tok_begin + n * kTileTokens;
      if (n == 0 && ntiles > 1) {  // tile 0, not tile 1 behind it
        if (nl == 19)
          wait_loads<19>();
        else
          wait_loads<18>();
      } else {
        wait_loads<0>();
      }
      lds_barrier();  // tile n everywhere; everyone is past tile n - 1 (and its P)
      if (n >= 1 && n + 1 < ntiles) issue(n + 1);  // into the buffer tile n - 1 used
      attend_tile<F, PAGED>(sh, tiles.tile[n & 1], qf, o, m_ref, l_part, tok0, tok_last, xscale, wave, lane,
                            k_off, v_off_lo, v_off_hi);
    }
    lds_barrier();  // the last P.V reads are done
  } else {
    // ---- register-staged tiles through one LDS buffer ----
    TileRegs<F, PAGED> regs;
    regs.issue(a, seq_base, item.tok_begin, tok_last, tid);
    regs.store(tiles.tile[0], tid);
    if (Traits<F>::kPrefetch && ntiles > 1)
      regs.issue(a, seq_base, item.tok_begin + kTileTokens, tok_last, tid);
    __syncthreads();
    for (int n = 0; n < ntiles; ++n) {
      const int tok0 = item.tok_begin + n * kTileTokens;
      attend_tile<F, PAGED>(sh, tiles.tile[0], qf, o, m_ref, l_part, tok0, tok_last, xscale, wave, lane,
                     k_off, v_off_lo, v_off_hi);
      __syncthreads();  // P, maxima and the tile buffer are free again
      if (n + 1 < ntiles) {
        if (!Traits<F>::kPrefetch) regs.issue(a, seq_base, tok0 + kTileTokens, tok_last, tid);
        regs.store(tiles.tile[0], tid);
        if (Traits<F>::kPrefetch && n + 2 < ntiles)
          regs.issue(a, seq_base, tok0 + 2 * kTileTokens, tok_last, tid);
        __syncthreads();
      }
    }
  }

  // ---- normalise: every wave shares m_ref, so only the sums need adding ----
  const float l_w = xor_sum_groups(l_part);
  if (g == 0) sh.lsum[wave][r16] = l_w;
  __syncthreads();
  const float L = (sh.lsum[0][r16] + sh.lsum[1][r16]) + (sh.lsum[2][r16] + sh.lsum[3][r16]);
  finish_item<8>(a, item, tid, wave, 0, lane, o, 1.0f / L, m_ref + __log2f(L));
}

// A workgroup runs one item, or with bins (bf16 cache) the items of bin
// blockIdx.x in order (see Stage1Args).  Between two items every load and
// store of the first is complete and every wave is past it, so the next may
// reuse LDS.
template <int F, bool PAGED>
__global__ __launch_bounds__(kStage1Threads, F == kBf16 ? 1 : 2) void mla_stage1(Stage1Args a) {
  __shared__ __attribute__((aligned(16))) Stage1Buffers<F> tiles;
  __shared__ __attribute__((aligned(16))) Stage1Lds<F, PAGED> sh;
  int i = a.bins ? a.bins[blockIdx.x] : (int)blockIdx.x;
  const int i_end = a.bins ? a.bins[blockIdx.x + 1] : i + 1;
  while (i < i_end) {
    const WorkItem item = a.uniform_splits
                              ? uniform_item(xcd_block(blockIdx.x, gridDim.x), a.uniform_splits, a.uniform_chunk,
                                             a.uniform_len, a.uniform_base)
                              : a.items[i];
    stage1_item<F, PAGED>(a, item, tiles, sh);
    if (++i == i_end) break;
    wait_loads<0>();
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// mla_merge: LSE merge of the partials of one sequence,
//   M = max_s lse_s,  out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M)
// (727205 `mla_rd`; 700955 `reduce_lse_v71`; 599694 `_flash_fp8_split_s2`).
// One workgroup per (sequence, quarter of the columns): thread t merges
// float4 numbers t and t + 256 of that quarter of every partial (both of head
// t % 16, see kSlotFloat4), reading kMergeBatch partials at a time so that
// their loads are in flight together.  BF: the partials' O is bf16.
// ---------------------------------------------------------------------------
constexpr int kMergeBatch = 4;

// Float4 number e of the partial O at slot offset `slot` (in float4), fp32 or
// bf16 (four bf16 in place of each float4).
template <bool BF>
__device__ __forceinline__ f32x4 load_partial(const float* part_o, int64_t slot, int e) {
  if constexpr (BF) {
    const uint2 u = reinterpret_cast<const uint2*>(part_o)[slot + e];
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xFFFF0000u)};
  } else {
    return reinterpret_cast<const f32x4*>(part_o)[slot + e];
  }
}

template <bool BF>
__global__ __launch_bounds__(kMergeThreads) void mla_merge(MergeArgs a) {
  const int job = a.uniform_nslots > 0 ? xcd_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const MergeSeq seq = a.uniform_nslots > 0
                           ? MergeSeq{job >> 2, (job >> 2) * a.uniform_nslots, a.uniform_nslots, 0}
                           : a.work[job >> 2];
  const int quarter = job & 3;
  const int t = threadIdx.x;
  const int h = t & 15;
  const float* lse = a.part_lse + (int64_t)seq.slot_begin * kNumHeads + h;
  const int64_t po = (int64_t)seq.slot_begin * kSlotFloat4;
  const int e0 = 512 * quarter + t;
  float M = kNegInf;  // running maximum of the lse seen so far
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  for (int s0 = 0; s0 < seq.nslots; s0 += kMergeBatch) {
    float l[kMergeBatch];
    f32x4 x0[kMergeBatch], x1[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {  // all loads of the batch in flight together
      const int s = min(s0 + k, seq.nslots - 1);
      l[k] = lse[s * kNumHeads];
      x0[k] = load_partial<BF>(a.part_o, po + (int64_t)s * kSlotFloat4, e0);
      x1[k] = load_partial<BF>(a.part_o, po + (int64_t)s * kSlotFloat4, e0 + 256);
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      if (s0 + k < seq.nslots) mb = fmaxf(mb, l[k]);
    const float r = __builtin_amdgcn_exp2f(M - mb);  // 0 on the first batch
    acc0 *= r;
    acc1 *= r;
    W *= r;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float wk = (s0 + k < seq.nslots) ? __builtin_amdgcn_exp2f(l[k] - mb) : 0.f;
      W += wk;
      acc0 += wk * x0[k];
      acc1 += wk * x1[k];
    }
    M = mb;
  }
  const float inv = 1.0f / W;
  // float4 e (= t or t + 256) of this quarter: column tile v = e / 64,
  // lane e % 64, i.e. dims 128 quarter + 16 v + 4 ((e % 64) / 16)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int e = t + 256 * half;
    const int d = 128 * quarter + 16 * (e >> 6) + 4 * ((e & 63) >> 4);
    const f32x4 r = (half ? acc1 : acc0) * inv;
    *reinterpret_cast<uint2*>(a.out + ((int64_t)seq.batch * kNumHeads + h) * kVDim + d) =
        uint2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  }
}

// The same merge for a few sequences with many partials each: a job's 2048
// float4 of output are cut into P parts (8, 16 or 32), one workgroup each, so
// that a small batch still spreads its merge over many compute units.  The
// workgroup's 256 threads are S = P / 8 groups of 2048 / P threads; thread t
// of group q merges float4 e = (2048 / P) part + t over the partials q,
// q + S, q + 2S, .., and group 0 then merges the S results (running maximum,
// weight sum and accumulator) through LDS.
template <int P, bool BF>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_wide(MergeArgs a) {
  constexpr int kPart = 2048 / P;  // float4 per part
  constexpr int S = kMergeThreads / kPart;
  static_assert(kPart * S == kMergeThreads && S >= 1, "part split");
  __shared__ float sh_m[S][kPart], sh_w[S][kPart];
  __shared__ f32x4 sh_acc[S][kPart];
  // uniform plans: numbered like their stage-1 items (xcd_block), so that a
  // sequence's merge runs on the XCD whose L2 holds its partials
  const int idx = a.uniform_nslots > 0 ? xcd_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int job = idx / P, part = idx % P;
  const MergeSeq seq = a.uniform_nslots > 0 ? MergeSeq{job, job * a.uniform_nslots, a.uniform_nslots, 0}
                                            : a.work[job];
  const int t = threadIdx.x % kPart, grp = threadIdx.x / kPart;
  const int e = kPart * part + t;  // float4 of the slot; its head is e % 16
  const int h = e & 15;
  const float* lse = a.part_lse + (int64_t)seq.slot_begin * kNumHeads + h;
  const int64_t po = (int64_t)seq.slot_begin * kSlotFloat4;
  float M = kNegInf;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  for (int s0 = grp; s0 < seq.nslots; s0 += S * kMergeBatch) {
    float l[kMergeBatch];
    f32x4 x[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {  // all loads of the batch in flight together
      const int s = min(s0 + S * k, seq.nslots - 1);
      l[k] = lse[s * kNumHeads];
      x[k] = load_partial<BF>(a.part_o, po + (int64_t)s * kSlotFloat4, e);
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      if (s0 + S * k < seq.nslots) mb = fmaxf(mb, l[k]);
    const float r = __builtin_amdgcn_exp2f(M - mb);  // 0 on the first batch
    acc *= r;
    W *= r;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float wk = (s0 + S * k < seq.nslots) ? __builtin_amdgcn_exp2f(l[k] - mb) : 0.f;
      W += wk;
      acc += wk * x[k];
    }
    M = mb;
  }
  if constexpr (S > 1) {
    sh_m[grp][t] = M;
    sh_w[grp][t] = W;
    sh_acc[grp][t] = acc;
    __syncthreads();
    if (grp != 0) return;
    float Mall = M;
#pragma unroll
    for (int q = 1; q < S; ++q) Mall = fmaxf(Mall, sh_m[q][t]);
    const float r0 = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mall);
    acc *= r0;
    W *= r0;
#pragma unroll
    for (int q = 1; q < S; ++q) {
      const float mq = sh_m[q][t];
      const float rq = mq == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mq - Mall);
      W += rq * sh_w[q][t];
      acc += rq * sh_acc[q][t];
    }
  }
  const f32x4 res = acc * (1.0f / W);
  // float4 e: column tile v = (e % 512) / 64, lane group (e % 64) / 16 of the
  // 128-column quarter e / 512
  const int d = 128 * (e >> 9) + 16 * ((e & 511) >> 6) + 4 * ((e & 63) >> 4);
  *reinterpret_cast<uint2*>(a.out + ((int64_t)seq.batch * kNumHeads + h) * kVDim + d) =
      uint2{pack_bf16x2(res[0], res[1]), pack_bf16x2(res[2], res[3])};
}

template <int F, bool P>
const void* stage1_fn() {
  if constexpr (F == kFp8)
    return stage1_fp8_kernel(P, false);
  else if constexpr (F == kMxfp4)
    return stage1_mxfp4_kernel(P);
  else
    return reinterpret_cast<const void*>(&mla_stage1<F, P>);
}

const void* pick_stage1(int fmt, bool paged) {
  switch (fmt) {
    case kBf16: return paged ? stage1_fn<kBf16, true>() : stage1_fn<kBf16, false>();
    case kFp8: return paged ? stage1_fn<kFp8, true>() : stage1_fn<kFp8, false>();
    case kMxfp4: return paged ? stage1_fn<kMxfp4, true>() : stage1_fn<kMxfp4, false>();
    default: return nullptr;
  }
}

}  // namespace

// Scratch of the allocation-free run: every run on a GPU shares that GPU's
// copy (runs that overlap on one GPU race), and it keeps the last run's
// partials, which no run reads before writing them.  In host code `scratch`
// names a host-side stand-in, never the device memory: kernels get the
// address that hipGetSymbolAddress returns for the device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_address(int device, void** ptr) {
  static std::mutex mu;
  static std::vector<void*> addr;  // per device ordinal
  int cur = -1;
  if (device < 0 || hipGetDevice(&cur) != hipSuccess || cur != device) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<size_t>(device) >= addr.size()) addr.resize(static_cast<size_t>(device) + 1, nullptr);
  if (!addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

// With events, the launch records them at the start and the end of the
// kernel itself (hipExtLaunchKernel), so their difference is its duration.
static hipError_t launch(const void* fn, dim3 grid, dim3 block, void** params, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  if (start && stop) return hipExtLaunchKernel(fn, grid, block, params, 0, s, start, stop, 0);
  return hipLaunchKernel(fn, grid, block, params, 0, s);
}

bool stage1_dedicated(int fmt, const Stage1Args& a) {
  if (fmt == kFp8 || fmt == kBf16) return true;
  if (fmt == kMxfp4) return ((a.scale_stride | (int64_t)(uintptr_t)a.kv_mx_scales) & 1) == 0;
  return false;
}

hipError_t launch_stage1(int fmt, bool paged, bool row_pairs, const Stage1Args& a, int num_items, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  const void* fn = fmt == kFp8     ? stage1_fp8_kernel(paged, row_pairs, a.query_e4m3 != 0)
                   : fmt == kMxfp4 ? stage1_mxfp4_kernel(paged, a.query_e4m3 != 0)
                                   : pick_stage1(fmt, paged);
  if (fmt == kMxfp4 && !stage1_dedicated(fmt, a)) {  // two-byte scale loads need even addresses
    if (a.query_e4m3) return hipErrorNotSupported;
    fn = paged ? reinterpret_cast<const void*>(&mla_stage1<kMxfp4, true>)
               : reinterpret_cast<const void*>(&mla_stage1<kMxfp4, false>);
  }
  if (!fn) return hipErrorInvalidValue;
  const int threads = (fmt == kMxfp4 && stage1_dedicated(fmt, a)) ? kStage1ThreadsMxfp4 : kStage1Threads;
  Stage1Args args = a;
  void* params[] = {&args};
  return launch(fn, dim3(num_items), dim3(threads), params, s, start, stop);
}

int merge_parts(int num_merge_seqs) {
  // 4 parts down to 64 jobs, then up to 32 parts for the smallest batches
  // (32 sequences of 8 partials: 8 parts 31.9-32.2 us a call, 4 parts 32.4-32.5)
  if (num_merge_seqs >= 64) return 4;
  if (num_merge_seqs >= 16) return 8;
  if (num_merge_seqs >= 8) return 16;
  return 32;
}

hipError_t launch_merge(const MergeArgs& a, int num_merge_seqs, hipStream_t s, hipEvent_t start,
                        hipEvent_t stop) {
  MergeArgs args = a;
  void* params[] = {&args};
  const int parts = merge_parts(num_merge_seqs);
  const void* fn =
      a.part_bf16 ? (parts == 4    ? reinterpret_cast<const void*>(&mla_merge<true>)
                     : parts == 8  ? reinterpret_cast<const void*>(&mla_merge_wide<8, true>)
                     : parts == 16 ? reinterpret_cast<const void*>(&mla_merge_wide<16, true>)
                                   : reinterpret_cast<const void*>(&mla_merge_wide<32, true>))
                  : (parts == 4    ? reinterpret_cast<const void*>(&mla_merge<false>)
                     : parts == 8  ? reinterpret_cast<const void*>(&mla_merge_wide<8, false>)
                     : parts == 16 ? reinterpret_cast<const void*>(&mla_merge_wide<16, false>)
                                   : reinterpret_cast<const void*>(&mla_merge_wide<32, false>));
  return launch(fn, dim3(num_merge_seqs * parts), dim3(kMergeThreads), params, s, start, stop);
}

hipError_t kernel_attributes(int fmt, bool paged, bool row_pairs, bool query_e4m3, int which,
                             hipFuncAttributes* attr) {
  const void* fn = which != 0        ? reinterpret_cast<const void*>(&mla_merge<true>)
                   : fmt == kFp8     ? stage1_fp8_kernel(paged, row_pairs, query_e4m3)
                   : fmt == kMxfp4   ? stage1_mxfp4_kernel(paged, query_e4m3)
                                     : pick_stage1(fmt, paged);
  if (!fn) return hipErrorInvalidValue;
  return hipFuncGetAttributes(attr, fn);
}

hipError_t stage1_occupancy(int fmt, bool paged, int* blocks_per_cu) {
  const void* fn = pick_stage1(fmt, paged);
  if (!fn) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn,
                                                      fmt == kMxfp4 ? kStage1ThreadsMxfp4 : kStage1Threads, 0);
}

}  // namespace mla
