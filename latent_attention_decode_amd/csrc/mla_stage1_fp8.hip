// gfx950 split kernel for an fp8-e4m3 cache (per-tensor scale): single-token
// multi-head latent attention decode, one 256-thread workgroup per planned
// work item (a token range of one sequence), 128-token tiles streamed
// HBM -> LDS by cache-to-LDS loads, both contractions on the fp8 / MX matrix
// instructions straight on the cached codes.  A workgroup whose item is the
// whole sequence writes the bf16 output; otherwise it writes a normalised
// partial and its log-sum-exp, and for plans that ask for it the item of a
// sequence that finishes last merges that sequence's partials.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

// ---------------------------------------------------------------------------
// stage 1, fp8 cache: cooperative 128-token tiles streamed into LDS
// ---------------------------------------------------------------------------
// Both contractions run straight on the cached e4m3 codes (nothing is
// decoded), on the gfx950 MX matrix instruction v_mfma_scale_f32_16x16x128_
// f8f6f4 (fp8 x fp8; unit block scales for the scores), which takes 128
// k-values per step,
// and on v_mfma_f32_16x16x32_fp8_fp8 for the 64 rope columns.  The other
// operand is written as a sum of two e4m3 numbers, hi + lo, and each product
// is taken twice:
//   * the query row of head h is first scaled by 2^s_h (max |q| in [128, 256))
//     and split q = hi + lo with hi = e4m3(q) and lo = e4m3(q - hi).  A bf16
//     value has 8 significant bits and hi keeps the leading 4, so the rest fits
//     lo exactly whenever it is a normal e4m3 number (|scaled q| >= 1/4, i.e.
//     every element above 1/1024 of the row maximum; smaller ones are off by at
//     most 2^-10 in scaled units).  2^-s_h is folded into the score scale.
//   * the softmax weights are split the same way, each 32-token k-block of the
//     P.V step relative to its own maximum, which returns as the block's B
//     scale (see weight_block_scale): about 8 significant bits per weight, as
//     a bf16 weight has, and no weight lost to the range of e4m3 however far
//     the logits of different blocks lie apart.
//
// Data movement: every byte of the item's cache rows goes HBM -> LDS by
// cache-to-LDS loads (global_load_lds_dwordx4), in a ring of two 128-token
// tiles, so one tile is in flight while the other is computed; the query
// comes the same way.  A tile is its 128 rows at pitch 576 with no padding,
// 72 loads of 1 KB each (wave w issues loads 18w..18w+17).  One load writes
// 64 consecutive 16-byte LDS slots, lane l to slot l, and each lane fetches
// the chunk that belongs there; inside each aligned group of four chunks of a
// row the chunks are stored XOR-permuted by chunk_swz(row), which spreads
// the LDS reads below over the banks while each load still covers whole
// 64-byte runs of the rows (measured: the transposing V reads run without
// bank conflicts; the 16-byte score, rope and P reads still see some, about
// a third of the LDS's active cycles, and the LDS is active for a seventh of
// the kernel's).
//
// Per tile, with wave w:
//   1. S^T[token, head] = K (Qhi + Qlo)^T for the 32 tokens of k-block w of
//      the P.V step (two 16-token row blocks, tokens blk_base(w) + 32s +
//      0..15), all 576 columns; the query stays in registers;
//   2. softmax in the log2 domain; each wave writes the e4m3 hi/lo weights
//      of its block, relative to the block's maximum, to P^T in LDS.  The
//      running maximum is shared by the four waves and lazy: it moves (to an
//      integer, and O and the sums are rescaled by a power of two) only when
//      a tile maximum passes it by more than 8;
//   3. O^T[dim, head] += V^T (Phi + Plo)^T for dims 128w..128w+127 over all
//      128 tokens, one MX step per 16 columns; V^T comes from the tile through
//      the transposing LDS read ds_read_b64_tr_b8.
// Because the maximum is shared, the waves' outputs need no merge: each wave
// writes its own 128 columns.
constexpr int kCTile = 128;                         // tokens per tile
constexpr int kCTileBytes = kCTile * kQkDim;        // 73728
constexpr int kCRing = 2;                           // tiles in the LDS ring
constexpr int kCLoads = kCTileBytes / 1024;         // 72 loads per tile
constexpr int kCLoadsPerWave = kCLoads / kWaves;    // 18
constexpr int kQBytes = kNumHeads * kQkDim * 2;     // bf16 query of one sequence
constexpr int kQLoads = kQBytes / 1024;             // 18
constexpr int kPRow = kCTile + 16;                  // bytes per head row of P^T
static_assert(kCLoads == kWaves * kCLoadsPerWave && kQLoads * 1024 == kQBytes, "load split");
static_assert(2 * kQBytes <= kCTileBytes, "the query and its e4m3 words fit a ring slot");
static_assert(kQBytes <= kCTileBytes, "the query is staged in the last ring slot");

// Position of 16-byte chunk c of tile row r inside the row: c ^ chunk_swz(r),
// a permutation inside each aligned group of four chunks.  The LDS has 64
// banks of 4 bytes; with rows at pitch 576, the reads below touch, per phase,
// 16 rows r0..r0+15 of one chunk (score reads, 16 B per lane) or rows
// {32g + 8q + e : e < 8} of two neighbouring g (transposing V reads, 8 B per
// lane).  In a model of 64 four-byte banks this permutation puts each such
// phase on distinct banks.
__host__ __device__ constexpr int chunk_swz(int r) {
  return ((r >> 2) & 1) | ((((r >> 3) ^ (r >> 5)) & 1) << 1);
}
__host__ __device__ constexpr int tile_slot(int r, int c) { return r * 36 + (c ^ chunk_swz(r)); }
// Position of 16-byte chunk c (0..71) of query head h.
__host__ __device__ constexpr int q_slot(int h, int c) { return h * 72 + (c ^ (h & 7)); }

// Every slot of a tile holds exactly one chunk of one row, and vice versa.
constexpr bool tile_slots_are_a_permutation() {
  bool seen[kCLoads * 64] = {};
  for (int r = 0; r < kCTile; ++r)
    for (int c = 0; c < 36; ++c) {
      const int s = tile_slot(r, c);
      if (s / 36 != r || seen[s]) return false;
      seen[s] = true;
    }
  return true;
}
constexpr bool q_slots_are_a_permutation() {
  bool seen[kQLoads * 64] = {};
  for (int h = 0; h < kNumHeads; ++h)
    for (int c = 0; c < 72; ++c) {
      const int s = q_slot(h, c);
      if (s / 72 != h || seen[s]) return false;
      seen[s] = true;
    }
  return true;
}
static_assert(tile_slots_are_a_permutation() && q_slots_are_a_permutation(), "slot maps");

// Tokens of k-block j of a 128-token P.V step: blk_base(j) + 0..15 and
// blk_base(j) + 32..47.  P^T and V^T give lane group g the tile tokens
// 32g..32g+31 in its operand bytes 0..31, and the MX instruction's fp8 operand
// holds k-values 16g + b in bytes b < 16 and 64 + 16g + b - 16 in bytes
// 16..31; a block scale covers k-values 32j..32j+31.  Wave w scores the
// tokens of k-block w, so the block's maximum is the wave's own.
__host__ __device__ constexpr int blk_base(int j) { return 64 * (j & 1) + 16 * (j >> 1); }
constexpr bool blocks_match_operand_layout() {
  for (int tok = 0; tok < kCTile; ++tok) {
    const int g = tok / 32, b = tok % 32;
    const int k = b < 16 ? 16 * g + b : 64 + 16 * g + (b - 16);
    const int j = k / 32;
    const int d = tok - blk_base(j);
    if (!((d >= 0 && d < 16) || (d >= 32 && d < 48))) return false;
  }
  return true;
}
static_assert(blocks_match_operand_layout(), "k-blocks of the P.V step");

// LDS of the kernel for groups of up to NR query rows of one sequence (NR
// = 2 pairs two query tokens of a multi-token plan; it then stages fewer
// page ids per item to make room for the second row's P and maxima).
template <int NR>
struct Fp8Lds {
  static constexpr int kPages = NR == 1 ? kItemPagesFp8 : kItemPagesFp8Pair;
  uint8_t tile[kCRing][kCTileBytes];       // the ring; slot 1 first holds the query rows
  uint8_t p[NR][2][kNumHeads][kPRow];      // per row: P^T hi / lo as [head][token]
  float red_m[NR][kNumHeads][kWaves];      // per row: per-wave tile maxima
  float red_l[kNumHeads][kWaves];          // per-wave sums, at the end
  int32_t pages[kPages];                   // paged: page ids of the item
};
static_assert(sizeof(Fp8Lds<2>) <= 160 * 1024, "LDS of the paired kernel");
static_assert(2 * 2 * kQBytes <= kCTileBytes, "two query rows and their e4m3 words fit a ring slot");

// One group of NR work items: NR consecutive query rows of one sequence over
// the same tokens from tok_begin (NR = 1: any work item).  Row r stops at its
// own tok_end; the cache tiles are loaded once for all rows, and the score and
// value contractions share each operand read from them.  Q1: the query enters
// the scores as one e4m3 code per element (hi alone), not as hi + lo.
template <bool PAGED, int NR, bool Q1, int NRL>
__device__ __forceinline__ void fp8_item(const Stage1Args& a, const WorkItem* items, Fp8Lds<NRL>& sh) {
  constexpr int kMaxItemPages = Fp8Lds<NRL>::kPages;
  const WorkItem& item = items[0];  // the rows share kv_base and tok_begin
  const int tid = threadIdx.x;
  if (NR == 1 && item.slot == WorkItem::kEmpty) {  // empty sequence: its output is zero
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
  int tok_last_r[NR];         // last token of each row
  int tok_end = item.tok_end;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    tok_last_r[r] = items[r].tok_end - 1;
    tok_end = max(tok_end, items[r].tok_end);
  }
  const int tok_last = tok_end - 1;
  const int ntiles = (tok_end - item.tok_begin + kCTile - 1) / kCTile;
  const float kv_scale = *a.kv_scale;

  // The query rows first (they need only the row ids): 18 loads per row into
  // ring slot 1, row r at r * 18 KB, load k by wave k % 4.
  {
    const uint32_t qm0 = lds_u32(&sh.tile[kCRing - 1][0]);
    for (int k = wave; k < kQLoads * NR; k += kWaves) {
      const int r = k / kQLoads, kk = k - kQLoads * r;
      const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (int64_t)items[r].batch * kNumHeads * kQkDim);
      const int s = 64 * kk + lane;
      const int h = s / 72;
      const int c = (s - 72 * h) ^ (h & 7);
      dma_one(qsrc + (h * 72 + c) * 16, qm0 + r * kQBytes + 1024 * kk);
    }
  }
  const int64_t seq_base = item.kv_base;  // kv_indptr[b]: first row, or first page slot

  int page0 = 0;
  if constexpr (PAGED) {
    page0 = item.tok_begin >> a.page_shift;
    const int npages = min(((tok_end - 1) >> a.page_shift) - page0 + 1, kMaxItemPages);
    // the item's page ids into LDS by four-byte cache-to-LDS loads, all in
    // flight together (lanes past the last page repeat it)
    const int32_t* psrc = a.page_indices + seq_base + page0;
    const uint32_t pm0 = lds_u32(&sh.pages[0]);
    for (int j = wave; 64 * j < npages; j += kWaves)
      dma_u32(psrc + min(64 * j + lane, npages - 1), pm0 + 256 * j);
  }
  // The query (and the page ids) land before tile 0 is issued: issued
  // together with the first tile of every CU, the query rows would queue
  // behind those 19 MB at the memory and land last.
  wait_loads<0>();
  lds_barrier();

  // This lane's slot in each of its wave's 18 loads of a tile: (tile row << 8)
  // | chunk.  Load j = 4q + e of a group goes to LDS m0_q + 1024 e.
  uint32_t rc[kCLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kCLoadsPerWave; ++j) {
    const int s = 64 * (kCLoadsPerWave * wave + j) + lane;
    const int r = s / 36;
    const int c = (s - 36 * r) ^ chunk_swz(r);
    rc[j] = (uint32_t)(r << 8 | c);
  }
  const uint32_t ring0 = lds_u32(&sh.tile[0][0]) + 1024 * kCLoadsPerWave * wave;

  // Issue part `part` of this wave's 18 loads of tile t into ring slot t % 2:
  // loads 4 part .. 4 part + 3 (part 0..3), loads 16 and 17 (part 4), or all
  // of them (part -1).  Rows past the group's last token fetch that token's
  // row (finite data, masked later).
  auto issue = [&](int t, int part) {
    const int tok0 = item.tok_begin + t * kCTile;
    const int lim = tok_last - tok0;  // last valid tile row
    const uint32_t m0 = ring0 + (uint32_t)((t & (kCRing - 1)) * kCTileBytes);
    if constexpr (!PAGED) {
      // base 3072 bytes before the tile, so that no per-lane offset (which
      // excludes the instruction offset of up to 3072) is negative
      const uint8_t* base = uniform_ptr(a.kv + (seq_base + tok0) * kQkDim - 3072);
      uint32_t off[kCLoadsPerWave];
#pragma unroll
      for (int j = 0; j < kCLoadsPerWave; ++j) {
        const uint32_t r = min((int)(rc[j] >> 8), lim);
        off[j] = r * kQkDim + 16 * (rc[j] & 0xFF) + 3072 - 1024 * (j & 3);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (part < 0 || part == q) dma_group<4>(base, off + 4 * q, m0 + 4096 * q);
      if (part < 0 || part == 4) dma_group<2>(base, off + 16, m0 + 4096 * 4);
    } else {
      const int pmask = (1 << a.page_shift) - 1;
      const uint8_t* src[kCLoadsPerWave];
#pragma unroll
      for (int j = 0; j < kCLoadsPerWave; ++j) {
        const int tok = tok0 + min((int)(rc[j] >> 8), lim);
        const uint32_t page = (uint32_t)sh.pages[(tok >> a.page_shift) - page0];
        const int64_t row = (int64_t)((page << a.page_shift) + (uint32_t)(tok & pmask));
        src[j] = a.kv + row * kQkDim + 16 * (rc[j] & 0xFF) - 1024 * (j & 3);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (part < 0 || part == q) dma_group<4>(src + 4 * q, m0 + 4096 * q);
      if (part < 0 || part == 4) dma_group<2>(src + 16, m0 + 4096 * 4);
    }
  };

  issue(0, -1);

  // Query rows, B operands of S^T = K Q^T, scaled by 2^s and split into
  // e4m3 hi + lo: for 128-column block K (0..3) lane (head r16, group g)
  // holds q[head][128K + 32g .. +32]; for the rope columns, k-step h (0, 1),
  // q[head][512 + 16g + 8h .. +8].  Every wave needs all of it; wave w
  // converts block K = w (and waves 0, 1 rope step h = w) of every row, and
  // the waves trade their head maxima and then the converted words through
  // LDS, in the query's ring slot behind the bf16 rows.
  fp8x32 qh[NR][4], ql[NR][4];
  fp8x8 rh[NR][2], rl[NR][2];
  float xscale[NR];
  {
    const bool rope = wave < 2;
    bf16x8 qv[NR][5];  // [r][i]: chunk 16 wave + 4g + i; [r][4]: rope chunk 64 + 2g + wave
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint8_t* qlds = &sh.tile[kCRing - 1][r * kQBytes];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qv[r][i] = *reinterpret_cast<const bf16x8*>(qlds + 16 * q_slot(r16, 16 * wave + 4 * g + i));
      qv[r][4] = rope ? *reinterpret_cast<const bf16x8*>(qlds + 16 * q_slot(r16, 64 + 2 * g + wave)) : bf16x8{};
      float am[5];
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        float m0 = fmaxf(fabsf((float)qv[r][k][0]), fabsf((float)qv[r][k][1]));
        float m1 = fmaxf(fabsf((float)qv[r][k][2]), fabsf((float)qv[r][k][3]));
        float m2 = fmaxf(fabsf((float)qv[r][k][4]), fabsf((float)qv[r][k][5]));
        float m3 = fmaxf(fabsf((float)qv[r][k][6]), fabsf((float)qv[r][k][7]));
        am[k] = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
      }
      const float amax = xor_max_groups(fmaxf(fmaxf(fmaxf(am[0], am[1]), fmaxf(am[2], am[3])), am[4]));
      if (g == 0) sh.red_m[r][r16][wave] = amax;
    }
    lds_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      uint32_t* const qcv = reinterpret_cast<uint32_t*>(&sh.tile[kCRing - 1][(NR + r) * kQBytes]);
      const f32x4 wm = *reinterpret_cast<const f32x4*>(&sh.red_m[r][r16][0]);
      const float amax = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
      // 2^s with amax * 2^s in [128, 256)
      const int s = (amax > 0.f) ? 8 - __builtin_amdgcn_frexp_expf(amax) : 0;
      xscale[r] = a.score_scale * kv_scale * __builtin_ldexpf(1.0f, -s);
      uint32_t hw[10], lw[10];  // word 2k + m: elements 4m..4m+3 of qv[r][k]
#pragma unroll
      for (int k = 0; k < 5; ++k)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          split_fp8x4(__builtin_ldexpf((float)qv[r][k][4 * m], s), __builtin_ldexpf((float)qv[r][k][4 * m + 1], s),
                      __builtin_ldexpf((float)qv[r][k][4 * m + 2], s),
                      __builtin_ldexpf((float)qv[r][k][4 * m + 3], s), hw[2 * k + m], lw[2 * k + m]);
      u32x4* const kh = reinterpret_cast<u32x4*>(qcv + ((2 * wave) * 64 + lane) * 8);
      u32x4* const kl = reinterpret_cast<u32x4*>(qcv + ((2 * wave + 1) * 64 + lane) * 8);
      kh[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
      kh[1] = u32x4{hw[4], hw[5], hw[6], hw[7]};
      if constexpr (!Q1) {
        kl[0] = u32x4{lw[0], lw[1], lw[2], lw[3]};
        kl[1] = u32x4{lw[4], lw[5], lw[6], lw[7]};
      }
      if (rope) {
        *reinterpret_cast<uint2*>(qcv + 4096 + ((2 * wave) * 64 + lane) * 2) = uint2{hw[8], hw[9]};
        if constexpr (!Q1) *reinterpret_cast<uint2*>(qcv + 4096 + ((2 * wave + 1) * 64 + lane) * 2) = uint2{lw[8], lw[9]};
      }
    }
    lds_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t* const qcv = reinterpret_cast<const uint32_t*>(&sh.tile[kCRing - 1][(NR + r) * kQBytes]);
#pragma unroll
      for (int K = 0; K < 4; ++K) {
        const u32x4* h = reinterpret_cast<const u32x4*>(qcv + ((2 * K) * 64 + lane) * 8);
        const u32x4* l = reinterpret_cast<const u32x4*>(qcv + ((2 * K + 1) * 64 + lane) * 8);
        qh[r][K] = join16(h[0], h[1]);
        if constexpr (!Q1) ql[r][K] = join16(l[0], l[1]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint2 wh = *reinterpret_cast<const uint2*>(qcv + 4096 + ((2 * h) * 64 + lane) * 2);
        rh[r][h] = pack_fp8x8(wh.x, wh.y);
        if constexpr (!Q1) {
          const uint2 wl = *reinterpret_cast<const uint2*>(qcv + 4096 + ((2 * h + 1) * 64 + lane) * 2);
          rl[r][h] = pack_fp8x8(wl.x, wl.y);
        }
      }
    }
  }

  f32x4 o[NR][8];     // O^T[dim 128w + 16v + 4g + i][head r16] of each row
  float m_ref[NR];    // shared running maximum (log2 units) of head r16
  float l_part[NR];   // this lane's share of the running sum
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int v = 0; v < 8; ++v) o[r][v] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[r] = kNegInf;
    l_part[r] = 0.f;
  }

  // LDS byte offsets of this lane's reads within a tile.  Score rows
  // blk_base(w) + 32s + r16 (s = 0, 1); value rows 32g + 8q + (r16 >> 1) have
  // chunk_swz(32g + 8(q & 1) + (r16 >> 1)).
  const int base = blk_base(wave);
  int k_off0[2], k_off1[2], k_offr[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int row = base + 32 * s + r16;
    const int ksw = chunk_swz(row);
    k_off0[s] = row * kQkDim + 16 * ((2 * g) ^ ksw);      // chunk 8K + 2g
    k_off1[s] = row * kQkDim + 16 * ((2 * g + 1) ^ ksw);  // chunk 8K + 2g + 1
    k_offr[s] = row * kQkDim + 16 * (32 + (g ^ ksw));     // chunk 32 + g
  }
  int v_off[2][4];  // [q % 2][v % 4]; + 64 (v / 4) + 4608 (q & ~1); column chunk 8w + v
#pragma unroll
  for (int qp = 0; qp < 2; ++qp) {
    const int vrow = 32 * g + 8 * qp + (r16 >> 1);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      v_off[qp][c4] = vrow * kQkDim + 16 * (8 * wave + (c4 ^ chunk_swz(vrow))) + 8 * (r16 & 1);
  }

  // Tile 1 goes into the query's slot as soon as every wave has its query in
  // registers, so that the first two tiles stream in together.
  if (ntiles > 1) {
    lds_barrier();
    issue(1, -1);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int tok0 = item.tok_begin + t * kCTile;
    if (t == 0 && ntiles > 1)
      wait_loads<kCLoadsPerWave>();  // tile 0, not tile 1 behind it
    else
      wait_loads<0>();  // this wave's part of tile t
    lds_barrier();      // all of tile t; everyone is past tile t-1 (and the query)
    // From tile 1 on, tile t+1 goes into the other slot in five parts spread
    // over this tile's work, so that the loads queue while the matrix cores run.
    const bool more = t > 0 && t + 1 < ntiles;
    if (more) issue(t + 1, 0);
    const uint8_t* cur = &sh.tile[t & (kCRing - 1)][0];

    // ---- scores of tokens base + 32s + (0..15), s = 0, 1 ----
    f32x4 sacc[NR][2][2];  // [row][s][hi/lo]
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c) sacc[r][s][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = 0; K < 4; ++K) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const fp8x32 ka = join16(*reinterpret_cast<const u32x4*>(cur + k_off0[s] + 128 * K),
                                 *reinterpret_cast<const u32x4*>(cur + k_off1[s] + 128 * K));
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          sacc[r][s][0] = mfma_fp8_k128(ka, qh[r][K], sacc[r][s][0]);
          if constexpr (!Q1) sacc[r][s][1] = mfma_fp8_k128(ka, ql[r][K], sacc[r][s][1]);
        }
      }
      if (more && (K == 1 || K == 3)) issue(t + 1, K == 1 ? 1 : 2);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(cur + k_offr[s]);
      const fp8x8 ka = pack_fp8x8(w[0], w[1]);
      const fp8x8 kb = pack_fp8x8(w[2], w[3]);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        sacc[r][s][0] = mfma_fp8(ka, rh[r][0], sacc[r][s][0]);
        if constexpr (Q1) {
          // the second rope step on the idle accumulator: no two of these
          // steps chained back to back on one accumulator
          sacc[r][s][1] = mfma_fp8(kb, rh[r][1], sacc[r][s][1]);
        } else {
          sacc[r][s][1] = mfma_fp8(ka, rl[r][0], sacc[r][s][1]);
          sacc[r][s][0] = mfma_fp8(kb, rh[r][1], sacc[r][s][0]);
          sacc[r][s][1] = mfma_fp8(kb, rl[r][1], sacc[r][s][1]);
        }
      }
    }

    // ---- softmax: x[s][i] is token base + 32s + 4g + i of head r16 ----
    // The wave's tokens are k-block w of the P.V step: their weights are
    // written relative to the block's own maximum (weight_block_scale).
    float psum[NR];  // this lane's weights as written, in units of 2^(F - 7 - m_ref)
    float fblk[NR];  // F = floor of the wave's block maximum (0 if all masked)
    bool live[NR];   // the block has a valid token
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float x[2][4];
      float tmax = kNegInf;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[s][i] = (sacc[r][s][0][i] + sacc[r][s][1][i]) * xscale[r];
          if (tok0 + base + 32 * s + 4 * g + i > tok_last_r[r]) x[s][i] = kNegInf;
          tmax = fmaxf(tmax, x[s][i]);
        }
      tmax = xor_max_groups(tmax);
      if (g == 0) sh.red_m[r][r16][wave] = tmax;
      live[r] = tmax != kNegInf;
      fblk[r] = weight_block_floor(tmax);
      const float shift = 7.0f - fblk[r];  // x + shift < 8
      uint8_t* const p_hi = &sh.p[r][0][r16][0];
      uint8_t* const p_lo = &sh.p[r][1][r16][0];
      float ps = 0.f;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float p[4];
        uint32_t ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[s][i] + shift);
        split_fp8x4(p[0], p[1], p[2], p[3], ph, pl);
        *reinterpret_cast<uint32_t*>(p_hi + base + 32 * s + 4 * g) = ph;
        *reinterpret_cast<uint32_t*>(p_lo + base + 32 * s + 4 * g) = pl;
        ps += (p[0] + p[1]) + (p[2] + p[3]);
      }
      psum[r] = ps;
    }
    if (more) issue(t + 1, 3);
    lds_barrier();  // P^T and the block maxima of all waves

    fp8x32 bh[NR], bl[NR];
    int sb[NR];  // B block scale of k-block g (wave g's tokens) for head r16
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const f32x4 maxima = *reinterpret_cast<const f32x4*>(&sh.red_m[r][r16][0]);
      const uint8_t* const p_hi = &sh.p[r][0][r16][0];
      const uint8_t* const p_lo = &sh.p[r][1][r16][0];
      bh[r] = join16(*reinterpret_cast<const u32x4*>(p_hi + 32 * g),
                     *reinterpret_cast<const u32x4*>(p_hi + 32 * g + 16));
      bl[r] = join16(*reinterpret_cast<const u32x4*>(p_lo + 32 * g),
                     *reinterpret_cast<const u32x4*>(p_lo + 32 * g + 16));
      const float tile_max = fmaxf(fmaxf(maxima[0], maxima[1]), fmaxf(maxima[2], maxima[3]));
      // Every wave reads the same maxima, so this branch is uniform.
      if (__ballot(tile_max > m_ref[r] + kLazyRescale) != 0) {
        const float m_new = floorf(fmaxf(m_ref[r], tile_max));
        const float alpha = (m_ref[r] == kNegInf) ? 0.0f : __builtin_ldexpf(1.0f, (int)(m_ref[r] - m_new));
#pragma unroll
        for (int v = 0; v < 8; ++v) o[r][v] *= alpha;
        l_part[r] *= alpha;
        m_ref[r] = m_new;
      }
      if (live[r]) l_part[r] += __builtin_ldexpf(psum[r], (int)fblk[r] - 7 - (int)m_ref[r]);
      const float bm = g == 0 ? maxima[0] : g == 1 ? maxima[1] : g == 2 ? maxima[2] : maxima[3];
      sb[r] = weight_block_scale(bm, m_ref[r]);
    }

    // ---- O^T += V^T P^T over the 128 tokens, two column tiles at a time ----
#pragma unroll
    for (int v = 0; v < 8; v += 2) {
      fp8x32 va[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2*)(cur + v_off[q & 1][(v + u) & 3] + 64 * ((v + u) >> 2) +
                           8 * kQkDim * (q & ~1)));
          va[u][2 * q] = raw[0];
          va[u][2 * q + 1] = raw[1];
        }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        o[r][v] = mfma_fp8_k128_sb(va[0], bh[r], o[r][v], sb[r]);
        o[r][v + 1] = mfma_fp8_k128_sb(va[1], bh[r], o[r][v + 1], sb[r]);
        o[r][v] = mfma_fp8_k128_sb(va[0], bl[r], o[r][v], sb[r]);
        o[r][v + 1] = mfma_fp8_k128_sb(va[1], bl[r], o[r][v + 1], sb[r]);
      }
      if (more && v == 2) issue(t + 1, 4);
    }
  }

  // ---- sums over each row; each wave writes its 128 columns ----
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r > 0) lds_barrier();  // everyone has read the previous row's sums
    const float l_w = xor_sum_groups(l_part[r]);
    if (g == 0) sh.red_l[r16][wave] = l_w;
    lds_barrier();
    const f32x4 ls = *reinterpret_cast<const f32x4*>(&sh.red_l[r16][0]);
    const float L = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    const float f = kv_scale / L;
    finish_item<8>(a, items[r], tid, wave, 0, lane, o[r], f, m_ref[r] + __log2f(L));
  }
}

// A workgroup runs one item, or with bins the items of bin blockIdx.x in
// order (see Stage1Args).  Between two items every load and store of the
// first is complete and every wave is past it, so the next may reuse LDS.
// MAXROWS = 2 (multi-token plans): two items next to each other in a bin
// that are consecutive query rows of one sequence over the same tokens run
// together.
template <bool PAGED, int MAXROWS, bool Q1>
__global__ __launch_bounds__(kStage1Threads, 1) void mla_stage1_fp8(Stage1Args a) {
  __shared__ __attribute__((aligned(16))) Fp8Lds<MAXROWS> sh;
  int i = a.bins ? a.bins[blockIdx.x] : (int)blockIdx.x;
  const int i_end = a.bins ? a.bins[blockIdx.x + 1] : i + 1;
  while (i < i_end) {
    if constexpr (MAXROWS == 2) {
      if (i + 1 < i_end) {
        WorkItem pair[2] = {a.items[i], a.items[i + 1]};
        if (pair[0].slot != WorkItem::kEmpty && pair[1].slot != WorkItem::kEmpty &&
            pair[1].batch == pair[0].batch + 1 && pair[1].kv_base == pair[0].kv_base &&
            pair[1].tok_begin == pair[0].tok_begin) {
          fp8_item<PAGED, 2, Q1>(a, pair, sh);
          i += 2;
          if (i == i_end) break;
          wait_loads<0>();
          lds_barrier();
          continue;
        }
      }
    }
    const WorkItem item = a.uniform_splits
                              ? uniform_item(xcd_block(blockIdx.x, gridDim.x), a.uniform_splits, a.uniform_chunk,
                                             a.uniform_len, a.uniform_base)
                              : a.items[i];
    fp8_item<PAGED, 1, Q1>(a, &item, sh);
    if (++i == i_end) break;
    wait_loads<0>();
    lds_barrier();
  }
}

}  // namespace

template <bool Q1>
const void* fp8_kernel(bool paged, bool row_pairs) {
  if (row_pairs)
    return paged ? reinterpret_cast<const void*>(&mla_stage1_fp8<true, 2, Q1>)
                 : reinterpret_cast<const void*>(&mla_stage1_fp8<false, 2, Q1>);
  return paged ? reinterpret_cast<const void*>(&mla_stage1_fp8<true, 1, Q1>)
               : reinterpret_cast<const void*>(&mla_stage1_fp8<false, 1, Q1>);
}

const void* stage1_fp8_kernel(bool paged, bool row_pairs, bool query_e4m3) {
  return query_e4m3 ? fp8_kernel<true>(paged, row_pairs) : fp8_kernel<false>(paged, row_pairs);
}

}  // namespace mla
