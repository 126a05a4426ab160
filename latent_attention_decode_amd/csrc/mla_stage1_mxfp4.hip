// gfx950 split kernel for an MXFP4 cache (e2m1 codes, one e8m0 scale per 32
// columns of a row): single-token multi-head latent attention decode, one
// 512-thread workgroup (eight waves, two per SIMD) per planned work item,
// 128-token tiles streamed HBM -> LDS by cache-to-LDS loads, both
// contractions on the MX matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4.
// Wave w scores tokens 16w..16w+15 and accumulates output columns
// 64w..64w+63; the second wave on each SIMD hides the latencies of the first
// (the V conversion below makes this kernel heavier in vector and LDS work
// than the fp8 one, and its tiles are half the bytes).
//
// Operand layout of that instruction on gfx950 (measured): in each group g of
// 16 lanes, an fp4 operand holds 32 consecutive k-values 32g..32g+31, an fp8
// operand holds k = 16g + b in its bytes b < 16 and k = 64 + 16g + (b - 16)
// in bytes 16..31, and the block scale given by the lanes of group g applies
// to k-values 32g..32g+31.
//
// Scores, S^T[token, head] = K Q^T: the cached e2m1 rows are the A operand
// as they are, with the cache's own e8m0 scales as block scales (lane group g
// of k-step K holds columns 128K + 32g..+32 of its row and that block's
// scale), so the contraction is exact for any scale; the query is the fp8
// B operand, split into e4m3 hi + lo as for the fp8 cache, and laid out to
// match (bytes b < 16: column 128K + 16g + b, bytes 16..31: column
// 128K + 64 + 16g + b - 16).  The 64 rope columns take one more k-step with
// lane groups 2 and 3 zero.
//
// Values, O^T[dim, head] = V^T P^T: a scale of V belongs to a (token, 32
// columns) block, i.e. runs along the output dimension, which no block scale
// of a contraction over tokens can express.  So each tile's V is converted
// once to e4m3 in LDS, each token row relative to its own largest V scale E:
// value = e2m1 x 2^(e - E), exact whenever the row's scales of columns
// 0..511 lie within 8 binades of E (smaller ones are rounded to e4m3,
// subnormals included).  The row's 2^(E - 127) joins the token's softmax
// weight, so the weight of P.V is 2^(x + E - 127 - m) for logit x; those of
// each 32-token k-block are written relative to the block's largest and the
// block's B scale restores them (weight_block_scale).  The k-values are laid
// out so that k-block g is tokens 32g..32g+31 (bytes b < 16: token 16g + b,
// bytes 16..31: token 64 + 16g + b - 16, for V^T and P^T alike); the two
// waves that score a block trade their maxima through LDS before writing P.
//
// Data movement: per tile, 36 cache-to-LDS loads of 1 KB bring the 128 rows
// of e2m1 codes (288 bytes each, rows past the item's end repeat its last
// row) and 20 two-byte loads bring the 18 scale bytes of each row, two per
// LDS dword (the two-byte form writes one dword per lane); waves 0-3 issue
// five code and two scale loads, waves 4-7 four and three.  Two
// raw tiles are in flight while a third is worked on: a raw slot is free
// again as soon as its tile is scored and its V converted.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kXWaves = 8;
constexpr int kXThreads = 64 * kXWaves;
static_assert(kXThreads == kStage1ThreadsMxfp4, "launch shape");
constexpr int kXTile = 128;                        // tokens per tile
constexpr int kXRow = kQkDim / 2;                  // 288 bytes of e2m1 codes per row
constexpr int kXFp4Bytes = kXTile * kXRow;         // 36864
constexpr int kXFp4Loads = kXFp4Bytes / 1024;      // 36
constexpr int kXScalePairs = kQkDim / 64;          // 9 two-byte scale pairs per row
constexpr int kXScaleItems = kXTile * kXScalePairs;  // 1152
constexpr int kXScaleLoads = 20;                   // 1280 lanes >= 1152 pairs
constexpr int kXScaleBytes = kXScaleLoads * 256;   // one dword per lane
constexpr int kXRawBytes = kXFp4Bytes + kXScaleBytes;
constexpr int kXLoadsPerWave = 7;                  // 5 + 2 (waves 0-3) or 4 + 3 (waves 4-7)
constexpr int kXVRow = kVDim + 16;                 // bytes per row of the e4m3 V tile (512 + pad)
constexpr int kXVBytes = kXTile * kXVRow;
constexpr int kQBytes = kNumHeads * kQkDim * 2;    // bf16 query of one sequence
constexpr int kQLoads = kQBytes / 1024;            // 18
constexpr int kPRow = kXTile + 16;                 // bytes per head row of P^T
constexpr int kMaxItemPages = kItemPagesMxfp4;     // page ids of one item staged in LDS
static_assert(4 * 5 + 4 * 4 == kXFp4Loads && 4 * 2 + 4 * 3 == kXScaleLoads && kXScaleLoads * 64 >= kXScaleItems,
              "load split");
static_assert(2 * kQBytes <= kXVBytes, "the query and its e4m3 words are staged in the V tile");

// Position of 16-byte chunk c (0..71) of query head h.  (The V tile needs
// no permutation: at a row pitch of 528 bytes = 132 banks, the eight rows of
// a transposing read fall on distinct banks.)
__host__ __device__ constexpr int q_slot(int h, int c) { return h * 72 + (c ^ (h & 7)); }

struct Fp4Lds {
  uint8_t raw[2][kXRawBytes];              // e2m1 rows, then the scale dwords
  uint8_t v[kXVBytes];                     // V of the current tile as e4m3 [token][dim]; first the query
  uint8_t p[2][kNumHeads][kPRow];          // P^T hi / lo as [head][token]
  float red_m[kNumHeads][kXWaves];         // query head maxima (8 waves), then per scoring wave logit maxima
  float red_y[kNumHeads][4];               // per scoring wave: maxima of logit + row scale
  float red_l[kNumHeads][4];               // per scoring wave: weight sums, at the end
  int32_t pages[kMaxItemPages];            // paged: page ids of the item
};

// Two-byte cache-to-LDS load: lane l's two bytes at src go to LDS dword
// m0 + 4 l.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_u16(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off nt"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}
// The same from base + off (off: per lane, unsigned 32-bit).
__device__ __forceinline__ void dma_u16(const uint8_t* base, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ushort %0, %1 nt"
               :
               : "v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// An fp4 MX operand (16 bytes per lane) in the instruction's 8-register
// tuple, whose upper half the instruction does not read.
__device__ __forceinline__ fp8x32 fp4_operand(u32x4 w) {
  typedef int i32x4v __attribute__((ext_vector_type(4)));
  const i32x4v v = __builtin_bit_cast(i32x4v, w);
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// fp4 (A) x fp8 (B) MX step with A block scale sa (e8m0) and unit B scale.
__device__ __forceinline__ f32x4 mfma_fp4_fp8(fp8x32 a, fp8x32 b, f32x4 c, uint32_t sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, (int)sa, 0, 127);
}
// 8 e2m1 codes (low nibble first) times 2^j -> 8 e4m3 codes (two words),
// through f16 (exact for the products here) and a rounding conversion.
__device__ __forceinline__ void fp4x8_to_fp8(uint32_t w, float scale, uint32_t& lo, uint32_t& hi) {
  typedef short i16x2 __attribute__((ext_vector_type(2)));
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3);
  i16x2 a = {0, 0}, b = {0, 0};
  a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(a, p0, 1.0f, false);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(a, p1, 1.0f, true);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(b, p2, 1.0f, false);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(b, p3, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

// 8 e2m1 codes (low nibble first) times 2^-k, 0 <= k <= 5, -> 8 e4m3 codes
// by table lookup: every nonzero e2m1 magnitude {0.5, 1, 1.5, 2, 3, 4, 6}
// times 2^-k is a normal e4m3 number whose code is the k = 0 code less k in
// the exponent field, so the 8-entry table (lut_lo: magnitudes 0..3, lut_hi:
// 4..7) is a shifted constant; v_perm_b32 looks up four magnitudes at once
// and the sign bit moves from bit 3 to bit 7.  The codes come out as the V
// tile stores a group of 8 columns: even columns (0, 2, 4, 6) in `ev`, odd
// ones in `od`.
__device__ __forceinline__ void fp4x8_to_fp8_lut(uint32_t w, uint32_t lut_lo, uint32_t lut_hi, uint32_t& ev,
                                                 uint32_t& od) {
  ev = ((w << 4) & 0x80808080u) | __builtin_amdgcn_perm(lut_hi, lut_lo, w & 0x07070707u);
  od = (w & 0x80808080u) | __builtin_amdgcn_perm(lut_hi, lut_lo, (w >> 4) & 0x07070707u);
}

// One work item: tokens [tok_begin, tok_end) of one sequence.
template <bool PAGED>
__device__ __forceinline__ void mxfp4_item(const Stage1Args& a, const WorkItem& item, Fp4Lds& sh) {
  const int tid = threadIdx.x;
  if (item.slot == WorkItem::kEmpty) {  // empty sequence: its output is zero
    uint4* dst = reinterpret_cast<uint4*>(a.out + (int64_t)item.batch * kNumHeads * kVDim);
#pragma unroll
    for (int k = 0; k < (kNumHeads * kVDim * 2 / 16) / kXThreads; ++k)
      dst[tid + kXThreads * k] = uint4{0u, 0u, 0u, 0u};
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int b = item.batch;
  const int tok_last = item.tok_end - 1;
  const int ntiles = (item.tok_end - item.tok_begin + kXTile - 1) / kXTile;
  const bool lowq = wave < 4;  // waves 0-3: five code loads and two scale loads per tile

  // The query first: 18 loads into the V tile, load k by wave k % 8.
  {
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (int64_t)b * kNumHeads * kQkDim);
    const uint32_t qm0 = lds_u32(&sh.v[0]);
    for (int k = wave; k < kQLoads; k += kXWaves) {
      const int s = 64 * k + lane;
      const int h = s / 72;
      const int c = (s - 72 * h) ^ (h & 7);
      dma_one(qsrc + (h * 72 + c) * 16, qm0 + 1024 * k);
    }
  }
  const int64_t seq_base = item.kv_base;

  int page0 = 0;
  if constexpr (PAGED) {
    page0 = item.tok_begin >> a.page_shift;
    const int npages = min(((item.tok_end - 1) >> a.page_shift) - page0 + 1, kMaxItemPages);
    // the item's page ids into LDS by four-byte cache-to-LDS loads, all in
    // flight together (lanes past the last page repeat it)
    const int32_t* psrc = a.page_indices + seq_base + page0;
    const uint32_t pm0 = lds_u32(&sh.pages[0]);
    for (int j = wave; 64 * j < npages; j += kXWaves)
      dma_u32(psrc + min(64 * j + lane, npages - 1), pm0 + 256 * j);
    wait_loads<0>();
    lds_barrier();
  }

  // This wave's loads of a tile: code loads j0 .. j0 + 4 (or + 3), scale
  // loads s0 .. s0 + 1 (or + 2); code load j fetches 16-byte chunk
  // (row << 8 | chunk), scale load s the scale pair (row << 8 | pair).
  const int j0 = lowq ? 5 * wave : 20 + 4 * (wave - 4);
  const int s0 = lowq ? 2 * wave : 8 + 3 * (wave - 4);
  uint32_t rc[5], rs[3];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int s = min(64 * (j0 + j) + lane, 64 * kXFp4Loads - 1);
    const int r = s / 18;
    rc[j] = (uint32_t)(r << 8 | (s - 18 * r));
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int s = min(64 * (s0 + j) + lane, kXScaleItems - 1);
    const int r = s / kXScalePairs;
    rs[j] = (uint32_t)(r << 8 | (s - kXScalePairs * r));
  }
  auto row_of = [&](int tok) -> int64_t {  // cache row of logical token tok
    if constexpr (PAGED) {
      const int pmask = (1 << a.page_shift) - 1;
      const uint32_t page = (uint32_t)sh.pages[(tok >> a.page_shift) - page0];
      return (int64_t)((page << a.page_shift) + (uint32_t)(tok & pmask));
    } else {
      return seq_base + tok;
    }
  };
  // Offsets from the tile's first row (contiguous cache): code load j at
  // coff[j] + 1024 j (the instruction offset within its group of four, none
  // for j = 4; 3072 bytes of bias keep coff >= 0), scale load j at soff[j].
  uint32_t coff[5], soff[3];
#pragma unroll
  for (int j = 0; j < 5; ++j) coff[j] = (rc[j] >> 8) * kXRow + 16 * (rc[j] & 0xFF) + 3072 - 1024 * (j & 3);
#pragma unroll
  for (int j = 0; j < 3; ++j) soff[j] = (uint32_t)((rs[j] >> 8) * a.scale_stride) + 2 * (rs[j] & 0xFF);

  // All of this wave's loads of tile t into raw slot t % 2.  Rows past the
  // item's last token fetch that token's row (finite data, masked later).
  auto issue = [&](int t) {
    const int tok0 = item.tok_begin + t * kXTile;
    const int lim = tok_last - tok0;
    const uint32_t m0c = lds_u32(&sh.raw[t & 1][0]) + 1024 * j0;
    const uint32_t m0s = lds_u32(&sh.raw[t & 1][kXFp4Bytes]) + 256 * s0;
    if constexpr (!PAGED) {
      const uint8_t* cbase = uniform_ptr(a.kv + (seq_base + tok0) * kXRow - 3072);
      const uint8_t* sbase = uniform_ptr(a.kv_mx_scales + (seq_base + tok0) * a.scale_stride);
      uint32_t off[5], so[3];
      if (lim >= kXTile - 1) {  // a whole tile
#pragma unroll
        for (int j = 0; j < 5; ++j) off[j] = coff[j];
#pragma unroll
        for (int j = 0; j < 3; ++j) so[j] = soff[j];
      } else {
#pragma unroll
        for (int j = 0; j < 5; ++j)
          off[j] = min((int)(rc[j] >> 8), lim) * kXRow + 16 * (rc[j] & 0xFF) + 3072 - 1024 * (j & 3);
#pragma unroll
        for (int j = 0; j < 3; ++j)
          so[j] = (uint32_t)(min((int)(rs[j] >> 8), lim) * a.scale_stride) + 2 * (rs[j] & 0xFF);
      }
      dma_group<4>(cbase, off, m0c);
      if (lowq) dma_group<1>(cbase, off + 4, m0c + 4096);
      dma_u16(sbase, so[0], m0s);
      dma_u16(sbase, so[1], m0s + 256);
      if (!lowq) dma_u16(sbase, so[2], m0s + 512);
    } else {
      const uint8_t* src[5];
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const int r = min((int)(rc[j] >> 8), lim);
        src[j] = a.kv + row_of(tok0 + r) * kXRow + 16 * (rc[j] & 0xFF) - 1024 * (j & 3);
      }
      dma_group<4>(src, m0c);
      if (lowq) dma_one(src[4], m0c + 4096);  // no instruction offset
      const uint8_t* ssrc[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int r = min((int)(rs[j] >> 8), lim);
        ssrc[j] = a.kv_mx_scales + row_of(tok0 + r) * a.scale_stride + 2 * (rs[j] & 0xFF);
      }
      dma_u16(ssrc[0], m0s);
      dma_u16(ssrc[1], m0s + 256);
      if (!lowq) dma_u16(ssrc[2], m0s + 512);
    }
  };

  issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 1)
    wait_loads<2 * kXLoadsPerWave>();  // the query has landed
  else
    wait_loads<kXLoadsPerWave>();
  lds_barrier();

  // Query, B operand of the scores, scaled by 2^s and split into e4m3 hi +
  // lo.  K-step K (0..3): bytes b < 16 column 128K + 16g + b, bytes 16..31
  // column 128K + 64 + 16g + b - 16; rope step: bytes b < 16 column
  // 512 + 16g + b, bytes 16..31 zero.  Every wave needs all of it; wave w
  // converts half j = w & 1 (bytes 16j .. 16j + 15) of K-step w >> 1, and
  // waves 0, 1 half w of the rope step; the waves trade their head maxima
  // and then the converted words through LDS, behind the bf16 query.
  fp8x32 qh[4], ql[4], rh, rl;
  float xscale;
  {
    const uint8_t* qlds = &sh.v[0];
    // converted words: [K][hi, lo][lane][8], then rope [hi, lo][lane][4]
    uint32_t* const qcv = reinterpret_cast<uint32_t*>(&sh.v[kQBytes]);
    const int K0 = wave >> 1, j = wave & 1;
    const bool rope = wave < 2;
    bf16x8 qv[3];  // [i]: chunk 16 K0 + 2g + 8j + i; [2]: rope chunk 64 + 2g + wave
#pragma unroll
    for (int i = 0; i < 2; ++i)
      qv[i] = *reinterpret_cast<const bf16x8*>(qlds + 16 * q_slot(r16, 16 * K0 + 2 * g + 8 * j + i));
    qv[2] = rope ? *reinterpret_cast<const bf16x8*>(qlds + 16 * q_slot(r16, 64 + 2 * g + wave)) : bf16x8{};
    float am[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      float m0 = fmaxf(fabsf((float)qv[k][0]), fabsf((float)qv[k][1]));
      float m1 = fmaxf(fabsf((float)qv[k][2]), fabsf((float)qv[k][3]));
      float m2 = fmaxf(fabsf((float)qv[k][4]), fabsf((float)qv[k][5]));
      float m3 = fmaxf(fabsf((float)qv[k][6]), fabsf((float)qv[k][7]));
      am[k] = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
    }
    float amax = xor_max_groups(fmaxf(fmaxf(am[0], am[1]), am[2]));
    if (g == 0) sh.red_m[r16][wave] = amax;
    lds_barrier();
    const f32x4 wm0 = *reinterpret_cast<const f32x4*>(&sh.red_m[r16][0]);
    const f32x4 wm1 = *reinterpret_cast<const f32x4*>(&sh.red_m[r16][4]);
    amax = fmaxf(fmaxf(fmaxf(wm0[0], wm0[1]), fmaxf(wm0[2], wm0[3])),
                 fmaxf(fmaxf(wm1[0], wm1[1]), fmaxf(wm1[2], wm1[3])));
    const int s = (amax > 0.f) ? 8 - __builtin_amdgcn_frexp_expf(amax) : 0;
    xscale = a.score_scale * __builtin_ldexpf(1.0f, -s);
    uint32_t hw[6], lw[6];  // word 2k + m: elements 4m..4m+3 of qv[k]
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        split_fp8x4(__builtin_ldexpf((float)qv[k][4 * m], s), __builtin_ldexpf((float)qv[k][4 * m + 1], s),
                    __builtin_ldexpf((float)qv[k][4 * m + 2], s), __builtin_ldexpf((float)qv[k][4 * m + 3], s),
                    hw[2 * k + m], lw[2 * k + m]);
    *reinterpret_cast<u32x4*>(qcv + ((2 * K0) * 64 + lane) * 8 + 4 * j) = u32x4{hw[0], hw[1], hw[2], hw[3]};
    *reinterpret_cast<u32x4*>(qcv + ((2 * K0 + 1) * 64 + lane) * 8 + 4 * j) = u32x4{lw[0], lw[1], lw[2], lw[3]};
    if (rope) {
      *reinterpret_cast<uint2*>(qcv + 4096 + lane * 4 + 2 * wave) = uint2{hw[4], hw[5]};
      *reinterpret_cast<uint2*>(qcv + 4096 + (64 + lane) * 4 + 2 * wave) = uint2{lw[4], lw[5]};
    }
    lds_barrier();
#pragma unroll
    for (int K = 0; K < 4; ++K) {
      const u32x4* h = reinterpret_cast<const u32x4*>(qcv + ((2 * K) * 64 + lane) * 8);
      const u32x4* l = reinterpret_cast<const u32x4*>(qcv + ((2 * K + 1) * 64 + lane) * 8);
      qh[K] = join16(h[0], h[1]);
      ql[K] = join16(l[0], l[1]);
    }
    const u32x4 wh = *reinterpret_cast<const u32x4*>(qcv + 4096 + lane * 4);
    const u32x4 wl = *reinterpret_cast<const u32x4*>(qcv + 4096 + (64 + lane) * 4);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      rh[d] = d < 4 ? (int)wh[d] : 0;
      rl[d] = d < 4 ? (int)wl[d] : 0;
    }
  }

  f32x4 o[4];  // O^T[dim 64w + 16v + 4g + i][head r16]
#pragma unroll
  for (int v = 0; v < 4; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;
  float l_part = 0.f;

  // Roles.  Waves 0-3 score: wave s takes the 32 tokens 32s..32s+31 of the
  // tile (two 16-row MFMA blocks), which are exactly k-block s of the P.V
  // step, so the maximum that scales the block's weights is the wave's own.
  // Waves 4-7 convert V: wave 4 + c converts token rows 32c..32c+31, lane l
  // row 32c + (l & 31) and column blocks 8(l >> 5)..+7.  With one scoring and
  // one converting wave on each SIMD, the matrix steps of one overlap the
  // vector work of the other.  Then every wave runs P.V for its 64 columns.
  // Reads of this lane for P.V: tr8 read q (0..3) gives tokens tb(q) +
  // (0..7), tb = 16g + 8q (q < 2) or 64 + 16g + 8(q - 2), from rows tb(q) +
  // (r16 >> 1), columns 64w + 16v + 8(r16 & 1).
  const bool scorer = wave < 4;
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    voff[q] = ((q < 2 ? 16 * g + 8 * q : 64 + 16 * g + 8 * (q - 2)) + (r16 >> 1)) * kXVRow + 64 * wave +
              8 * (r16 & 1);
  uint8_t* const p_hi = &sh.p[0][r16][0];
  uint8_t* const p_lo = &sh.p[1][r16][0];

  for (int t = 0; t < ntiles; ++t) {
    const int tok0 = item.tok_begin + t * kXTile;
    if (t + 1 < ntiles)
      wait_loads<kXLoadsPerWave>();  // tile t, not tile t + 1 behind it
    else
      wait_loads<0>();
    lds_barrier();  // tile t everywhere; everyone is past tile t - 1
    const uint8_t* raw = &sh.raw[t & 1][0];
    const uint8_t* sdw = raw + kXFp4Bytes;  // scale pair (row, p) at dword 9 row + p

    float lsum = 0.f, cw = 0.f;  // scorers: this lane's weights against the wave's reference cw
    bool wlive = false;
    if (scorer) {
      // ---- scores of tokens 32s + 16h + (0..15), h = 0, 1 ----
      // The fp4 A operand is 16 bytes; the upper half of its register tuple
      // is not read, so it is left undefined rather than zeroed.
      f32x4 sacc[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) sacc[h][0] = sacc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 32 * wave + 16 * h + r16;
        const uint8_t* rp = raw + row * kXRow;
        const uint8_t* sp = sdw + 4 * kXScalePairs * row;
#pragma unroll
        for (int K = 0; K < 4; ++K) {
          const int blk = 4 * K + g;
          const uint32_t sa = sp[4 * (blk >> 1) + (blk & 1)];
          const fp8x32 ka = fp4_operand(*reinterpret_cast<const u32x4*>(rp + 64 * K + 16 * g));
          sacc[h][0] = mfma_fp4_fp8(ka, qh[K], sacc[h][0], sa);
          sacc[h][1] = mfma_fp4_fp8(ka, ql[K], sacc[h][1], sa);
        }
        u32x4 w = {0u, 0u, 0u, 0u};
        uint32_t sa = 127;
        if (g < 2) {
          w = *reinterpret_cast<const u32x4*>(rp + 256 + 16 * g);
          sa = sp[4 * 8 + g];
        }
        const fp8x32 ka = fp4_operand(w);
        sacc[h][0] = mfma_fp4_fp8(ka, rh, sacc[h][0], sa);
        sacc[h][1] = mfma_fp4_fp8(ka, rl, sacc[h][1], sa);
      }

      // E of the wave's tokens (the largest of each row's 16 scales of
      // columns 0..511): lanes l and l ^ 32 take 8 scales each of token
      // 32s + (l & 31); then lane (head r16, group g) fetches the E of its
      // tokens 16h + 4g + i.
      float erow;
      {
        const uint32_t* srow = reinterpret_cast<const uint32_t*>(sdw) + kXScalePairs * (32 * wave + (lane & 31)) +
                               4 * (lane >> 5);
        uint32_t em = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t d = srow[k];  // scale pair in the low 16 bits
          em = max(em, max(d & 0xFFu, (d >> 8) & 0xFFu));
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(em, em, false, false);
        erow = (float)max((uint32_t)sw[0], (uint32_t)sw[1]);
      }

      // ---- softmax: x[h][i] is token 32s + 16h + 4g + i of head r16 ----
      // y = x + E - 127 is the log2 size of the token's weight times its row
      // scale 2^(E - 127), which the e4m3 V rows leave out; the block's
      // weights are written relative to its largest y (weight_block_scale).
      // The sum of this lane's weights is taken against the wave's integral
      // reference cw (the floor of its logit maximum) and moved to the running
      // maximum's scale once that is known.
      float x[2][4], y[2][4];
      float tmax = kNegInf, ymax = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ei =
              __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (16 * h + 4 * g + i), __float_as_int(erow)));
          x[h][i] = (sacc[h][0][i] + sacc[h][1][i]) * xscale;
          if (tok0 + 32 * wave + 16 * h + 4 * g + i > tok_last) x[h][i] = kNegInf;
          y[h][i] = x[h][i] + (ei - 127.0f);
          tmax = fmaxf(tmax, x[h][i]);
          ymax = fmaxf(ymax, y[h][i]);
        }
      tmax = xor_max_groups(tmax);
      ymax = xor_max_groups(ymax);
      if (g == 0) {
        sh.red_m[r16][wave] = tmax;
        sh.red_y[r16][wave] = ymax;
      }
      wlive = tmax != kNegInf;
      cw = weight_block_floor(tmax);
      const float shift = 7.0f - weight_block_floor(ymax);  // y + shift < 8
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float pw[4];
        uint32_t ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[i] = __builtin_amdgcn_exp2f(y[h][i] + shift);
          lsum += __builtin_amdgcn_exp2f(x[h][i] - cw);
        }
        split_fp8x4(pw[0], pw[1], pw[2], pw[3], ph, pl);
        *reinterpret_cast<uint32_t*>(p_hi + 32 * wave + 16 * h + 4 * g) = ph;
        *reinterpret_cast<uint32_t*>(p_lo + 32 * wave + 16 * h + 4 * g) = pl;
      }
    } else {
      // ---- V of this tile to e4m3, each token row relative to its own
      // largest V scale E: lanes l and l ^ 32 hold the row's 16 scales ----
      // By table, exact for blocks within 5 binades of the row's E (nearly
      // all); a block further below is converted again by rounding
      // conversions (exact within 8 binades, rounded to e4m3 beyond).
      const int row = 32 * (wave - 4) + (lane & 31);
      const int cb0 = 8 * (lane >> 5);
      uint32_t e[8];
      u32x4 wv[8];
      const uint8_t* rsrc = raw + row * kXRow + 16 * cb0;
      const uint8_t* ssrc = sdw + 4 * kXScalePairs * row + 2 * cb0;  // pair cb/2 at dword 9 row + cb/2
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        e[k] = ssrc[4 * (k >> 1) + (k & 1)];
        wv[k] = *reinterpret_cast<const u32x4*>(rsrc + 16 * k);
      }
      uint32_t em = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) em = max(em, e[k]);
      const auto sw = __builtin_amdgcn_permlane32_swap(em, em, false, false);
      const int E = (int)max((uint32_t)sw[0], (uint32_t)sw[1]);
      uint8_t* const vdst = &sh.v[row * kXVRow + 32 * cb0];
      int jmin = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = max((int)e[k] - E, -126);  // <= 0
        jmin = min(jmin, j);
        const uint32_t kk = (uint32_t)min(-j, 5);
        const uint32_t lut_lo = 0x3C383000u - kk * 0x08080800u;
        const uint32_t lut_hi = 0x4C484440u - kk * 0x08080808u;
        uint32_t e8[8];  // 32 e4m3 codes: word 2i columns 32cb + 8i + {0,2,4,6}, word 2i+1 the odd ones
#pragma unroll
        for (int i = 0; i < 4; ++i) fp4x8_to_fp8_lut(wv[k][i], lut_lo, lut_hi, e8[2 * i], e8[2 * i + 1]);
        *reinterpret_cast<u32x4*>(vdst + 32 * k) = u32x4{e8[0], e8[1], e8[2], e8[3]};
        *reinterpret_cast<u32x4*>(vdst + 32 * k + 16) = u32x4{e8[4], e8[5], e8[6], e8[7]};
      }
      if (__ballot(jmin < -5) != 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int j = max((int)e[k] - E, -126);
          if (j >= -5) continue;
          const float scale = __uint_as_float((uint32_t)(127 + j) << 23);
          uint32_t e8[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t lo, hi;  // columns 0..3, 4..7
            fp4x8_to_fp8(wv[k][i], scale, lo, hi);
            e8[2 * i] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);      // columns 0, 2, 4, 6
            e8[2 * i + 1] = __builtin_amdgcn_perm(hi, lo, 0x07050301u);  // columns 1, 3, 5, 7
          }
          *reinterpret_cast<u32x4*>(vdst + 32 * k) = u32x4{e8[0], e8[1], e8[2], e8[3]};
          *reinterpret_cast<u32x4*>(vdst + 32 * k + 16) = u32x4{e8[4], e8[5], e8[6], e8[7]};
        }
      }
    }
    lds_barrier();  // P^T, the maxima and the V tile; raw slot t % 2 is free
    if (t + 2 < ntiles) issue(t + 2);

    const f32x4 mx = *reinterpret_cast<const f32x4*>(&sh.red_m[r16][0]);
    const f32x4 my = *reinterpret_cast<const f32x4*>(&sh.red_y[r16][0]);
    const float tile_max = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    // Every wave reads the same maxima, so this branch is uniform.
    if (__ballot(tile_max > m_ref + kLazyRescale) != 0) {
      const float m_new = floorf(fmaxf(m_ref, tile_max));
      const float alpha = (m_ref == kNegInf) ? 0.0f : __builtin_ldexpf(1.0f, (int)(m_ref - m_new));
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] *= alpha;
      l_part *= alpha;
      m_ref = m_new;
    }
    if (wlive) l_part += __builtin_ldexpf(lsum, (int)cw - (int)m_ref);
    // B scale of k-block g (scoring wave g's tokens) for head r16
    const int sb = weight_block_scale(g == 0 ? my[0] : g == 1 ? my[1] : g == 2 ? my[2] : my[3], m_ref);
    const fp8x32 bh = join16(*reinterpret_cast<const u32x4*>(p_hi + 16 * g),
                             *reinterpret_cast<const u32x4*>(p_hi + 64 + 16 * g));
    const fp8x32 bl = join16(*reinterpret_cast<const u32x4*>(p_lo + 16 * g),
                             *reinterpret_cast<const u32x4*>(p_lo + 64 + 16 * g));

    // ---- O^T += V^T P^T, columns 64w + 16v ----
#pragma unroll
    for (int v = 0; v < 4; v += 2) {
      fp8x32 va[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x2 raw2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(&sh.v[voff[q] + 16 * (v + u)]));
          va[u][2 * q] = raw2[0];
          va[u][2 * q + 1] = raw2[1];
        }
      o[v] = mfma_fp8_k128_sb(va[0], bh, o[v], sb);
      o[v + 1] = mfma_fp8_k128_sb(va[1], bh, o[v + 1], sb);
      o[v] = mfma_fp8_k128_sb(va[0], bl, o[v], sb);
      o[v + 1] = mfma_fp8_k128_sb(va[1], bl, o[v + 1], sb);
    }
  }

  // Only the scoring waves hold weight sums.
  const float l_w = xor_sum_groups(l_part);
  if (scorer && g == 0) sh.red_l[r16][wave] = l_w;
  lds_barrier();
  const f32x4 ls = *reinterpret_cast<const f32x4*>(&sh.red_l[r16][0]);
  const float L = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  // The V tile holds each group of 8 columns as (0, 2, 4, 6, 1, 3, 5, 7), so
  // lane group g has output columns 8(g >> 1) + 2i + (g & 1) of each column
  // tile; lanes l and l ^ 16 trade two values each to return to columns
  // 4g + i.
  {
    const int partner = (lane ^ 16) << 2;
    const bool odd = (g & 1) != 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float r0 = __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(odd ? o[v][0] : o[v][2])));
      const float r1 = __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(odd ? o[v][1] : o[v][3])));
      o[v] = odd ? f32x4{r0, o[v][2], r1, o[v][3]} : f32x4{o[v][0], r0, o[v][1], r1};
    }
  }
  finish_item<4>(a, item, tid, wave >> 1, 4 * (wave & 1), lane, o, 1.0f / L, m_ref + __log2f(L));
}

// A workgroup runs one item, or with bins the items of bin blockIdx.x in
// order (see Stage1Args).  Between two items every load and store of the
// first is complete and every wave is past it, so the next may reuse LDS.
template <bool PAGED>
__global__ __launch_bounds__(kXThreads, 1) void mla_stage1_mxfp4(Stage1Args a) {
  __shared__ __attribute__((aligned(16))) Fp4Lds sh;
  int i = a.bins ? a.bins[blockIdx.x] : (int)blockIdx.x;
  const int i_end = a.bins ? a.bins[blockIdx.x + 1] : i + 1;
  while (i < i_end) {
    const WorkItem item = a.uniform_splits
                              ? uniform_item(xcd_block(blockIdx.x, gridDim.x), a.uniform_splits, a.uniform_chunk,
                                             a.uniform_len, a.uniform_base)
                              : a.items[i];
    mxfp4_item<PAGED>(a, item, sh);
    if (++i == i_end) break;
    wait_loads<0>();
    lds_barrier();
  }
}

}  // namespace

const void* stage1_mxfp4_kernel(bool paged) {
  return paged ? reinterpret_cast<const void*>(&mla_stage1_mxfp4<true>)
               : reinterpret_cast<const void*>(&mla_stage1_mxfp4<false>);
}

}  // namespace mla
