// gfx950 split kernel for an MXFP4 cache (e2m1 codes, one e8m0 scale per 32
// columns of a row): single-token multi-head latent attention decode, one
// 512-thread workgroup (eight waves, two per SIMD) per planned work item,
// 128-token tiles streamed HBM -> LDS by cache-to-LDS loads, both
// contractions on the MX matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4.
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
// block's B scale restores them (weight_block_scale).  The k-values of P.V
// are the tile's tokens in order (bytes b < 16 of lane group g: token
// 16g + b, bytes 16..31: token 64 + 16g + b - 16, for V^T and P^T alike), so
// k-block g is tokens 32g..32g+31.
//
// Roles.  Waves 0-3 score: wave s takes tokens 32s..32s+31 of each tile
// (two 16-row blocks), exactly k-block s of P.V, so the maximum that scales
// the block's weights is the wave's own; these waves also issue every cache
// load.  Waves 4-7 hold V: wave 4 + c converts columns 128c..128c+127 of
// every token of a tile into its own e4m3 block of LDS and contracts them
// with P.  Each SIMD runs one wave of each kind.
//
// Pipeline, iteration i of an item: barrier; every wave copies what it needs
// of raw tile i into registers, and the scoring waves find the row exponents E;
// barrier, after which the raw slot is free and the tile after next is
// issued into it.  Then the scoring waves score tile i and write its weights
// P_i, while each V wave runs P.V of tile i - 1 over its own columns and
// converts tile i into them (its stores come after its last read of tile
// i - 1), so that the vector work of converting shares an instruction stream
// with the matrix work of P.V, and the scoring wave's contraction runs beside
// both on the same SIMD.  P and the block maxima alternate between two
// buffers by tile parity; one iteration more than tiles drains the last P.V.
//
// Data movement: per tile, 36 cache-to-LDS loads of 1 KB bring the 128 rows
// of e2m1 codes (288 bytes each, rows past the item's end repeat its last
// row) and 20 two-byte loads bring the 18 scale bytes of each row, two per
// LDS dword (the two-byte form writes one dword per lane); each scoring wave
// issues nine code and five scale loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kXWaves = 8;
constexpr int kXThreads = 64 * kXWaves;
static_assert(kXThreads == kStage1ThreadsMxfp4, "launch shape");
constexpr int kXTile = 128;                          // tokens per tile
constexpr int kXRow = kQkDim / 2;                    // 288 bytes of e2m1 codes per row
constexpr int kXFp4Bytes = kXTile * kXRow;           // 36864
constexpr int kXFp4Loads = kXFp4Bytes / 1024;        // 36
constexpr int kXScalePairs = kQkDim / 64;            // 9 two-byte scale pairs per row
constexpr int kXScaleItems = kXTile * kXScalePairs;  // 1152
constexpr int kXScaleLoads = 20;                     // 1280 lanes >= 1152 pairs
constexpr int kXScaleBytes = kXScaleLoads * 256;     // one dword per lane
constexpr int kXRawBytes = kXFp4Bytes + kXScaleBytes;
constexpr int kXCodeLoads = kXFp4Loads / 4;          // per scoring wave
constexpr int kXPairLoads = kXScaleLoads / 4;        // per scoring wave
constexpr int kXLoadsPerWave = kXCodeLoads + kXPairLoads;
constexpr int kXCols = kVDim / 4;                    // V columns per V wave
constexpr int kXVBytes = kXTile * kXCols;            // its e4m3 block: [16-column chunk][token][16]
constexpr int kQBytes = kNumHeads * kQkDim * 2;      // bf16 query of one sequence
constexpr int kQLoads = kQBytes / 1024;              // 18
constexpr int kMaxItemPages = kItemPagesMxfp4;       // page ids of one item staged in LDS
static_assert(4 * kXCodeLoads == kXFp4Loads && 4 * kXPairLoads == kXScaleLoads && kXScaleLoads * 64 >= kXScaleItems,
              "load split");
static_assert(2 * kQBytes <= 4 * kXVBytes, "the query and its e4m3 words are staged in the V blocks");
static_assert(4 * 8 * 64 * 16 <= kXRawBytes, "the output hand-over fits a raw slot");

// Position of 16-byte chunk c (0..71) of query head h.
__host__ __device__ constexpr int q_slot(int h, int c) { return h * 72 + (c ^ (h & 7)); }
// A V block stores 16-column chunk c of token row r at 2048 c + 16 v_slot(r):
// the 16 rows that one store instruction writes, and the eight rows of a
// transposing read, are consecutive 16-byte words, and the two halves of odd
// groups of 16 rows trade places, so that lane groups 0 and 1 of a read (rows
// 8q.. and 16 + 8q..) fall on different banks as well.
constexpr int kXVChunk = kXTile * 16;
__host__ __device__ constexpr int v_slot(int r) { return r ^ (((r >> 4) & 1) << 3); }
// Chunk c (0..7) of head row h of P^T (rows of 128 bytes), permuted so that
// the 16 head rows reading one chunk fall on distinct banks.
__host__ __device__ constexpr int p_chunk(int h, int c) { return c ^ ((h >> 1) & 7); }

struct Fp4Lds {
  uint8_t raw[2][kXRawBytes];            // e2m1 rows, then the scale dwords
  uint8_t v[4][kXVBytes];                // V wave c's e4m3 columns; first the query
  uint8_t p[2][2][kNumHeads][kXTile];    // [tile parity][hi, lo][head][token]: P^T
  float red_m[2][kNumHeads][4];          // [tile parity][head][scoring wave]: logit maxima
  float red_y[2][kNumHeads][4];          // the same for logit + row exponent
  int32_t erow[kXTile];                  // row exponents E of the tile in hand
  int32_t pages[kMaxItemPages];          // paged: page ids of the item
};
static_assert(sizeof(Fp4Lds) <= 160 * 1024, "LDS");

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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// An fp4 MX operand (16 bytes per lane) in the instruction's 8-register
// tuple, whose upper half the instruction does not read.
__device__ __forceinline__ fp8x32 fp4_operand(u32x4 w) {
  const i32x4 v = __builtin_bit_cast(i32x4, w);
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
// blocks store a group of 8 columns: even columns (0, 2, 4, 6) in `ev`, odd
// ones in `od`.
__device__ __forceinline__ void fp4x8_to_fp8_lut(uint32_t w, uint32_t lut_lo, uint32_t lut_hi, uint32_t& ev,
                                                 uint32_t& od) {
  ev = ((w << 4) & 0x80808080u) | __builtin_amdgcn_perm(lut_hi, lut_lo, w & 0x07070707u);
  od = (w & 0x80808080u) | __builtin_amdgcn_perm(lut_hi, lut_lo, (w >> 4) & 0x07070707u);
}
// The thread's index, hidden from the optimiser at the point of the call, so
// that values derived from it are computed there instead of being hoisted out
// of the item and tile loops and kept live (or spilled) across them.
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int opaque_lane() { return opaque_tid() & 63; }

// Table words for 2^-k: 8k off every byte but that of magnitude 0.
__device__ __forceinline__ void fp4_lut(uint32_t k, uint32_t& lut_lo, uint32_t& lut_hi) {
  const uint32_t k8 = k << 3;
  const uint32_t rep = __builtin_amdgcn_perm(0u, k8, 0u);  // k8 in every byte
  lut_lo = (0x3C383000u | k8) - rep;
  lut_hi = 0x4C484440u - rep;
}

// One work item: tokens [tok_begin, tok_end) of one sequence.  Q1: the query
// enters the scores as one e4m3 code per element (hi alone), not as hi + lo.
template <bool PAGED, bool Q1>
__device__ __forceinline__ void mxfp4_item(const Stage1Args& a, const WorkItem& item, Fp4Lds& sh) {
  const int tid = opaque_tid();
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
  const bool scorer = wave < 4;

  // The query first: 18 loads into the V blocks, load k by wave k % 8.
  {
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (int64_t)b * kNumHeads * kQkDim);
    const uint32_t qm0 = lds_u32(&sh.v[0][0]);
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
  }
  // The query (and the page ids) land before the first tiles are issued:
  // issued together with the first tiles of every CU, the query would queue
  // behind them at the memory and land last.
  wait_loads<0>();
  lds_barrier();

  auto row_of = [&](int tok) -> int64_t {  // cache row of logical token tok
    if constexpr (PAGED) {
      const int pmask = (1 << a.page_shift) - 1;
      const uint32_t page = (uint32_t)sh.pages[(tok >> a.page_shift) - page0];
      return (int64_t)((page << a.page_shift) + (uint32_t)(tok & pmask));
    } else {
      return seq_base + tok;
    }
  };
  // Scale loads of whole tiles of a contiguous cache: pair sp = 64 j' + lane
  // of the tile (row sp / 9, pair sp % 9) at soff[j] from the tile's first
  // scale row, j' = 5 wave + j (the offsets fit 32 bits for strides up to
  // 2^24).
  const bool short_stride = a.scale_stride <= (int64_t(1) << 24);
  uint32_t soff[kXPairLoads];
#pragma unroll
  for (int j = 0; j < kXPairLoads; ++j) {
    const int sp = min(64 * (kXPairLoads * wave + j) + lane, kXScaleItems - 1);
    const int r = sp / kXScalePairs;
    soff[j] = (uint32_t)(r * (short_stride ? (int)a.scale_stride : 0)) + 2 * (sp - kXScalePairs * r);
  }

  // All loads of tile t into raw slot t % 2, issued by scoring wave `wave`:
  // code loads j' = 9 wave .. 9 wave + 8 (16-byte chunk 64 j' + lane of the
  // tile's rows: row / 18, chunk % 18) and scale loads 5 wave .. 5 wave + 4.
  // Rows past the item's last token fetch that token's row (finite data,
  // masked later).
  auto issue = [&](int t) {
    const int tok0 = item.tok_begin + t * kXTile;
    const int lim = tok_last - tok0;
    const uint32_t m0c = lds_u32(&sh.raw[t & 1][0]) + 1024 * kXCodeLoads * wave;
    const uint32_t m0s = lds_u32(&sh.raw[t & 1][kXFp4Bytes]) + 256 * kXPairLoads * wave;
    if (!PAGED && lim >= kXTile - 1 && short_stride) {  // a whole tile of a contiguous cache
      const uint8_t* cb = uniform_ptr(a.kv + (seq_base + tok0) * kXRow + 1024 * kXCodeLoads * wave);
      const uint32_t o16 = 16 * lane;
      const uint32_t off[4] = {o16, o16, o16, o16};
      dma_group<4>(cb, off, m0c);
      dma_group<4>(cb + 4096, off, m0c + 4096);
      dma_group<1>(cb + 8192, off, m0c + 8192);
      const uint8_t* sbase = uniform_ptr(a.kv_mx_scales + (seq_base + tok0) * a.scale_stride);
#pragma unroll
      for (int j = 0; j < kXPairLoads; ++j) dma_u16(sbase, soff[j], m0s + 256 * j);
    } else {
      const uint8_t* src[kXCodeLoads];  // less the instruction offset 1024 (j % 4)
#pragma unroll
      for (int j = 0; j < kXCodeLoads; ++j) {
        const int c = 64 * (kXCodeLoads * wave + j) + lane;
        const int r = c / 18;
        src[j] = a.kv + row_of(tok0 + min(r, lim)) * kXRow + 16 * (c - 18 * r) - 1024 * (j & 3);
      }
      dma_group<4>(src, m0c);
      dma_group<4>(src + 4, m0c + 4096);
      dma_one(src[8], m0c + 8192);
#pragma unroll
      for (int j = 0; j < kXPairLoads; ++j) {
        const int sp = min(64 * (kXPairLoads * wave + j) + lane, kXScaleItems - 1);
        const int r = sp / kXScalePairs;
        dma_u16(a.kv_mx_scales + row_of(tok0 + min(r, lim)) * a.scale_stride + 2 * (sp - kXScalePairs * r),
                m0s + 256 * j);
      }
    }
  };

  if (scorer) {
    issue(0);
    if (ntiles > 1) issue(1);
  }

  // Query, B operand of the scores, scaled by 2^s and split into e4m3 hi +
  // lo.  K-step K (0..3): bytes b < 16 column 128K + 16g + b, bytes 16..31
  // column 128K + 64 + 16g + b - 16; rope step: bytes b < 16 column
  // 512 + 16g + b, bytes 16..31 zero.  The scoring waves need all of it;
  // wave w converts half j = w & 1 (bytes 16j .. 16j + 15) of K-step w >> 1,
  // and waves 0, 1 half w of the rope step; the waves trade their head
  // maxima and then the converted words through LDS, behind the bf16 query.
  uint32_t* const qcv = reinterpret_cast<uint32_t*>(&sh.v[0][0] + kQBytes);
  float xscale;
  {
    float(*const qmax)[8] = reinterpret_cast<float(*)[8]>(&sh.red_m[0][0][0]);
    const uint8_t* qlds = &sh.v[0][0];
    // converted words: [K][hi, lo][lane][8], then rope [hi, lo][lane][4]
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
    if (g == 0) qmax[r16][wave] = amax;
    lds_barrier();
    const f32x4 wm0 = *reinterpret_cast<const f32x4*>(&qmax[r16][0]);
    const f32x4 wm1 = *reinterpret_cast<const f32x4*>(&qmax[r16][4]);
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
  }

  // At the end, raw slot 0 hands the V waves' output over ([V wave][column
  // tile][lane]) and raw slot 1 holds the weight sums and references.
  f32x4* const hand = reinterpret_cast<f32x4*>(&sh.raw[0][0]);
  float* const fin_m = reinterpret_cast<float*>(&sh.raw[1][0]);  // [head]: running maximum of P.V
  float(*const fin_l)[4] = reinterpret_cast<float(*)[4]>(&sh.raw[1][256]);   // [head][scoring wave]
  float(*const fin_ls)[4] = reinterpret_cast<float(*)[4]>(&sh.raw[1][512]);  // their references

  if (scorer) {
    const int s = wave;
    fp8x32 qh[4], ql[4], rh, rl;
#pragma unroll
    for (int K = 0; K < 4; ++K) {
      const u32x4* h = reinterpret_cast<const u32x4*>(qcv + ((2 * K) * 64 + lane) * 8);
      const u32x4* l = reinterpret_cast<const u32x4*>(qcv + ((2 * K + 1) * 64 + lane) * 8);
      qh[K] = join16(h[0], h[1]);
      ql[K] = join16(l[0], l[1]);
    }
    {
      const u32x4 wh = *reinterpret_cast<const u32x4*>(qcv + 4096 + lane * 4);
      const u32x4 wl = *reinterpret_cast<const u32x4*>(qcv + 4096 + (64 + lane) * 4);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        rh[d] = d < 4 ? (int)wh[d] : 0;
        rl[d] = d < 4 ? (int)wl[d] : 0;
      }
    }
    // This wave's weight sum per head, against its own integral reference.
    float m_s = kNegInf, l_s = 0.f;
    const int pw_off = r16 * kXTile + 4 * g;  // + 16 p_chunk(r16, 2s + h): tokens 32s + 16h + 4g ..

    for (int i = 0; i <= ntiles; ++i) {
      if (i < ntiles) {
        if (i + 1 < ntiles)
          wait_loads<kXLoadsPerWave>();  // tile i, not tile i + 1 behind it
        else
          wait_loads<0>();
      }
      lds_barrier();  // tile i everywhere; every wave is past iteration i - 1
      // Rows 32s + 16h + r16 of tile i: lane group g of k-step K holds
      // columns 128K + 32g .. +31 and their scale; the rope step groups 0, 1.
      u32x4 kc[2][5];
      uint32_t sa[2][5];
      if (i < ntiles) {
        const uint8_t* raw = &sh.raw[i & 1][0];
        const uint8_t* sdw = raw + kXFp4Bytes;  // scale pair (row, p) at dword 9 row + p
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 32 * s + 16 * h + r16;
          const uint8_t* rp = raw + row * kXRow;
          const uint8_t* sp = sdw + 4 * kXScalePairs * row;
#pragma unroll
          for (int K = 0; K < 4; ++K) {
            const int blk = 4 * K + g;
            kc[h][K] = *reinterpret_cast<const u32x4*>(rp + 64 * K + 16 * g);
            sa[h][K] = sp[4 * (blk >> 1) + (blk & 1)];
          }
          kc[h][4] = u32x4{0u, 0u, 0u, 0u};
          sa[h][4] = 127;
          if (g < 2) {
            kc[h][4] = *reinterpret_cast<const u32x4*>(rp + 256 + 16 * g);
            sa[h][4] = sp[4 * 8 + g];
          }
        }
        // E of rows 32s + (lane & 31), the largest of the row's 16 scales of
        // columns 0..511: lanes l and l ^ 32 take pairs 0..3 / 4..7.
        const uint32_t* er =
            reinterpret_cast<const uint32_t*>(sdw) + kXScalePairs * (32 * s + (lane & 31)) + 4 * (lane >> 5);
        uint32_t em = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t d = er[k];  // scale pair in the low 16 bits
          em = max(em, max(d & 0xFFu, (d >> 8) & 0xFFu));
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(em, em, false, false);
        if (lane < 32) sh.erow[32 * s + lane] = (int)max((uint32_t)sw[0], (uint32_t)sw[1]);
      }
      lds_barrier();  // raw slot i % 2 is read; the row exponents of tile i are in LDS
      if (i + 2 < ntiles) issue(i + 2);
      if (i == ntiles) continue;

      // ---- scores of tokens 32s + 16h + (0..15) ----
      // The fp4 A operand is 16 bytes; the upper half of its register tuple
      // is not read, so it is left undefined rather than zeroed.
      f32x4 sacc[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sacc[h][0] = sacc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < 5; ++K) {
          const fp8x32 ka = fp4_operand(kc[h][K]);
          sacc[h][0] = mfma_fp4_fp8(ka, K < 4 ? qh[K] : rh, sacc[h][0], sa[h][K]);
          if constexpr (!Q1) sacc[h][1] = mfma_fp4_fp8(ka, K < 4 ? ql[K] : rl, sacc[h][1], sa[h][K]);
        }
      }

      // ---- softmax: x[h][i] is token 32s + 16h + 4g + i of head r16 ----
      // y = x + E - 127 is the log2 size of the token's weight times its row
      // scale 2^(E - 127), which the e4m3 V rows leave out; the block's
      // weights are written relative to its largest y, F = floor(max y)
      // (weight_block_scale).  With cw = floor(max x), u = 2^(x - cw) is the
      // token's share of this wave's weight sum and its stored weight is
      // 2^(y - F + 7) = u 2^(E - 120 - F + cw), both exact powers of two away.
      const int tok0 = item.tok_begin + i * kXTile;
      i32x4 ev[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) ev[h] = *reinterpret_cast<const i32x4*>(&sh.erow[32 * s + 16 * h + 4 * g]);
      float x[2][4];
      float tmax = kNegInf, ymax = kNegInf;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[h][k] = (sacc[h][0][k] + sacc[h][1][k]) * xscale;
          if (tok0 + 32 * s + 16 * h + 4 * g + k > tok_last) x[h][k] = kNegInf;
          tmax = fmaxf(tmax, x[h][k]);
          ymax = fmaxf(ymax, x[h][k] + (float)(ev[h][k] - 127));
        }
      tmax = xor_max_groups(tmax);
      ymax = xor_max_groups(ymax);
      if (g == 0) {
        sh.red_m[i & 1][r16][s] = tmax;
        sh.red_y[i & 1][r16][s] = ymax;
      }
      const float cw = weight_block_floor(tmax);
      const int kbase = (int)cw - 120 - (int)weight_block_floor(ymax);
      float lsum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float pw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float u = __builtin_amdgcn_exp2f(x[h][k] - cw);
          lsum += u;
          pw[k] = __builtin_ldexpf(u, ev[h][k] + kbase);
        }
        uint32_t ph, pl;
        split_fp8x4(pw[0], pw[1], pw[2], pw[3], ph, pl);
        const int at = pw_off + 16 * p_chunk(r16, 2 * s + h);
        *reinterpret_cast<uint32_t*>(&sh.p[i & 1][0][0][0] + at) = ph;
        *reinterpret_cast<uint32_t*>(&sh.p[i & 1][1][0][0] + at) = pl;
      }
      if (tmax != kNegInf) {
        if (cw > m_s) {
          l_s = (m_s == kNegInf) ? 0.0f : __builtin_ldexpf(l_s, (int)(m_s - cw));
          m_s = cw;
        }
        l_s += __builtin_ldexpf(lsum, (int)(cw - m_s));
      }
    }
    const float l_w = xor_sum_groups(l_s);
    const int lane_f = opaque_lane();
    if (lane_f < 16) {
      fin_l[lane_f][s] = l_w;
      fin_ls[lane_f][s] = m_s;
    }
  } else {
    const int c = wave - 4;
    uint8_t* const vblk = &sh.v[c][0];
    f32x4 o[8];  // O^T[128c + 16v + (columns of lane group g)][head r16]
#pragma unroll
    for (int v = 0; v < 8; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = kNegInf;
    // Reads of this lane for P.V: tr8 read q (0..3) gives tokens tb(q) +
    // (0..7), tb = 16g + 8q (q < 2) or 64 + 16g + 8(q - 2), from rows tb(q) +
    // (r16 >> 1), bytes 8(r16 & 1) .. +7 of chunk v: at voff[q] + 2048 v.
    int voff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      voff[q] = 16 * v_slot((q < 2 ? 16 * g + 8 * q : 64 + 16 * g + 8 * (q - 2)) + (r16 >> 1)) + 8 * (r16 & 1);
    const int pr0 = r16 * kXTile + 16 * p_chunk(r16, g);      // P^T tokens 16g .. +15
    const int pr1 = r16 * kXTile + 16 * p_chunk(r16, 4 + g);  // tokens 64 + 16g .. +15

    // P.V of tile i - 1, first the running maximum and the B scale of k-block
    // g (scoring wave g's tokens) for head r16.
    auto pv_scale = [&](const f32x4& mx, const f32x4& my) -> int {
      const float tile_max = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
      // Every V wave reads the same maxima, so this branch is uniform.
      if (__ballot(tile_max > m_ref + kLazyRescale) != 0) {
        const float m_new = floorf(fmaxf(m_ref, tile_max));
        const float alpha = (m_ref == kNegInf) ? 0.0f : __builtin_ldexpf(1.0f, (int)(m_ref - m_new));
#pragma unroll
        for (int v = 0; v < 8; ++v) o[v] *= alpha;
        m_ref = m_new;
      }
      return weight_block_scale(g == 0 ? my[0] : g == 1 ? my[1] : g == 2 ? my[2] : my[3], m_ref);
    };
    // Block k of row rr of tile i to e4m3, relative to the row's E, by table
    // (exact for blocks within 5 binades of E, nearly all); returns E - e.
    auto convert_block = [&](const u32x4 (&wv)[2][4], const uint32_t (&sd)[2][2], const int (&E)[2], int rr,
                             int k) -> int {
      const int d = E[rr] - (int)((sd[rr][k >> 1] >> (8 * (k & 1))) & 0xFFu);  // >= 0
      uint32_t lut_lo, lut_hi;
      fp4_lut((uint32_t)min(d, 5), lut_lo, lut_hi);
      uint32_t e8[8];  // 32 e4m3 codes: word 2i columns 32k + 8i + {0,2,4,6}, word 2i+1 the odd ones
#pragma unroll
      for (int m = 0; m < 4; ++m) fp4x8_to_fp8_lut(wv[rr][k][m], lut_lo, lut_hi, e8[2 * m], e8[2 * m + 1]);
      uint8_t* const vrow = vblk + 16 * v_slot(lane + 64 * rr);
      *reinterpret_cast<u32x4*>(vrow + kXVChunk * (2 * k)) = u32x4{e8[0], e8[1], e8[2], e8[3]};
      *reinterpret_cast<u32x4*>(vrow + kXVChunk * (2 * k + 1)) = u32x4{e8[4], e8[5], e8[6], e8[7]};
      return d;
    };
    // Blocks further than 5 binades below their row's E, converted again by
    // rounding conversions (exact within 8 binades, rounded to e4m3 beyond).
    auto convert_far = [&](const u32x4 (&wv)[2][4], const uint32_t (&sd)[2][2], const int (&E)[2]) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        uint8_t* const vrow = vblk + 16 * v_slot(lane + 64 * rr);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = max((int)((sd[rr][k >> 1] >> (8 * (k & 1))) & 0xFFu) - E[rr], -126);
          if (j >= -5) continue;
          const float scale = __uint_as_float((uint32_t)(127 + j) << 23);
          uint32_t e8[8];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            uint32_t lo, hi;  // columns 0..3, 4..7
            fp4x8_to_fp8(wv[rr][k][m], scale, lo, hi);
            e8[2 * m] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);      // columns 0, 2, 4, 6
            e8[2 * m + 1] = __builtin_amdgcn_perm(hi, lo, 0x07050301u);  // columns 1, 3, 5, 7
          }
          *reinterpret_cast<u32x4*>(vrow + kXVChunk * (2 * k)) = u32x4{e8[0], e8[1], e8[2], e8[3]};
          *reinterpret_cast<u32x4*>(vrow + kXVChunk * (2 * k + 1)) = u32x4{e8[4], e8[5], e8[6], e8[7]};
        }
      }
    };

    for (int i = 0; i <= ntiles; ++i) {
      lds_barrier();  // tile i everywhere; P of tile i - 1 written
      const bool pv = i >= 1, cv = i < ntiles;
      // Token rows lane and lane + 64 of tile i, column blocks 4c .. 4c + 3
      // (16 code bytes each) and their scales (pairs 2c, 2c + 1).
      u32x4 wv[2][4];
      uint32_t sd[2][2];
      if (cv) {
        const uint8_t* raw = &sh.raw[i & 1][0];
        const uint32_t* sdw = reinterpret_cast<const uint32_t*>(raw + kXFp4Bytes);
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int row = lane + 64 * rr;
#pragma unroll
          for (int k = 0; k < 4; ++k) wv[rr][k] = *reinterpret_cast<const u32x4*>(raw + row * kXRow + 64 * c + 16 * k);
          sd[rr][0] = sdw[kXScalePairs * row + 2 * c];
          sd[rr][1] = sdw[kXScalePairs * row + 2 * c + 1];
        }
      }
      // The operands of P.V for tile i - 1, read together with the above:
      // the block maxima and P^T (this wave's V^T follows below).
      f32x4 mx, my;
      fp8x32 bh, bl;
      if (pv) {
        const int par = (i - 1) & 1;
        mx = *reinterpret_cast<const f32x4*>(&sh.red_m[par][r16][0]);
        my = *reinterpret_cast<const f32x4*>(&sh.red_y[par][r16][0]);
        const uint8_t* pt = &sh.p[par][0][0][0];
        bh = join16(*reinterpret_cast<const u32x4*>(pt + pr0), *reinterpret_cast<const u32x4*>(pt + pr1));
        pt = &sh.p[par][1][0][0];
        bl = join16(*reinterpret_cast<const u32x4*>(pt + pr0), *reinterpret_cast<const u32x4*>(pt + pr1));
      }
      lds_barrier();  // the row exponents of tile i; raw slot i % 2 is read
      // Column tile v of V^T for P.V of tile i - 1, by transposing reads.
      auto read_va = [&](int v) -> fp8x32 {
        fp8x32 va;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vblk + voff[q] + kXVChunk * v));
          va[2 * q] = r2[0];
          va[2 * q + 1] = r2[1];
        }
        return va;
      };
      // Converting tile i is vector work, P.V of tile i - 1 LDS reads and
      // matrix work.  Step j converts block j & 3 of row half j >> 2, which
      // overwrites column tiles 2(j & 3) and 2(j & 3) + 1 of the block: steps
      // 0..3 first read those two tiles of tile i - 1 (a wave's LDS accesses
      // execute in order), and their MFMAs follow the step, the lo halves one
      // step after the hi ones.  So the reads and the matrix unit work while
      // this wave converts.
      if (cv) {
        const int E[2] = {sh.erow[lane], sh.erow[lane + 64]};
        int gap = 0;
        if (pv) {
          const int sb = pv_scale(mx, my);
          fp8x32 va0, va1, vp0, vp1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (j < 4) {
              va0 = read_va(2 * j);
              va1 = read_va(2 * j + 1);
            }
            gap = max(gap, convert_block(wv, sd, E, j >> 2, j & 3));
            __builtin_amdgcn_sched_barrier(0);
            if (j < 4) {
              o[2 * j] = mfma_fp8_k128_sb(va0, bh, o[2 * j], sb);
              o[2 * j + 1] = mfma_fp8_k128_sb(va1, bh, o[2 * j + 1], sb);
            }
            if (j >= 1 && j <= 4) {
              o[2 * j - 2] = mfma_fp8_k128_sb(vp0, bl, o[2 * j - 2], sb);
              o[2 * j - 1] = mfma_fp8_k128_sb(vp1, bl, o[2 * j - 1], sb);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (j < 4) {
              vp0 = va0;
              vp1 = va1;
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) gap = max(gap, convert_block(wv, sd, E, j >> 2, j & 3));
        }
        if (__ballot(gap > 5) != 0) convert_far(wv, sd, E);
      } else if (pv) {
        const int sb = pv_scale(mx, my);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const fp8x32 va = read_va(v);
          o[v] = mfma_fp8_k128_sb(va, bh, o[v], sb);
          o[v] = mfma_fp8_k128_sb(va, bl, o[v], sb);
        }
      }
    }

    // The V blocks hold each group of 8 columns as (0, 2, 4, 6, 1, 3, 5, 7),
    // so lane group g has output columns 8(g >> 1) + 2i + (g & 1) of each
    // column tile; lanes l and l ^ 16 trade two values each to return to
    // columns 4g + i.  Then the output goes to raw slot 0 for all waves.
    const int lane_h = opaque_lane();
    const int partner = (lane_h ^ 16) << 2;
    const bool odd = ((lane_h >> 4) & 1) != 0;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float r0 = __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(odd ? o[v][0] : o[v][2])));
      const float r1 = __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(odd ? o[v][1] : o[v][3])));
      hand[(8 * c + v) * 64 + lane_h] = odd ? f32x4{r0, o[v][2], r1, o[v][3]} : f32x4{o[v][0], r0, o[v][1], r1};
    }
    if (c == 0 && lane_h < 16) fin_m[lane_h] = m_ref;
  }
  lds_barrier();  // the output, the weight sums and the references

  // Lane values for the epilogue are derived afresh here, so that none of
  // them stays live (or spilled) through the tile loop.
  const int tid_e = opaque_tid();
  const int lane_e = tid_e & 63, r16_e = lane_e & 15;

  const float m_ref = fin_m[r16_e];
  const f32x4 lv = *reinterpret_cast<const f32x4*>(&fin_l[r16_e][0]);
  const f32x4 mv = *reinterpret_cast<const f32x4*>(&fin_ls[r16_e][0]);
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (mv[k] != kNegInf) L += __builtin_ldexpf(lv[k], (int)(mv[k] - m_ref));
  // Wave w finishes columns 64w .. 64w + 63: tiles 4(w & 1) .. +3 of V wave w >> 1.
  const int W = wave >> 1, vb = 4 * (wave & 1);
  f32x4 ow[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) ow[v] = hand[(8 * W + vb + v) * 64 + lane_e];
  finish_item<4>(a, item, tid_e, W, vb, lane_e, ow, 1.0f / L, m_ref + __log2f(L));
}

// A workgroup runs one item, or with bins the items of bin blockIdx.x in
// order (see Stage1Args).  Between two items every load and store of the
// first is complete and every wave is past it, so the next may reuse LDS.
template <bool PAGED, bool Q1>
__global__ __launch_bounds__(kXThreads, 1) void mla_stage1_mxfp4(Stage1Args a) {
  __shared__ __attribute__((aligned(16))) Fp4Lds sh;
  int i = a.bins ? a.bins[blockIdx.x] : (int)blockIdx.x;
  const int i_end = a.bins ? a.bins[blockIdx.x + 1] : i + 1;
  while (i < i_end) {
    const WorkItem item = a.uniform_splits
                              ? uniform_item(xcd_block(blockIdx.x, gridDim.x), a.uniform_splits, a.uniform_chunk,
                                             a.uniform_len, a.uniform_base)
                              : a.items[i];
    mxfp4_item<PAGED, Q1>(a, item, sh);
    if (++i == i_end) break;
    wait_loads<0>();
    lds_barrier();
  }
}

}  // namespace

const void* stage1_mxfp4_kernel(bool paged, bool query_e4m3) {
  if (query_e4m3)
    return paged ? reinterpret_cast<const void*>(&mla_stage1_mxfp4<true, true>)
                 : reinterpret_cast<const void*>(&mla_stage1_mxfp4<false, true>);
  return paged ? reinterpret_cast<const void*>(&mla_stage1_mxfp4<true, false>)
               : reinterpret_cast<const void*>(&mla_stage1_mxfp4<false, false>);
}

}  // namespace mla
