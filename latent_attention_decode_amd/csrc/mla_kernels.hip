// HIP kernels (gfx950) for single-token multi-head latent attention decode.
//
// Stage 1 (mla_stage1): one 256-thread workgroup per planned work item, i.e. a
// token range of one sequence, streamed in 64-token tiles with an online
// softmax (flash-decoding, as in the split-K kernels of amd-mixed-mla
// submissions 727205 "v25: LEAN" `mla_s1` and 599694 "overhead elimination"
// `_flash_fp8_split_s1`).  The workgroup writes the normalised partial plus its
// log-sum-exp or, when the item is the whole sequence, the bf16 output.
// Stage 2 (mla_merge): per (sequence, head), the log-sum-exp weighted merge of
// the partials (727205 `mla_rd`; 700955 "locked baseline dispatch"
// `reduce_lse_v71`; 599694 `_flash_fp8_split_s2`).
//
// Per 64-token tile:
//   1. every thread loads 16-byte chunks of the tile's cache rows into
//      registers one tile ahead and writes them to LDS -- fp8 codes as stored,
//      bf16 as stored, MXFP4 decoded to bf16 with its block scale (exact);
//   2. wave w scores tokens 16w..16w+15 against the 16 heads:
//      S^T[token, head] = K Q^T on v_mfma_f32_16x16x32_bf16, A = cache rows
//      (fp8 decoded to bf16 in registers, exact), B = the query, held in
//      registers for the whole item.  The 576-long contraction runs in a
//      permuted column order (any order common to both operands is valid) so
//      that one 16-byte LDS read feeds two MFMA steps;
//   3. the waves exchange their tile maxima and bf16 probabilities through
//      LDS.  The softmax runs in the log2 domain with a lazy shared maximum:
//      it only moves (and O and the sums are rescaled) when a tile maximum
//      passes it by more than 8, which bounds every weight by 2^8 and keeps the
//      result exact;
//   4. wave w accumulates output columns 128w..128w+127 over the 64 tokens:
//      O^T[dim, head] += V^T P^T on the same MFMA.  The score registers of the
//      two waves that scored a 32-token step are the B operand as they are
//      (the token order inside the step is chosen to match), and V^T comes
//      from the LDS rows through the gfx950 transposing reads
//      ds_read_b64_tr_b8 (fp8) / ds_read_b64_tr_b16 (bf16).
// Everything accumulates in fp32; the fp8 per-tensor scale is folded into the
// score scale and the final normalisation.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyRescale = 8.0f;  // log2 headroom before O is rescaled

// ---------------------------------------------------------------------------
// format traits
// ---------------------------------------------------------------------------
template <int F> struct Traits;
template <> struct Traits<kFp8> {
  static constexpr int kRowBytes = 576;  // stored row
  static constexpr int kLdsPitch = 592;  // LDS row pitch (fp8 codes + 16 B)
  static constexpr bool kLdsFp8 = true;
  static constexpr int kBuffers = 2;     // LDS tile buffers (double-buffered)
  static constexpr bool kPrefetch = true;  // next tile's loads in flight during compute
};
template <> struct Traits<kBf16> {
  static constexpr int kRowBytes = 1152;
  static constexpr int kLdsPitch = 1168;  // bf16 elements + 16 B
  static constexpr bool kLdsFp8 = false;
  static constexpr int kBuffers = 1;
  static constexpr bool kPrefetch = false;  // a bf16 tile is 72 registers per lane
};
template <> struct Traits<kMxfp4> {
  static constexpr int kRowBytes = 288;   // e2m1 nibbles; scales live apart
  static constexpr int kLdsPitch = 1168;  // decoded to bf16 in LDS
  static constexpr bool kLdsFp8 = false;
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
  // Each group of 16 rows sits 64 B further on than the one before, so that
  // the transposing reads of an fp8 V step (rows 4g..4g+3 and 16+4g..16+4g+3
  // together) fall on distinct banks.
  static constexpr int kBytes = kTileTokens * Traits<F>::kLdsPitch + (kTileTokens / 16) * 64;
  __host__ __device__ static constexpr int row_offset(int r) {
    return r * Traits<F>::kLdsPitch + (r >> 4) * 64;
  }
};

// bytes one LDS row holds: stored row, or the decoded bf16 row for MXFP4
template <int F> constexpr int kLdsRowBytes = Traits<F>::kLdsFp8 ? kQkDim : 2 * kQkDim;

template <int F> constexpr bool rows_disjoint() {
  for (int r = 0; r + 1 < kTileTokens; ++r)
    if (Tile<F>::row_offset(r) + kLdsRowBytes<F> > Tile<F>::row_offset(r + 1)) return false;
  return Tile<F>::row_offset(kTileTokens - 1) + kLdsRowBytes<F> <= Tile<F>::kBytes;
}
static_assert(rows_disjoint<kFp8>() && rows_disjoint<kBf16>() && rows_disjoint<kMxfp4>(),
              "LDS tile rows overlap");

static_assert(Tile<kFp8>::kChunks == 9 && Tile<kBf16>::kChunks == 18 && Tile<kMxfp4>::kChunks == 5,
              "tile chunking");

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

// 8 fp8 (e4m3fn) codes -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;  // round to nearest even
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float xor_max_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ float xor_sum_groups(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
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
        d[j] = *reinterpret_cast<const u32x4*>(base + j * (16 * kStage1Threads));
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
        d[j] = *reinterpret_cast<const u32x4*>(a.kv + (int64_t)row * kRB + cc * 16);
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
// LDS: tile buffer(s), the bf16 P^T fragments of the four waves, and the
// per-wave tile maxima.
template <int F>
struct Stage1Lds {
  uint8_t tile[Traits<F>::kBuffers][Tile<F>::kBytes];
  uint2 p[kWaves][64];           // 4 bf16 probabilities per lane
  float tmax[kWaves][kNumHeads];
  float lsum[kWaves][kNumHeads];
};

template <int F, bool PAGED>
__global__ __launch_bounds__(kStage1Threads, 2) void mla_stage1(Stage1Args a) {
  __shared__ __attribute__((aligned(16))) Stage1Lds<F> sh;
  constexpr int NB = Traits<F>::kBuffers;

  const WorkItem item = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;  // MFMA row/column index of this lane
  const int g = lane >> 4;    // MFMA k-group of this lane
  const int b = item.batch;
  const int tok_last = item.tok_end - 1;
  const int ntiles = (item.tok_end - item.tok_begin + kTileTokens - 1) / kTileTokens;
  const int64_t seq_base = a.kv_indptr[b];  // first row, or first page slot

  float vscale = 1.0f;
  float xscale = a.score_scale;
  if constexpr (F == kFp8) {
    const float s = *a.kv_scale;
    vscale = s;
    xscale *= s;
  }

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
  const int k_off = Tile<F>::row_offset(16 * wave + r16) + (Traits<F>::kLdsFp8 ? 16 * g : 32 * g);
  const int dv0 = 128 * wave;  // first output column of this wave
  int v_off_lo, v_off_hi = 0;
  if constexpr (Traits<F>::kLdsFp8) {
    // ds_read_b64_tr_b8: lane pair (2e, 2e+1) names row e of an 8 x 16-byte
    // block (8 bytes each); lane i receives byte i of each of the 8 rows.
    v_off_lo = Tile<F>::row_offset(pv_token(g, r16 >> 1)) + (r16 & 1) * 8 + dv0;
  } else {
    // ds_read_b64_tr_b16: lane quad (4e..4e+3) names row e of a 4 x 16-element
    // block (4 elements each); lane i receives element i of each of the 4 rows.
    v_off_lo = Tile<F>::row_offset(pv_token(g, r16 >> 2)) + (r16 & 3) * 8 + 2 * dv0;
    v_off_hi = Tile<F>::row_offset(pv_token(g, 4 + (r16 >> 2))) + (r16 & 3) * 8 + 2 * dv0;
  }

  TileRegs<F, PAGED> regs;
  regs.issue(a, seq_base, item.tok_begin, tok_last, tid);
  regs.store(sh.tile[0], tid);
  if (Traits<F>::kPrefetch && ntiles > 1)
    regs.issue(a, seq_base, item.tok_begin + kTileTokens, tok_last, tid);
  __syncthreads();

  for (int n = 0; n < ntiles; ++n) {
    const int tok0 = item.tok_begin + n * kTileTokens;
    const uint8_t* cur = sh.tile[NB == 2 ? (n & 1) : 0];

    // ---- scores S^T for tokens 16*wave .. +15 of the tile ----
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = sa;
    {
      const uint8_t* kr = cur + k_off;
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        bf16x8 kl, kh;
        if constexpr (Traits<F>::kLdsFp8) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(kr + 64 * j);
          kl = fp8x8_to_bf16(w[0], w[1]);
          kh = fp8x8_to_bf16(w[2], w[3]);
        } else {
          const bf16x8* p = reinterpret_cast<const bf16x8*>(kr + 128 * j);
          kl = p[0];
          kh = p[1];
        }
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qf[2 * j], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qf[2 * j + 1], sb, 0, 0, 0);
      }
    }
    float x[4];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (sa[i] + sb[i]) * xscale;
      if (tok0 + 16 * wave + 4 * g + i > tok_last) x[i] = kNegInf;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = xor_max_groups(tmax);
    if (g == 0) sh.tmax[wave][r16] = tmax;
    float p[4];
    {
      const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mr);
      sh.p[wave][lane] = uint2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    }
    __syncthreads();  // scores, maxima and P of all waves are in LDS

    if constexpr (NB == 2) {
      // the other buffer's last readers finished before this barrier
      if (n + 1 < ntiles) {
        regs.store(sh.tile[(n + 1) & 1], tid);
        if (n + 2 < ntiles) regs.issue(a, seq_base, tok0 + 2 * kTileTokens, tok_last, tid);
      }
    }

    // ---- lazy rescale: only when a tile max passes m_ref + 8 ----
    float tile_max = sh.tmax[0][r16];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) tile_max = fmaxf(tile_max, sh.tmax[w][r16]);
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
      __syncthreads();  // everyone has read the old maxima
      sh.p[wave][lane] = uint2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      __syncthreads();
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
        bf16x8 va;
        if constexpr (Traits<F>::kLdsFp8) {
          const i32x2 raw =
              __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vb + v_off_lo + 16 * v));
          va = fp8x8_to_bf16((uint32_t)raw[0], (uint32_t)raw[1]);
        } else {
          const i16x4 lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off_lo + 32 * v));
          const i16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + v_off_hi + 32 * v));
          const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
          const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
          va = bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
        }
        o[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pt, o[v], 0, 0, 0);
      }
    }
    __syncthreads();  // P, maxima (and a single tile buffer) are free again

    if constexpr (NB == 1) {
      if (n + 1 < ntiles) {
        if (!Traits<F>::kPrefetch) regs.issue(a, seq_base, tok0 + kTileTokens, tok_last, tid);
        regs.store(sh.tile[0], tid);
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
  const float f = vscale / L;
  if (item.slot < 0) {
    uint16_t* dst = a.out + ((int64_t)b * kNumHeads + r16) * kVDim + dv0 + 4 * g;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f32x4 val = o[v] * f;
      *reinterpret_cast<uint2*>(dst + 16 * v) =
          uint2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
    }
  } else {
    float* dst = a.part_o + ((int64_t)item.slot * kNumHeads + r16) * kVDim + dv0 + 4 * g;
#pragma unroll
    for (int v = 0; v < 8; ++v) *reinterpret_cast<f32x4*>(dst + 16 * v) = o[v] * f;
    if (tid < kNumHeads) a.part_lse[(int64_t)item.slot * kNumHeads + tid] = m_ref + __log2f(L);
  }
}

// ---------------------------------------------------------------------------
// stage 2: log-sum-exp merge of the partials, one workgroup per (seq, head)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMergeThreads) void mla_merge(MergeArgs a) {
  const int b = blockIdx.x / kNumHeads;
  const int h = blockIdx.x % kNumHeads;
  const int d = threadIdx.x * 4;
  const SeqInfo info = a.seqs[b];
  if (info.nslots < 0) return;  // written by stage 1
  uint16_t* dst = a.out + ((int64_t)b * kNumHeads + h) * kVDim + d;
  if (info.nslots == 0) {
    *reinterpret_cast<uint2*>(dst) = uint2{0u, 0u};
    return;
  }
  const float* lse = a.part_lse + (int64_t)info.slot_begin * kNumHeads + h;
  float M = kNegInf;
  for (int s = 0; s < info.nslots; ++s) M = fmaxf(M, lse[s * kNumHeads]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  for (int s = 0; s < info.nslots; ++s) {
    const float w = __builtin_amdgcn_exp2f(lse[s * kNumHeads] - M);
    const f32x4 po = *reinterpret_cast<const f32x4*>(
        a.part_o + ((int64_t)(info.slot_begin + s) * kNumHeads + h) * kVDim + d);
    acc += w * po;
    W += w;
  }
  const float inv = 1.0f / W;
  uint2 packed;
  packed.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  packed.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(dst) = packed;
}

template <int F, bool P>
const void* stage1_fn() {
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

hipError_t launch_stage1(int fmt, bool paged, const Stage1Args& a, int num_items, hipStream_t s) {
  const void* fn = pick_stage1(fmt, paged);
  if (!fn) return hipErrorInvalidValue;
  Stage1Args args = a;
  void* params[] = {&args};
  return hipLaunchKernel(fn, dim3(num_items), dim3(kStage1Threads), params, 0, s);
}

hipError_t launch_merge(const MergeArgs& a, int batch, hipStream_t s) {
  MergeArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mla_merge), dim3(batch * kNumHeads),
                         dim3(kMergeThreads), params, 0, s);
}

hipError_t kernel_attributes(int fmt, bool paged, int which, hipFuncAttributes* attr) {
  const void* fn = which == 0 ? pick_stage1(fmt, paged) : reinterpret_cast<const void*>(&mla_merge);
  if (!fn) return hipErrorInvalidValue;
  return hipFuncGetAttributes(attr, fn);
}

hipError_t stage1_occupancy(int fmt, bool paged, int* blocks_per_cu) {
  const void* fn = pick_stage1(fmt, paged);
  if (!fn) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kStage1Threads, 0);
}

}  // namespace mla
