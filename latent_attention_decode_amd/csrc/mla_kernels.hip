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
//   mla_stage1_fp8  fp8 cache: 128-token tiles moved HBM -> LDS by
//                   cache-to-LDS loads; both contractions on fp8 / MX matrix
//                   instructions straight on the cached codes (section below).
//   mla_stage1      bf16 and MXFP4 caches: 64-token tiles staged through
//                   registers, MXFP4 decoded to bf16 exactly on the way into
//                   LDS, both contractions on v_mfma_f32_16x16x32_bf16.
//   mla_merge       per (sequence, quarter of the columns) of the split
//                   sequences, the log-sum-exp weighted merge of the partials
//                   (727205 `mla_rd`; 700955 "locked baseline dispatch"
//                   `reduce_lse_v71`; 599694 `_flash_fp8_split_s2`).
//
// In both stage-1 kernels wave w scores a quarter of the tile's tokens
// against the 16 heads (S^T[token, head] = K Q^T) and accumulates output
// columns 128w..128w+127 over all of the tile's tokens (O^T[dim, head] +=
// V^T P^T, V^T through the gfx950 transposing LDS reads); the softmax runs in
// the log2 domain with a lazy maximum shared by the four waves, which only
// moves (and O and the sums are rescaled) when a tile maximum passes it by
// more than 8, bounding every weight by 2^8 and keeping the result exact.
// Contractions over the 576 columns run in a permuted column order (any order
// common to both operands is valid).  Everything accumulates in fp32; the fp8
// per-tensor scale is folded into the score scale and the final
// normalisation.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
  static constexpr int kBuffers = 1;     // unused: fp8 runs mla_stage1_fp8
  static constexpr bool kPrefetch = false;
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

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four MFMA k-groups
// of one row), with the gfx950 lane-swap instructions: permlane32_swap(x, x)
// gives every lane the value of its own half in one result and of the other
// half in the other, and permlane16_swap does the same for 16-lane rows.
__device__ __forceinline__ float xor_max_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float xor_sum_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Token (within a 32-token P.V step) of element e (0..7) of lane group g.
// Elements 0..3 are the score registers of lane group g of the wave that
// scored the step's first 16 tokens (tokens 4g..4g+3), elements 4..7 those
// of the wave that scored the next 16 (16+4g..16+4g+3).
__device__ __forceinline__ int pv_token(int g, int e) {
  return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4);
}

// Layout of one partial O (a workspace slot, 16 x 512 fp32): the float4 that
// lane l of wave w holds for column tile v (heads l % 16, dims
// 128w + 16v + 4(l / 16) .. +3) is float4 number (8w + v) * 64 + l of the
// slot, so that each store instruction of a wave writes 1 KB contiguously.
constexpr int kSlotFloat4 = kNumHeads * kVDim / 4;
__device__ __forceinline__ void store_partial(float* part_o, int slot, int wave, int lane,
                                              const f32x4 (&o)[8], float f) {
  f32x4* dst = reinterpret_cast<f32x4*>(part_o) + (int64_t)slot * kSlotFloat4 + 8 * 64 * wave + lane;
#pragma unroll
  for (int v = 0; v < 8; ++v) dst[64 * v] = o[v] * f;
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
// workgroup barrier that orders LDS only
// ---------------------------------------------------------------------------
// s_waitcnt immediates (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8.  Waiting on lgkmcnt(0) alone leaves the cache-to-LDS
// loads of later tiles in flight across the barrier.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | (0x7 << 4) | ((lgkm & 0xF) << 8) | (((vm >> 4) & 0x3) << 14);
}
constexpr int kWaitLgkm0 = waitcnt_imm(63, 0);

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's LDS reads/writes are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


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
template <int F, bool PAGED>
struct Stage1Lds {
  uint2 p[kWaves][64];               // 4 bf16 probabilities per lane
  f32x4 tmax[kWaves][kNumHeads];     // [wave][head][lane group] tile maxima
  float lsum[kWaves][kNumHeads];
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
}

template <int F, bool PAGED>
__global__ __launch_bounds__(kStage1Threads, 2) void mla_stage1(Stage1Args a) {
  __shared__ __attribute__((aligned(16))) Stage1Tiles<F> tiles;
  __shared__ __attribute__((aligned(16))) Stage1Lds<F, PAGED> sh;

  const WorkItem item = a.uniform_splits
                            ? uniform_item(xcd_block(blockIdx.x, gridDim.x), a.uniform_splits, a.uniform_chunk,
                                           a.uniform_len, a.uniform_base)
                            : a.items[blockIdx.x];
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

  {
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
  const float f = vscale / L;
  if (item.slot < 0) {
    uint16_t* dst = a.out + ((int64_t)b * kNumHeads + r16) * kVDim + dv0 + 4 * g;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f32x4 val = o[v] * f;
      *reinterpret_cast<uint2*>(dst + 16 * v) =
          uint2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
    }
    return;
  }
  store_partial(a.part_o, item.slot, wave, lane, o, f);
  if (tid < kNumHeads) a.part_lse[(int64_t)item.slot * kNumHeads + tid] = m_ref + __log2f(L);
}

// ---------------------------------------------------------------------------
// stage 1, fp8 cache: cooperative 128-token tiles streamed into LDS
// ---------------------------------------------------------------------------
// Both contractions run straight on the cached e4m3 codes (nothing is
// decoded), on the gfx950 MX matrix instruction v_mfma_scale_f32_16x16x128_
// f8f6f4 (fp8 x fp8, unit block scales), which takes 128 k-values per step,
// and on v_mfma_f32_16x16x32_fp8_fp8 for the 64 rope columns.  The other
// operand is written as a sum of two e4m3 numbers, hi + lo, and each product
// is taken twice:
//   * the query row of head h is first scaled by 2^s_h (max |q| in [128, 256))
//     and split q = hi + lo with hi = e4m3(q) and lo = e4m3(q - hi).  A bf16
//     value has 8 significant bits and hi keeps the leading 4, so the rest fits
//     lo exactly whenever it is a normal e4m3 number (|scaled q| >= 1/4, i.e.
//     every element above 1/1024 of the row maximum; smaller ones are off by at
//     most 2^-10 in scaled units).  2^-s_h is folded into the score scale.
//   * the softmax weights p <= 2^8 (lazy maximum) are split the same way,
//     which keeps about 8 significant bits, as many as a bf16 weight has.
//
// Data movement: every byte of the item's cache rows goes HBM -> LDS by
// cache-to-LDS loads (global_load_lds_dwordx4), in a ring of two 128-token
// tiles, so one tile is in flight while the other is computed; the query
// comes the same way.  A tile is its 128 rows at pitch 576 with no padding,
// 72 loads of 1 KB each (wave w issues loads 18w..18w+17).  One load writes
// 64 consecutive 16-byte LDS slots, lane l to slot l, and each lane fetches
// the chunk that belongs there; inside each aligned group of four chunks of a
// row the chunks are stored XOR-permuted by chunk_swz(row), which makes every
// LDS read below free of bank conflicts while each load still covers whole
// 64-byte runs of the rows.
//
// Per tile, with wave w:
//   1. S^T[token, head] = K (Qhi + Qlo)^T for tokens 32w..32w+31 (two 16-token
//      row blocks), all 576 columns; the query stays in registers;
//   2. softmax in the log2 domain with a lazy maximum shared by the four
//      waves: it moves (and O and the sums are rescaled) only when a tile
//      maximum passes it by more than 8, so p <= 2^8; each wave writes its
//      e4m3 hi/lo weights P^T to LDS;
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
constexpr int kMaxItemPages = 512;                  // page ids of one item staged in LDS
static_assert(kCLoads == kWaves * kCLoadsPerWave && kQLoads * 1024 == kQBytes, "load split");
static_assert(kQBytes <= kCTileBytes, "the query is staged in the last ring slot");

// Position of 16-byte chunk c of tile row r inside the row: c ^ chunk_swz(r),
// a permutation inside each aligned group of four chunks.  The LDS has 64
// banks of 4 bytes; with rows at pitch 576, the reads below touch, per phase,
// 16 rows r0..r0+15 of one chunk (score reads, 16 B per lane) or rows
// {32g + 8q + e : e < 8} of two neighbouring g (transposing V reads, 8 B per
// lane), and this permutation puts every phase on distinct banks.
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

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Cache-to-LDS loads: load b of a group writes lane l's 16 bytes to LDS
// m0 + 1024 b + 16 l; the instruction offset 1024 b is added to the global
// address as well, so the per-lane address passed in excludes it.  Written as
// inline assembly so that the compiler does not guard later LDS reads with a
// wait for every such load in flight; the kernel waits for them explicitly.
// The loads carry the non-temporal hint: each byte is read once, and
// streaming reads that do not try to stay in the caches reach a higher HBM
// rate.  They name m0 as clobbered, which they do write; nothing else in
// these kernels keeps a value in m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int N>
__device__ __forceinline__ void dma_group(const uint8_t* base, const uint32_t* off, uint32_t m0) {
  static_assert(N >= 1 && N <= 4, "group size");
  if constexpr (N == 4)
    asm volatile(
        "s_mov_b32 m0, %5\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %4 nt\n\t"
        "global_load_lds_dwordx4 %1, %4 offset:1024 nt\n\t"
        "global_load_lds_dwordx4 %2, %4 offset:2048 nt\n\t"
        "global_load_lds_dwordx4 %3, %4 offset:3072 nt"
        :
        : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(base), "s"(m0)
        : "memory", "m0");
  else if constexpr (N == 2)
    asm volatile(
        "s_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2 nt\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:1024 nt"
        :
        : "v"(off[0]), "v"(off[1]), "s"(base), "s"(m0)
        : "memory", "m0");
  else
    static_assert(N == 4 || N == 2, "group size");
}
template <int N>
__device__ __forceinline__ void dma_group(const uint8_t* const* src, uint32_t m0) {
  if constexpr (N == 4)
    asm volatile(
        "s_mov_b32 m0, %4\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off nt\n\t"
        "global_load_lds_dwordx4 %1, off offset:1024 nt\n\t"
        "global_load_lds_dwordx4 %2, off offset:2048 nt\n\t"
        "global_load_lds_dwordx4 %3, off offset:3072 nt"
        :
        : "v"(src[0]), "v"(src[1]), "v"(src[2]), "v"(src[3]), "s"(m0)
        : "memory", "m0");
  else if constexpr (N == 2)
    asm volatile(
        "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off nt\n\t"
        "global_load_lds_dwordx4 %1, off offset:1024 nt"
        :
        : "v"(src[0]), "v"(src[1]), "s"(m0)
        : "memory", "m0");
  else
    static_assert(N == 4 || N == 2, "group size");
}
// One load, lane l's 16 bytes at src to LDS m0 + 16 l.
__device__ __forceinline__ void dma_one(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's loads are outstanding (loads complete
// in issue order).
template <int N>
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 15));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

struct Fp8Lds {
  uint8_t tile[kCRing][kCTileBytes];       // the ring; slot 1 first holds the query
  uint8_t p[2][kNumHeads][kPRow];          // P^T hi / lo as [head][token]
  float red_m[kNumHeads][kWaves];          // per-wave tile maxima
  float red_l[kNumHeads][kWaves];          // per-wave sums, at the end
  int32_t pages[kMaxItemPages];            // paged: page ids of the item
};

typedef long fp8x8;                                             // 8 e4m3 codes
typedef int fp8x32 __attribute__((ext_vector_type(8)));         // 32 e4m3 codes

__device__ __forceinline__ fp8x8 pack_fp8x8(uint32_t lo, uint32_t hi) {
  return (fp8x8)(((uint64_t)hi << 32) | lo);
}

// Four floats (|x| <= 448) -> e4m3 hi + lo codes (see above), one word each.
__device__ __forceinline__ void split_fp8x4(float x0, float x1, float x2, float x3,
                                            uint32_t& hi, uint32_t& lo) {
  int h = 0, l = 0;
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, h, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - a[0], x1 - a[1], l, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - b[0], x3 - b[1], l, true);
  hi = (uint32_t)h;
  lo = (uint32_t)l;
}

__device__ __forceinline__ f32x4 mfma_fp8(fp8x8 a, fp8x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}
// fp8 x fp8, 128 k-values, block scales 2^0 (e8m0 code 127).
__device__ __forceinline__ f32x4 mfma_fp8_k128(fp8x32 a, fp8x32 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ fp8x32 join16(u32x4 a, u32x4 b) {
  return fp8x32{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <bool PAGED>
__global__ __launch_bounds__(kStage1Threads, 1) void mla_stage1_fp8(Stage1Args a) {
  __shared__ __attribute__((aligned(16))) Fp8Lds sh;

  const WorkItem item = a.uniform_splits
                            ? uniform_item(xcd_block(blockIdx.x, gridDim.x), a.uniform_splits, a.uniform_chunk,
                                           a.uniform_len, a.uniform_base)
                            : a.items[blockIdx.x];
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
  const int ntiles = (item.tok_end - item.tok_begin + kCTile - 1) / kCTile;
  const float kv_scale = *a.kv_scale;

  // The query first (it needs only the sequence id): 18 loads into ring slot
  // 1, load k by wave k % 4.
  {
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (int64_t)b * kNumHeads * kQkDim);
    const uint32_t qm0 = lds_u32(&sh.tile[kCRing - 1][0]);
    for (int k = wave; k < kQLoads; k += kWaves) {
      const int s = 64 * k + lane;
      const int h = s / 72;
      const int c = (s - 72 * h) ^ (h & 7);
      dma_one(qsrc + (h * 72 + c) * 16, qm0 + 1024 * k);
    }
  }
  const int64_t seq_base = item.kv_base;  // kv_indptr[b]: first row, or first page slot

  int page0 = 0;
  if constexpr (PAGED) {
    page0 = item.tok_begin >> a.page_shift;
    const int npages = min(((item.tok_end - 1) >> a.page_shift) - page0 + 1, kMaxItemPages);
    for (int i = tid; i < npages; i += kStage1Threads)
      sh.pages[i] = a.page_indices[seq_base + page0 + i];
    __syncthreads();
  }

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
  // of them (part -1).  Rows past the item's last token fetch that token's row
  // (finite data, masked later).
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
  wait_loads<kCLoadsPerWave>();  // this wave's query loads have landed
  lds_barrier();                 // ... and everyone's

  // Query, B operand of S^T = K Q^T, scaled by 2^s and split into e4m3
  // hi + lo: for 128-column block K (0..3) lane (head r16, group g) holds
  // q[head][128K + 32g .. +32]; for the rope columns, k-step h (0, 1),
  // q[head][512 + 16g + 8h .. +8].
  fp8x32 qh[4], ql[4];
  fp8x8 rh[2], rl[2];
  float xscale;
  {
    const uint8_t* qlds = &sh.tile[kCRing - 1][0];
    bf16x8 qv[18];  // [4K + i]: chunk 16K + 4g + i; [16 + h]: chunk 64 + 2g + h
#pragma unroll
    for (int K = 0; K < 4; ++K)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qv[4 * K + i] = *reinterpret_cast<const bf16x8*>(qlds + 16 * q_slot(r16, 16 * K + 4 * g + i));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      qv[16 + h] = *reinterpret_cast<const bf16x8*>(qlds + 16 * q_slot(r16, 64 + 2 * g + h));
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 18; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qv[k][e]));
    amax = xor_max_groups(amax);
    // 2^s with amax * 2^s in [128, 256)
    const int s = (amax > 0.f) ? 8 - __builtin_amdgcn_frexp_expf(amax) : 0;
    xscale = a.score_scale * kv_scale * __builtin_ldexpf(1.0f, -s);
    uint32_t hw[36], lw[36];  // word 2k + m: elements 4m..4m+3 of qv[k]
#pragma unroll
    for (int k = 0; k < 18; ++k)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        split_fp8x4(__builtin_ldexpf((float)qv[k][4 * m], s), __builtin_ldexpf((float)qv[k][4 * m + 1], s),
                    __builtin_ldexpf((float)qv[k][4 * m + 2], s), __builtin_ldexpf((float)qv[k][4 * m + 3], s),
                    hw[2 * k + m], lw[2 * k + m]);
#pragma unroll
    for (int K = 0; K < 4; ++K)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        qh[K][d] = (int)hw[8 * K + d];
        ql[K][d] = (int)lw[8 * K + d];
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      rh[h] = pack_fp8x8(hw[32 + 2 * h], hw[33 + 2 * h]);
      rl[h] = pack_fp8x8(lw[32 + 2 * h], lw[33 + 2 * h]);
    }
  }

  f32x4 o[8];  // O^T[dim 128w + 16v + 4g + i][head r16]
#pragma unroll
  for (int v = 0; v < 8; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // shared running maximum (log2 units) of head r16
  float l_part = 0.f;     // this lane's share of the running sum

  // LDS byte offsets of this lane's reads within a tile.  Score rows
  // 32w + 16s + r16 have chunk_swz(32w + r16) whatever s; value rows
  // 32g + 8q + (r16 >> 1) have chunk_swz(32g + 8(q & 1) + (r16 >> 1)).
  const int ksw = chunk_swz(32 * wave + r16);
  const int k_row = (32 * wave + r16) * kQkDim;
  const int k_off0 = k_row + 16 * ((2 * g) ^ ksw);      // chunk 8K + 2g
  const int k_off1 = k_row + 16 * ((2 * g + 1) ^ ksw);  // chunk 8K + 2g + 1
  const int k_offr = k_row + 16 * (32 + (g ^ ksw));     // chunk 32 + g
  int v_off[2][4];  // [q % 2][v % 4]; + 64 (v / 4) + 4608 (q & ~1); column chunk 8w + v
#pragma unroll
  for (int qp = 0; qp < 2; ++qp) {
    const int vrow = 32 * g + 8 * qp + (r16 >> 1);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      v_off[qp][c4] = vrow * kQkDim + 16 * (8 * wave + (c4 ^ chunk_swz(vrow))) + 8 * (r16 & 1);
  }
  uint8_t* const p_hi = &sh.p[0][r16][0];
  uint8_t* const p_lo = &sh.p[1][r16][0];

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

    // ---- scores of tokens 32w + 16s + (0..15), s = 0, 1 ----
    f32x4 sacc[2][2];  // [s][hi/lo]
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c) sacc[s][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = 0; K < 4; ++K) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int ro = s * 16 * kQkDim + 128 * K;
        const fp8x32 ka = join16(*reinterpret_cast<const u32x4*>(cur + k_off0 + ro),
                                 *reinterpret_cast<const u32x4*>(cur + k_off1 + ro));
        sacc[s][0] = mfma_fp8_k128(ka, qh[K], sacc[s][0]);
        sacc[s][1] = mfma_fp8_k128(ka, ql[K], sacc[s][1]);
      }
      if (more && (K == 1 || K == 3)) issue(t + 1, K == 1 ? 1 : 2);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(cur + k_offr + s * 16 * kQkDim);
      const fp8x8 ka = pack_fp8x8(w[0], w[1]);
      const fp8x8 kb = pack_fp8x8(w[2], w[3]);
      sacc[s][0] = mfma_fp8(ka, rh[0], sacc[s][0]);
      sacc[s][1] = mfma_fp8(ka, rl[0], sacc[s][1]);
      sacc[s][0] = mfma_fp8(kb, rh[1], sacc[s][0]);
      sacc[s][1] = mfma_fp8(kb, rl[1], sacc[s][1]);
    }

    // ---- softmax: x[s][i] is token 32w + 16s + 4g + i of head r16 ----
    float x[2][4];
    float tmax = kNegInf;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[s][i] = (sacc[s][0][i] + sacc[s][1][i]) * xscale;
        if (tok0 + 32 * wave + 16 * s + 4 * g + i > tok_last) x[s][i] = kNegInf;
        tmax = fmaxf(tmax, x[s][i]);
      }
    tmax = xor_max_groups(tmax);
    if (g == 0) sh.red_m[r16][wave] = tmax;
    float p[2][4];
    uint32_t ph[2], pl[2];
    {
      const float mr = (m_ref == kNegInf) ? 0.0f : m_ref;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[s][i] = __builtin_amdgcn_exp2f(x[s][i] - mr);
        split_fp8x4(p[s][0], p[s][1], p[s][2], p[s][3], ph[s], pl[s]);
        *reinterpret_cast<uint32_t*>(p_hi + 32 * wave + 16 * s + 4 * g) = ph[s];
        *reinterpret_cast<uint32_t*>(p_lo + 32 * wave + 16 * s + 4 * g) = pl[s];
      }
    }
    if (more) issue(t + 1, 3);
    lds_barrier();  // P^T and the tile maxima of all waves

    const f32x4 maxima = *reinterpret_cast<const f32x4*>(&sh.red_m[r16][0]);
    fp8x32 bh = join16(*reinterpret_cast<const u32x4*>(p_hi + 32 * g),
                       *reinterpret_cast<const u32x4*>(p_hi + 32 * g + 16));
    fp8x32 bl = join16(*reinterpret_cast<const u32x4*>(p_lo + 32 * g),
                       *reinterpret_cast<const u32x4*>(p_lo + 32 * g + 16));
    const float tile_max = fmaxf(fmaxf(maxima[0], maxima[1]), fmaxf(maxima[2], maxima[3]));
    // Every wave reads the same maxima, so this branch is uniform.
    if (__ballot(tile_max > m_ref + kLazyRescale) != 0) {
      const float m_new = fmaxf(m_ref, tile_max);
      const float alpha = (m_ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int v = 0; v < 8; ++v) o[v] *= alpha;
      l_part *= alpha;
      m_ref = m_new;
      lds_barrier();  // everyone has read the old P^T
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p[s][i] = __builtin_amdgcn_exp2f(x[s][i] - m_ref);
        split_fp8x4(p[s][0], p[s][1], p[s][2], p[s][3], ph[s], pl[s]);
        *reinterpret_cast<uint32_t*>(p_hi + 32 * wave + 16 * s + 4 * g) = ph[s];
        *reinterpret_cast<uint32_t*>(p_lo + 32 * wave + 16 * s + 4 * g) = pl[s];
      }
      lds_barrier();
      bh = join16(*reinterpret_cast<const u32x4*>(p_hi + 32 * g),
                  *reinterpret_cast<const u32x4*>(p_hi + 32 * g + 16));
      bl = join16(*reinterpret_cast<const u32x4*>(p_lo + 32 * g),
                  *reinterpret_cast<const u32x4*>(p_lo + 32 * g + 16));
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) l_part += (p[s][0] + p[s][1]) + (p[s][2] + p[s][3]);

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
      o[v] = mfma_fp8_k128(va[0], bh, o[v]);
      o[v + 1] = mfma_fp8_k128(va[1], bh, o[v + 1]);
      o[v] = mfma_fp8_k128(va[0], bl, o[v]);
      o[v + 1] = mfma_fp8_k128(va[1], bl, o[v + 1]);
      if (more && v == 2) issue(t + 1, 4);
    }
  }

  // ---- sums over the item; each wave writes its 128 columns ----
  const float l_w = xor_sum_groups(l_part);
  if (g == 0) sh.red_l[r16][wave] = l_w;
  lds_barrier();
  const f32x4 ls = *reinterpret_cast<const f32x4*>(&sh.red_l[r16][0]);
  const float L = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  const float f = kv_scale / L;
  f32x4 res[8];  // this lane's normalised output, O^T[128w + 16v + 4g + i][r16]
#pragma unroll
  for (int v = 0; v < 8; ++v) res[v] = o[v] * f;
  if (item.slot >= 0) {
    const float lse = m_ref + __log2f(L);
    if (!a.counters) {  // the merge kernel combines the partials
      store_partial(a.part_o, item.slot, wave, lane, o, f);
      if (wave == 0 && g == 0) a.part_lse[(int64_t)item.slot * kNumHeads + r16] = lse;
      return;
    }

    // Fused merge.  The partial is written with device-scope (relaxed atomic)
    // stores, which go through to the level that all XCDs share, and the
    // workgroup counts itself finished only once they are complete; the other
    // partials are read back with device-scope loads.  That publishes the data
    // without a device-scope release / acquire fence, which would write back
    // or invalidate the whole L2 of the XCD.  The item that finishes last
    // merges; nothing waits on another workgroup.
    // Layout of a slot here: float (4v + i) of lane l of wave w at
    // 2048 w + 64 (4v + i) + l, so that each store writes 256 bytes in a row.
    float* pdst = a.part_o + (int64_t)item.slot * (4 * kSlotFloat4) + 2048 * wave + lane;
#pragma unroll
    for (int v = 0; v < 8; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __hip_atomic_store(pdst + 64 * (4 * v + i), res[v][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave == 0 && g == 0)
      __hip_atomic_store(a.part_lse + (int64_t)item.slot * kNumHeads + r16, lse, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __shared__ int s_last;
    __syncthreads();
    if (tid == 0) {
      int* cnt = a.counters + item.merge_job;
      const int done = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = done == item.nslots - 1;
      if (s_last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
    }
    __syncthreads();
    if (!s_last) return;
    // out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M), M = max_s lse_s,
    // summed in slot order over all the sequence's partials (this item's own
    // included, as stored), so the result does not depend on which item
    // finished last.  Each lane reads the float4 numbers it stored itself.
    float ls[kFusedMergeMaxSlots];
    f32x4 po[4][8];  // one group of four partials
    auto load_group = [&](int s0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int sl = item.slot_begin + min(s0 + k, item.nslots - 1);
        float* src = a.part_o + (int64_t)sl * (4 * kSlotFloat4) + 2048 * wave + lane;
#pragma unroll
        for (int v = 0; v < 8; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            po[k][v][i] = __hip_atomic_load(src + 64 * (4 * v + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    };
#pragma unroll
    for (int k = 0; k < kFusedMergeMaxSlots; ++k)
      ls[k] = __hip_atomic_load(a.part_lse + (int64_t)(item.slot_begin + min(k, item.nslots - 1)) * kNumHeads + r16,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    load_group(0);  // in flight together with the lse values
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < kFusedMergeMaxSlots; ++k)
      if (k < item.nslots) M = fmaxf(M, ls[k]);
    float W = 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v) res[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < kFusedMergeMaxSlots; s0 += 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = s0 + k < item.nslots ? __builtin_amdgcn_exp2f(ls[s0 + k] - M) : 0.0f;
        W += w;
#pragma unroll
        for (int v = 0; v < 8; ++v) res[v] += w * po[k][v];
      }
      if (s0 + 4 >= item.nslots) break;
      load_group(s0 + 4);
    }
    const float inv = 1.0f / W;
#pragma unroll
    for (int v = 0; v < 8; ++v) res[v] *= inv;
  }
  uint16_t* dst = a.out + ((int64_t)b * kNumHeads + r16) * kVDim + 128 * wave + 4 * g;
#pragma unroll
  for (int v = 0; v < 8; ++v)
    *reinterpret_cast<uint2*>(dst + 16 * v) =
        uint2{pack_bf16x2(res[v][0], res[v][1]), pack_bf16x2(res[v][2], res[v][3])};
}

// ---------------------------------------------------------------------------
// mla_merge: LSE merge of the partials of one sequence,
//   M = max_s lse_s,  out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M)
// (727205 `mla_rd`; 700955 `reduce_lse_v71`; 599694 `_flash_fp8_split_s2`).
// One workgroup per (sequence, quarter of the columns): thread t merges
// float4 numbers t and t + 256 of that quarter of every partial (both of head
// t % 16, see store_partial), reading kMergeBatch partials at a time so that
// their loads are in flight together.
// ---------------------------------------------------------------------------
constexpr int kMergeBatch = 4;

__global__ __launch_bounds__(kMergeThreads) void mla_merge(MergeArgs a) {
  const int job = a.uniform_nslots > 0 ? xcd_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const MergeSeq seq = a.uniform_nslots > 0
                           ? MergeSeq{job >> 2, (job >> 2) * a.uniform_nslots, a.uniform_nslots, 0}
                           : a.work[job >> 2];
  const int quarter = job & 3;
  const int t = threadIdx.x;
  const int h = t & 15;
  const float* lse = a.part_lse + (int64_t)seq.slot_begin * kNumHeads + h;
  const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o) + (int64_t)seq.slot_begin * kSlotFloat4 +
                    512 * quarter + t;
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
      x0[k] = po[(int64_t)s * kSlotFloat4];
      x1[k] = po[(int64_t)s * kSlotFloat4 + 256];
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

template <int F, bool P>
const void* stage1_fn() {
  if constexpr (F == kFp8)
    return reinterpret_cast<const void*>(&mla_stage1_fp8<P>);
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

// With events, the launch records them at the start and the end of the
// kernel itself (hipExtLaunchKernel), so their difference is its duration.
static hipError_t launch(const void* fn, dim3 grid, dim3 block, void** params, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  if (start && stop) return hipExtLaunchKernel(fn, grid, block, params, 0, s, start, stop, 0);
  return hipLaunchKernel(fn, grid, block, params, 0, s);
}

hipError_t launch_stage1(int fmt, bool paged, const Stage1Args& a, int num_items, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  const void* fn = pick_stage1(fmt, paged);
  if (!fn) return hipErrorInvalidValue;
  Stage1Args args = a;
  void* params[] = {&args};
  return launch(fn, dim3(num_items), dim3(kStage1Threads), params, s, start, stop);
}

hipError_t launch_merge(const MergeArgs& a, int num_merge_seqs, hipStream_t s, hipEvent_t start,
                        hipEvent_t stop) {
  MergeArgs args = a;
  void* params[] = {&args};
  return launch(reinterpret_cast<const void*>(&mla_merge), dim3(num_merge_seqs * 4),
                dim3(kMergeThreads), params, s, start, stop);
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
