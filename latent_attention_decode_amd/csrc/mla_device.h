// Device helpers shared by the gfx950 decode kernels: vector types, the
// LDS-only workgroup barrier, cross-group reductions, the partial-output
// layout, cache-to-LDS (LDS-DMA) loads and the fp8 / MX matrix-instruction
// wrappers.  Included by the kernel translation units only.
#ifndef MLA_DEVICE_H
#define MLA_DEVICE_H

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

// Layout of one partial O (a workspace slot, 16 x 512): the float4 that
// lane l of wave w holds for column tile v (heads l % 16, dims
// 128w + 16v + 4(l / 16) .. +3) is float4 number (8w + v) * 64 + l of the
// slot, so that each store instruction of a wave writes 1 KB contiguously
// (512 B with bf16 partials, four bf16 in place of each float4).
constexpr int kSlotFloat4 = kNumHeads * kVDim / 4;

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
  static_assert(N == 1 || N == 2 || N == 4, "group size");
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
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(off[0]), "s"(base), "s"(m0)
                 : "memory", "m0");
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
// One four-byte load, lane l's dword at src to LDS m0 + 4 l.
__device__ __forceinline__ void dma_u32(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
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
// The same with B block scale 2^(sb - 127) (e8m0 in the low byte of sb):
// the lanes of group g give the scale of k-values 32g..32g+31 of their column.
__device__ __forceinline__ f32x4 mfma_fp8_k128_sb(fp8x32 a, fp8x32 b, f32x4 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// Softmax weights on the MX instruction.  The weights of one 32-token k-block
// of a P.V step are written relative to that block's own maximum: with F =
// floor(block maximum) (log2 units), a token of logit x is stored as the e4m3
// hi + lo pair of 2^(x - F + 7), in [0, 256), and the block's B scale
// 2^(F - 7 - m_ref) restores 2^(x - m_ref).  The running maximum m_ref is kept
// integral, so that the scale is an exact power of two and the stored weights
// never depend on it.  Relative to the block's largest weight, the pair is
// exact to about 8 significant bits down to 2^-9 and off by at most 2^-18
// below, whatever the spread of the logits across blocks.
__device__ __forceinline__ float weight_block_floor(float block_max) {
  return block_max == kNegInf ? 0.0f : floorf(block_max);
}
// e8m0 code of that B scale (a block with no valid token has zero weights and
// takes 2^0; a block below 2^-127 of the running maximum is clamped there).
__device__ __forceinline__ int weight_block_scale(float block_max, float m_ref) {
  if (block_max == kNegInf) return 127;
  const int c = 127 + (int)floorf(block_max) - 7 - (int)m_ref;
  return min(max(c, 0), 254);
}

__device__ __forceinline__ fp8x32 join16(u32x4 a, u32x4 b) {
  return fp8x32{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// End of a split-kernel work item.  The lanes of the workgroup together hold
// O^T (unnormalised): this lane has, in o[v], O^T[128W + 16(vb + v) + 4g +
// i][r16] for its 128-column group W and column tiles vb .. vb + NV - 1 of
// it; f = scale / L is the normaliser and lse the item's log2-sum-exp.  The
// item is the whole sequence: write bf16 out.  It is one of several: write
// the partial (and, when a.counters is set, merge the sequence's partials if
// this item finishes last; see Stage1Args).
template <int NV>
__device__ __forceinline__ void finish_item(const Stage1Args& a, const WorkItem& item, int tid, int W, int vb,
                                            int lane, const f32x4 (&o)[NV], float f, float lse) {
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int b = item.batch;
  f32x4 res[NV];  // this lane's normalised output
#pragma unroll
  for (int v = 0; v < NV; ++v) res[v] = o[v] * f;
  if (item.slot >= 0) {
    if (!a.counters) {  // the merge kernel combines the partials
      const int64_t at = (int64_t)item.slot * kSlotFloat4 + 512 * W + lane;  // the layout above
      if (a.part_bf16) {
        uint2* dst = reinterpret_cast<uint2*>(a.part_o) + at;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          dst[64 * (vb + v)] = uint2{pack_bf16x2(res[v][0], res[v][1]), pack_bf16x2(res[v][2], res[v][3])};
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(a.part_o) + at;
#pragma unroll
        for (int v = 0; v < NV; ++v) dst[64 * (vb + v)] = res[v];
      }
      if (W == 0 && vb == 0 && g == 0) a.part_lse[(int64_t)item.slot * kNumHeads + r16] = lse;
      return;
    }

    // Fused merge.  The partial is written with device-scope (relaxed atomic)
    // stores, which go through to the level that all XCDs share, and the
    // workgroup counts itself finished only once they are complete; the other
    // partials are read back with device-scope loads.  That publishes the data
    // without a device-scope release / acquire fence, which would write back
    // or invalidate the whole L2 of the XCD.  The item that finishes last
    // merges; nothing waits on another workgroup.  The ordering rests on how
    // gfx950 executes these instructions (sc1 stores written through and
    // acknowledged before s_waitcnt returns, the counter atomic at the shared
    // level, sc1 loads missing the XCD's L2), not on the language's memory
    // model, under which relaxed operations alone would not order them.
    // Layout of a slot here: float (4v + i) of lane l in column group W at
    // 2048 W + 64 (4v + i) + l, so that each store writes 256 bytes in a row.
    float* pdst = a.part_o + (int64_t)item.slot * (4 * kSlotFloat4) + 2048 * W + lane;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __hip_atomic_store(pdst + 64 * (4 * (vb + v) + i), res[v][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (W == 0 && vb == 0 && g == 0)
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
    f32x4 po[4][NV];  // one group of four partials
    auto load_group = [&](int s0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int sl = item.slot_begin + min(s0 + k, item.nslots - 1);
        float* src = a.part_o + (int64_t)sl * (4 * kSlotFloat4) + 2048 * W + lane;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            po[k][v][i] =
                __hip_atomic_load(src + 64 * (4 * (vb + v) + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    float wsum = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) res[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < kFusedMergeMaxSlots; s0 += 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = s0 + k < item.nslots ? __builtin_amdgcn_exp2f(ls[s0 + k] - M) : 0.0f;
        wsum += w;
#pragma unroll
        for (int v = 0; v < NV; ++v) res[v] += w * po[k][v];
      }
      if (s0 + 4 >= item.nslots) break;
      load_group(s0 + 4);
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int v = 0; v < NV; ++v) res[v] *= inv;
  }
  uint16_t* dst = a.out + ((int64_t)b * kNumHeads + r16) * kVDim + 128 * W + 4 * g;
#pragma unroll
  for (int v = 0; v < NV; ++v)
    *reinterpret_cast<uint2*>(dst + 16 * (vb + v)) =
        uint2{pack_bf16x2(res[v][0], res[v][1]), pack_bf16x2(res[v][2], res[v][3])};
}

}  // namespace
}  // namespace mla

#endif  // MLA_DEVICE_H
