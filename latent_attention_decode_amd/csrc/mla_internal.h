// Internal interface between the host library (mla_decode.cpp) and the HIP
// kernels (mla_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace mla {

constexpr int kNumHeads = 16;
constexpr int kQkDim = 576;
constexpr int kVDim = 512;
constexpr int kTile = 32;        // token granularity of the planner's splits
constexpr int kPlanTile = 128;   // tokens per stage-1 tile (fp8); items are whole tiles
constexpr int kWaves = 4;        // waves per stage-1 workgroup
constexpr int kStage1Threads = 64 * kWaves;
constexpr int kStage1ThreadsMxfp4 = 512;  // the MXFP4 split kernel runs eight waves
// Page ids of one item that the fp8 / MXFP4 split kernels stage in LDS (what
// the rest of their LDS leaves); the planner keeps paged items within them.
constexpr int kItemPagesFp8 = 2560;
constexpr int kItemPagesFp8Pair = 1536;  // the fp8 kernel that runs pairs of query rows
constexpr int kItemPagesMxfp4 = 1024;
constexpr int kItemPagesBf16 = 2048;  // the bf16 kernel's LDS ring leaves room for this many
constexpr int kMergeThreads = 256;  // two float4 of one head per thread

enum KvFormat : int { kBf16 = 0, kFp8 = 1, kMxfp4 = 2 };

// One stage-1 workgroup's job: tokens [tok_begin, tok_end) of sequence
// `batch` (logical token indices within the sequence).  slot >= 0: write the
// normalised partial (O, lse) to partial slot `slot`; kWhole: the item is the
// whole sequence, write the bf16 output directly; kEmpty (with tok_begin ==
// tok_end): the sequence is empty, write zeros.  For a split sequence,
// merge_job indexes its merge job (and completion counter) and its partials
// are slots [slot_begin, slot_begin + nslots).
struct WorkItem;
__host__ __device__ inline WorkItem uniform_item(int i, int splits, int chunk, int len, int base);

struct WorkItem {
  int32_t batch;
  int32_t tok_begin;
  int32_t tok_end;
  int32_t slot;
  int32_t kv_base;  // kv_indptr[batch] as planned
  int32_t merge_job;
  int32_t slot_begin;
  int32_t nslots;
  static constexpr int32_t kWhole = -1;
  static constexpr int32_t kEmpty = -2;
};
static_assert(sizeof(WorkItem) == 32, "work item layout");

// Item i of a uniform plan (see Stage1Args).
__host__ __device__ inline WorkItem uniform_item(int i, int splits, int chunk, int len, int base) {
  const int b = i / splits;
  const int s = i - b * splits;
  WorkItem w{};
  w.batch = b;
  w.tok_begin = s * chunk;
  w.tok_end = (s + 1) * chunk < len ? (s + 1) * chunk : len;
  w.slot = splits == 1 ? WorkItem::kWhole : i;
  w.kv_base = base + b * len;
  w.merge_job = b;
  w.slot_begin = b * splits;
  w.nslots = splits;
  return w;
}

// Workgroups are handed to the eight XCDs in turn (workgroup x runs on XCD
// x % 8, each XCD with its own L2).  xcd_block(x, n) renumbers a grid of n
// so that each XCD takes one contiguous run of jobs: the splits of a sequence
// then share one L2 (the query is fetched once per XCD), and so do the merge
// jobs of the sequences whose partials that XCD wrote.  A bijection of [0, n).
__host__ __device__ constexpr int xcd_block(int x, int n) {
  return (x & 7) * (n >> 3) + ((x & 7) < (n & 7) ? (x & 7) : (n & 7)) + (x >> 3);
}
constexpr bool xcd_block_is_bijection(int n) {
  int seen = 0;
  for (int x = 0; x < n; ++x) {
    const int y = xcd_block(x, n);
    if (y < 0 || y >= n) return false;
    for (int z = 0; z < x; ++z)
      if (xcd_block(z, n) == y) return false;
    ++seen;
  }
  return seen == n;
}
static_assert(xcd_block_is_bijection(1) && xcd_block_is_bijection(7) && xcd_block_is_bijection(64) &&
                  xcd_block_is_bijection(131) && xcd_block_is_bijection(256),
              "xcd_block");

// One merge job: the partials of sequence `batch` are slots
// [slot_begin, slot_begin + nslots), nslots >= 2.
struct MergeSeq {
  int32_t batch;
  int32_t slot_begin;
  int32_t nslots;
  int32_t pad;
};

struct Stage1Args {
  const uint16_t* q;            // bf16 [batch, 16, 576]
  const uint8_t* kv;            // cache rows
  const uint8_t* kv_mx_scales;  // MXFP4 e8m0 [rows, stride]
  const float* kv_scale;        // FP8 per-tensor scale (device scalar)
  int64_t scale_stride;
  const int32_t* kv_indptr;
  const int32_t* page_indices;
  int page_shift;               // log2(page_size); 0 = contiguous
  const WorkItem* items;
  float* part_o;                // [slots, 16, 512]
  float* part_lse;              // [slots, 16], log2 domain
  uint16_t* out;                // bf16 [batch, 16, 512]
  float score_scale;            // sm_scale * log2(e)
  // Uniform plan (every sequence of length uniform_len, contiguous cache,
  // cut into uniform_splits items of uniform_chunk tokens, in order):
  // item i is computed, not loaded.  uniform_splits == 0: use `items`.
  int uniform_splits;
  int uniform_chunk;
  int uniform_len;
  int uniform_base;             // kv_indptr[0]
  // Non-null: the split kernel merges the partials itself.  counters[j] counts
  // the finished items of merge job j (zero between calls); the item that
  // finishes last reads the other partials of its sequence and writes the
  // output, so no merge kernel runs.
  int* counters;
  // Non-null (every split kernel but the MXFP4 one for odd scale addresses):
  // workgroup k runs items
  // bins[k] .. bins[k + 1] - 1, one after the other; null: workgroup k runs
  // item k.  The bins of a ragged batch carry about equal work.
  const int32_t* bins;
  // Host side only: launch the split kernel's variant that takes the query as
  // one e4m3 code per element (fp8 and MXFP4 split kernels).
  int query_e4m3;
  // Partials for the merge kernel as bf16 (fp8 and MXFP4 caches) instead of
  // fp32 (bf16 cache): slot s's O at 16 KB s of part_o, the fp32 layout's
  // float4 positions holding four bf16 each.  The merge inside the split
  // kernel always keeps fp32.
  int part_bf16;
};

struct MergeArgs {
  const MergeSeq* work;         // the sequences with >= 2 partials
  int uniform_nslots;           // > 0: merge job m is sequence m, slots [m n, m n + n)
  int part_bf16;                // the partials' O is bf16 (see Stage1Args)
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
};

// Largest number of splits of one sequence that a split kernel merges itself
// (the last item reads the other nslots - 1 partials in groups of four).
constexpr int kFusedMergeMaxSlots = 12;

// Size of the device array that the allocation-free run entry point uses in
// place of the caller's workspace (mla_kernels.hip): room for 511 partials,
// about twice what one item per compute unit of a 256-CU device needs.
constexpr size_t kScratchBytes = size_t(16) << 20;
// Device address of that array on `device`, which must be the current
// device; looked up once per device and kept.
hipError_t scratch_address(int device, void** ptr);

// The fp8 and MXFP4 split kernels (mla_stage1_fp8.hip, mla_stage1_mxfp4.hip).
// query_e4m3: the variant that takes the query as one e4m3 code per element.
const void* stage1_fp8_kernel(bool paged, bool row_pairs, bool query_e4m3 = false);
const void* stage1_mxfp4_kernel(bool paged, bool query_e4m3 = false);
// Whether launch_stage1 runs the format's own split kernel for these
// arguments (it does for fp8 and bf16 caches; for MXFP4 when the scale array
// and its row stride are 2-byte aligned, else the bf16-decoding kernel takes
// the MXFP4 items one per workgroup).  Only those kernels run bins and can
// merge partials themselves (Stage1Args::bins, Stage1Args::counters).
bool stage1_dedicated(int fmt, const Stage1Args& a);

// Launchers (mla_kernels.hip).  Return the launch status.
// row_pairs: the plan lists pairs of query rows to run together (fp8
// multi-token plans), for the fp8 kernel that does.
hipError_t launch_stage1(int fmt, bool paged, bool row_pairs, const Stage1Args& a, int num_items, hipStream_t s,
                         hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_merge(const MergeArgs& a, int num_merge_seqs, hipStream_t s,
                        hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Workgroups per merge job (column parts): 4 for 32 jobs or more, up to 32
// for fewer, so that a small batch's merge still spreads over many CUs.
int merge_parts(int num_merge_seqs);
// Static resources of a kernel (which: 0 the stage-1 kernel launch_stage1
// picks for `fmt`, `paged`, `row_pairs` and `query_e4m3` with even MXFP4
// scale addresses, 1 the merge).
hipError_t kernel_attributes(int fmt, bool paged, bool row_pairs, bool query_e4m3, int which,
                             hipFuncAttributes* attr);
// Resident stage-1 workgroups per compute unit.
hipError_t stage1_occupancy(int fmt, bool paged, int* blocks_per_cu);

}  // namespace mla
