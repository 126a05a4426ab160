// Host side of libmla_decode.so: argument validation, the split planner and
// the two kernel launches behind the C ABI of include/mla_decode.h.

#include "mla_decode.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "mla_internal.h"

struct mla_decode_s {
  int device = 0;
  int kv_dtype = 0;
  int page_size = 1;
  int page_shift = 0;
  float sm_scale = 0.f;
  std::string last_error;

  // plan
  bool planned = false;
  int batch = 0;
  int num_items = 0;
  int num_slots = 0;
  int max_splits = 0;
  int64_t total_tokens = 0;
  size_t workspace_bytes = 0;
  int num_merge = 0;  // sequences with >= 2 partials
  bool fused_merge = false;  // the split kernel merges them itself (no merge launch)
  int uniform_splits = 0, uniform_chunk = 0, uniform_len = 0, uniform_base = 0;
  int num_bins = 0;  // > 0: binned plan (see PlanOut)
  bool row_pairs = false;  // the fp8 kernel runs pairs of query rows (see PlanOut)
  // Device plan, two buffers used in turn: [num_items] WorkItem, [num_merge]
  // MergeSeq, [num_merge] int32 counters, [num_bins + 1] int32 bin starts.
  // plan() fills the pinned host copy of the other buffer and uploads it on
  // a stream of the handle (no host wait), so a decode loop can re-plan
  // while the previous run is in flight; the first run of a plan waits on
  // its upload (uploaded[]), and a buffer is written again only after the
  // runs that read it (released[], recorded on the last run's stream when
  // the next plan is made).
  void* dev_plan[2] = {nullptr, nullptr};
  size_t dev_plan_bytes[2] = {0, 0};
  void* host_plan[2] = {nullptr, nullptr};
  size_t host_plan_bytes[2] = {0, 0};
  hipEvent_t uploaded[2] = {nullptr, nullptr};
  hipEvent_t released[2] = {nullptr, nullptr};
  bool upload_pending[2] = {false, false};
  bool release_pending[2] = {false, false};
  hipStream_t upload_stream = nullptr;
  int cur = 1;                     // buffer of the current plan
  bool ran_since_plan = false;     // a run has used the current plan
  hipStream_t waited_stream = nullptr;  // a stream that already waits on the current upload
  bool waited = false;
  hipStream_t last_run_stream = nullptr;
  int num_cus = 0;
  int blocks_per_cu = 0;

  // measurement
  bool profiling = false;
  int query_format = MLA_QUERY_EXACT;
  bool events_ready = false;
  bool timed_run = false;
  bool merge_timed = false;
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
};

namespace {

constexpr int kVersion = 1 * 10000 + 5 * 100 + 0;
static_assert(MLA_SCRATCH_BYTES == mla::kScratchBytes, "scratch size in the header");

mla_status fail(mla_decode_t h, mla_status st, const char* fmt, ...) {
  if (h) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    h->last_error = buf;
  }
  return st;
}

// Restores the calling thread's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) return;
    ok = true;
  }
  ~DeviceGuard() {
    if (ok && prev >= 0) (void)hipSetDevice(prev);
  }
};

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// The integer a C caller passed for an enum parameter.  A C caller may pass
// any int, and loading a value outside the enumerators' range as the C++ enum
// type is undefined, so the value is read from its object representation.
template <class E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

size_t slot_bytes() {
  return static_cast<size_t>(mla::kNumHeads) * (mla::kVDim + 1) * sizeof(float);
}

}  // namespace

namespace mla {

// Sequence lengths from the host page table (or token offsets).
static bool seq_lengths(const int32_t* indptr, const int32_t* last, int batch, int page_size,
                        std::vector<int64_t>* lens, std::string* err) {
  lens->resize(batch);
  if (indptr[0] < 0) {
    *err = "kv_indptr[0] is negative";
    return false;
  }
  for (int b = 0; b < batch; ++b) {
    const int64_t n = static_cast<int64_t>(indptr[b + 1]) - indptr[b];
    if (n < 0) {
      *err = "kv_indptr is not non-decreasing at sequence " + std::to_string(b);
      return false;
    }
    if (page_size == 1) {
      (*lens)[b] = n;
    } else if (n == 0) {
      (*lens)[b] = 0;
    } else {
      const int lp = last[b];
      if (lp < 1 || lp > page_size) {
        *err = "kv_last_page_len[" + std::to_string(b) + "] outside [1, page_size]";
        return false;
      }
      (*lens)[b] = (n - 1) * page_size + lp;
    }
    if ((*lens)[b] > INT32_MAX) {
      *err = "sequence too long";
      return false;
    }
  }
  return true;
}

// Query tokens per sequence from qo_indptr (multi-token decode): at least
// none, at most the sequence's length (its query tokens' own rows are in the
// cache), at least one in all.
static bool query_counts(const int32_t* qo_indptr, int batch, const std::vector<int64_t>& lens,
                         std::vector<int32_t>* q, std::string* err) {
  if (qo_indptr[0] != 0) {
    *err = "qo_indptr[0] must be 0";
    return false;
  }
  q->resize(batch);
  for (int b = 0; b < batch; ++b) {
    const int64_t n = static_cast<int64_t>(qo_indptr[b + 1]) - qo_indptr[b];
    if (n < 0) {
      *err = "qo_indptr is not non-decreasing at sequence " + std::to_string(b);
      return false;
    }
    if (n > lens[b]) {
      *err = "sequence " + std::to_string(b) + " has more query tokens than cache tokens";
      return false;
    }
    (*q)[b] = static_cast<int32_t>(n);
  }
  if (qo_indptr[batch] < 1) {
    *err = "no query tokens";
    return false;
  }
  return true;
}

// The split planner.  Items are whole 128-token tiles (the last item of a
// sequence may end mid-tile).  With C compute units holding W workgroups
// each, the auto plan aims at C*W items of equal size for uniform batches (one
// wave of workgroups, nothing idle) and four times as many for ragged ones
// (the dispatcher then balances them as slots free up).  Longer items are
// listed first so the last workgroups to start are short ones; empty
// sequences get an item of their own that writes the zero output.
struct PlanOut {
  std::vector<WorkItem> items;
  std::vector<MergeSeq> merge;
  // Binned plan: workgroup k runs items bins[k] .. bins[k + 1] - 1 (bins has
  // one entry more than there are workgroups); empty: workgroup k runs item k.
  std::vector<int32_t> bins;
  // uniform plan (see Stage1Args): splits per sequence, chunk, length; 0 if not
  int uniform_splits = 0, uniform_chunk = 0, uniform_len = 0;
  int num_slots = 0;
  int max_splits = 0;
  // the items come in pairs of query rows for the fp8 kernel that runs them
  // together (see plan_multi)
  bool row_pairs = false;
};

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Items are whole tiles of the format's split kernel: 128 tokens (fp8 and
// MXFP4 kernels) or 64 (bf16 kernel).  A small batch is cut down to items of
// min_item_tokens, so that it reaches more compute units, with at most
// kMaxAutoSplits items per sequence (the merge kernel spreads a small
// batch's merge over up to 32 workgroups per sequence); bins cut a sequence
// into at most kMaxBinSplits items (merged inside the split kernel when there
// are at most kFusedMergeMaxSlots and the format takes the fused merge, else
// by the merge kernel).  Measured on bs4 x 8192
// fp8: 256 items of one tile 15.8 us a call, 128 of two tiles 14.9; on bs4 x
// 1024 bf16: 64 items of one 64-token tile 10.5 us, 32 of two 11.9.
constexpr int64_t kMaxAutoSplits = 256;
constexpr int64_t kMaxBinSplits = 32;
static int64_t plan_tile(int kv_dtype) { return kv_dtype == MLA_KV_BF16 ? kPlanTile / 2 : kPlanTile; }
static int64_t min_item_tokens(int kv_dtype) { return kv_dtype == MLA_KV_BF16 ? kPlanTile / 2 : 2 * kPlanTile; }
// Page ids of one item that the format's split kernel stages in LDS.
static int64_t item_pages(int kv_dtype) {
  return kv_dtype == MLA_KV_FP8_E4M3 ? kItemPagesFp8 : kv_dtype == MLA_KV_MXFP4 ? kItemPagesMxfp4 : kItemPagesBf16;
}

// Bins for a ragged batch (the split kernels, which run the items of a
// bin one after the other).  One item per workgroup leaves the compute units
// that drew the short items idle while the long ones finish (a quarter of
// the time on lengths spread evenly over 1024..8192); here the sequences,
// longest first, are laid end to end and cut into at most `slots` bins of
// about equal cost, a piece costing its tokens plus a fixed cost for its
// start and finish (measured with wall-clock stamps around the items: about
// 200 tokens of streaming for the fp8 kernel, more for the MXFP4 one, whose
// best value on ragged batches was 288; the bf16 kernel streams half as many
// tokens in the same time, so its fixed cost is about half the fp8 one in
// tokens, 96; 64 to 224 timed within 1 % of each other on ragged bf16
// batches).  A sequence cut across bins becomes
// several items, merged like any split.  No piece is shorter than kMinPiece
// unless its sequence is.
constexpr int64_t kMinPiece = 256;
static int64_t bin_piece_cost(int kv_dtype) {
  return kv_dtype == MLA_KV_MXFP4 ? 288 : kv_dtype == MLA_KV_FP8_E4M3 ? 192 : 96;
}

struct Piece {
  int32_t batch;
  int64_t t0, t1;
};

// x rounded toward zero to a multiple of the power of two `tile` (what
// x / tile * tile gives, without the division).
static_assert((kPlanTile & (kPlanTile - 1)) == 0 && kPlanTile >= 2, "planner tiles are powers of two");
static inline int64_t trunc_tile(int64_t x, int64_t tile) {
  return x >= 0 ? (x & ~(tile - 1)) : -((-x) & ~(tile - 1));
}

// Greedy fill of bins of cost capacity C in stream order; returns the number
// of bins and the largest number of pieces of one sequence.  With `pieces`,
// the pieces in bin order and, in `starts`, each bin's first piece (one more
// entry than there are bins).
static int64_t fill_bins(const std::vector<int64_t>& lens, const std::vector<int32_t>& order, int64_t C,
                         int64_t tile, int64_t max_item, int64_t kPieceCost, std::vector<Piece>* pieces,
                         std::vector<int32_t>* starts, int64_t* max_pieces) {
  int64_t bins = 1, r = C, most = 0;
  if (pieces) {
    pieces->clear();
    starts->assign(1, 0);
  }
  for (int32_t b : order) {
    const int64_t n = lens[b];
    int64_t pos = 0, count = 0;
    while (pos < n) {
      const int64_t rest = n - pos;
      int64_t take;
      if (rest <= max_item && rest + kPieceCost <= r) {
        take = rest;
      } else {
        take = std::min(trunc_tile(r - kPieceCost, tile), max_item);
        if (rest - take < kMinPiece) take = trunc_tile(rest - kMinPiece, tile);
        if (take < kMinPiece) {  // the bin is full
          ++bins;
          r = C;
          if (pieces) starts->push_back(static_cast<int32_t>(pieces->size()));
          continue;
        }
      }
      if (pieces) pieces->push_back(Piece{b, pos, pos + take});
      pos += take;
      r -= take + kPieceCost;
      ++count;
    }
    most = std::max(most, count);
  }
  if (pieces) starts->push_back(static_cast<int32_t>(pieces->size()));
  if (max_pieces) *max_pieces = most;
  return bins;
}

// Whether a batch gets bins, and then the plan.  Returns false (nothing
// written) for batches the one-item-per-workgroup plan serves as well:
// equal lengths, or too few tokens per slot for a bin to hold more than one
// piece of the minimum size.
static bool plan_bins(const std::vector<int64_t>& lens, const int32_t* indptr, int64_t slots, int64_t tile,
                      int64_t max_item, int64_t max_splits, int64_t kPieceCost, PlanOut* out) {
  const int batch = static_cast<int>(lens.size());
  int64_t total = 0, longest = 0;
  bool equal = true;
  for (int64_t n : lens) {
    total += n;
    longest = std::max(longest, n);
    equal = equal && n == lens[0];
  }
  const int64_t c_min = kPieceCost + 2 * kMinPiece;
  if (equal || slots < 1 || (total + slots - 1) / slots < c_min || max_item < 2 * kMinPiece) return false;
  // longest first, ties in sequence order (the order of a stable sort)
  std::vector<int32_t> order;
  order.reserve(batch);
  for (int b = 0; b < batch; ++b)
    if (lens[b]) order.push_back(b);
  std::sort(order.begin(), order.end(),
            [&](int32_t x, int32_t y) { return lens[x] > lens[y] || (lens[x] == lens[y] && x < y); });

  // the least capacity that fits the batch into `slots` bins, no sequence in
  // more than max_splits pieces (the fill is monotone in C)
  auto fits = [&](int64_t C) {
    int64_t most = 0;
    return fill_bins(lens, order, C, tile, max_item, kPieceCost, nullptr, nullptr, &most) <= slots &&
           most <= max_splits;
  };
  // every sequence has at least one piece, each costing kPieceCost beyond
  // its tokens, so no capacity below lo fits
  const int64_t nonempty = static_cast<int64_t>(order.size());
  int64_t lo = std::max((total + kPieceCost * nonempty + slots - 1) / slots, c_min);
  // one bin holds the whole batch beyond this capacity; if that still
  // splits a sequence too often (page staging), bins do not apply
  const int64_t one_bin = total + kPieceCost * (batch + total / kMinPiece + 2) + c_min;
  // the answer is usually within a quarter above lo: try that first
  int64_t hi = lo + lo / 4;
  if (fits(hi)) {
    // search [lo, hi]
  } else {
    lo = hi + 1;
    hi = 2 * hi;
    while (!fits(hi)) {
      if (hi > one_bin) return false;
      lo = hi + 1;
      hi *= 2;
    }
  }
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (fits(mid))
      hi = mid;
    else
      lo = mid + 1;
  }
  std::vector<Piece> pieces;
  std::vector<int32_t> starts;
  fill_bins(lens, order, lo, tile, max_item, kPieceCost, &pieces, &starts, nullptr);
  size_t nb = starts.size() - 1;  // bins, the last ones possibly empty
  while (nb > 0 && starts[nb - 1] == starts[nb]) --nb;

  // slots: the pieces of a sequence, in stream order
  std::vector<int32_t> npieces(batch, 0), first_slot(batch, 0), job(batch, -1), seen(batch, 0);
  for (const Piece& p : pieces) ++npieces[p.batch];
  out->items.clear();
  out->merge.clear();
  out->bins.clear();
  out->num_slots = 0;
  out->max_splits = 0;
  for (int b = 0; b < batch; ++b) {
    out->max_splits = std::max<int>(out->max_splits, npieces[b]);
    if (npieces[b] < 2) continue;
    job[b] = static_cast<int32_t>(out->merge.size());
    first_slot[b] = out->num_slots;
    out->merge.push_back(MergeSeq{b, out->num_slots, npieces[b], 0});
    out->num_slots += npieces[b];
  }
  // empty sequences: their zero-output items go to the bins in turn
  std::vector<int32_t> empties;
  for (int b = 0; b < batch; ++b)
    if (!lens[b]) empties.push_back(b);
  const size_t nbins = std::max<size_t>(nb, 1);
  out->items.reserve(pieces.size() + empties.size());
  out->bins.reserve(nbins + 1);
  for (size_t k = 0; k < nbins; ++k) {
    out->bins.push_back(static_cast<int32_t>(out->items.size()));
    if (k < nb)
      for (int32_t i = starts[k]; i < starts[k + 1]; ++i) {
        const Piece& p = pieces[i];
        const int b = p.batch;
        const bool whole = npieces[b] == 1;
        out->items.push_back(WorkItem{b, static_cast<int32_t>(p.t0), static_cast<int32_t>(p.t1),
                                      whole ? WorkItem::kWhole : first_slot[b] + seen[b]++, indptr[b],
                                      whole ? -1 : job[b], whole ? 0 : first_slot[b],
                                      whole ? 0 : npieces[b]});
      }
    for (size_t e = k; e < empties.size(); e += nbins)
      out->items.push_back(WorkItem{empties[e], 0, 0, WorkItem::kEmpty, indptr[empties[e]], -1, 0, 0});
  }
  out->bins.push_back(static_cast<int32_t>(out->items.size()));
  out->uniform_splits = out->uniform_chunk = out->uniform_len = 0;
  return true;
}

static void plan_items(const std::vector<int64_t>& lens, const int32_t* indptr, int split_override,
                       int num_cus, int blocks_per_cu, int page_size, int64_t tile, int64_t min_item,
                       int64_t max_pages, int64_t bin_cost, PlanOut* out) {
  const int batch = static_cast<int>(lens.size());
  int64_t total = 0;
  for (int64_t n : lens) total += n;
  // A paged item's page ids are staged in LDS: at most max_pages of them
  // (an item's first and last page may be partial).
  const int64_t max_item = page_size > 1 && max_pages < INT64_MAX / 2
                               ? (max_pages - 2) * static_cast<int64_t>(page_size) / tile * tile
                               : INT64_MAX;
  out->bins.clear();
  if (bin_cost > 0 && split_override == 0 &&
      plan_bins(lens, indptr, static_cast<int64_t>(num_cus) * std::max(blocks_per_cu, 1), tile, max_item,
                kMaxBinSplits, bin_cost, out))
    return;
  std::vector<int64_t> chunk(batch, 0);
  if (split_override > 0) {
    for (int b = 0; b < batch; ++b) {
      if (!lens[b]) continue;
      const int64_t ns = std::min<int64_t>(split_override, (lens[b] + kTile - 1) / kTile);
      chunk[b] = round_up((lens[b] + ns - 1) / ns, kTile);
    }
  } else if (total > 0) {
    // About one item per resident workgroup slot, ragged batches included:
    // every item start and end costs the streaming a few microseconds, which
    // outweighs the finer load balance of more, shorter items (measured on
    // the ragged bs256 batch: 1, 2, 4 items per slot -> 151, 156, 160 us).
    const int64_t slots = static_cast<int64_t>(num_cus) * std::max(blocks_per_cu, 1);
    const int64_t target = slots;
    const int64_t c = std::max<int64_t>(min_item, round_up((total + target - 1) / target, tile));
    for (int b = 0; b < batch; ++b) {
      if (!lens[b]) continue;
      // bound the partials one merge workgroup reads
      const int64_t ns = std::min<int64_t>((lens[b] + c - 1) / c, kMaxAutoSplits);
      // even out the pieces of this sequence
      chunk[b] = round_up((lens[b] + ns - 1) / ns, tile);
    }
  }
  out->items.clear();
  out->merge.clear();
  out->num_slots = 0;
  out->max_splits = 0;
  for (int b = 0; b < batch; ++b) {
    if (!lens[b]) {
      out->items.push_back(WorkItem{b, 0, 0, WorkItem::kEmpty, indptr[b], -1, 0, 0});
      continue;
    }
    if (chunk[b] > max_item) chunk[b] = max_item;
    const int64_t ns = (lens[b] + chunk[b] - 1) / chunk[b];
    out->max_splits = std::max<int>(out->max_splits, static_cast<int>(ns));
    if (ns == 1) {
      out->items.push_back(
          WorkItem{b, 0, static_cast<int32_t>(lens[b]), WorkItem::kWhole, indptr[b], -1, 0, 0});
      continue;
    }
    const int32_t job = static_cast<int32_t>(out->merge.size());
    out->merge.push_back(MergeSeq{b, out->num_slots, static_cast<int32_t>(ns), 0});
    for (int64_t s = 0; s < ns; ++s) {
      const int64_t t0 = s * chunk[b];
      const int64_t t1 = std::min(lens[b], t0 + chunk[b]);
      out->items.push_back(WorkItem{b, static_cast<int32_t>(t0), static_cast<int32_t>(t1),
                                    out->num_slots + static_cast<int32_t>(s), indptr[b], job,
                                    out->num_slots, static_cast<int32_t>(ns)});
    }
    out->num_slots += static_cast<int>(ns);
  }
  std::stable_sort(out->items.begin(), out->items.end(), [](const WorkItem& x, const WorkItem& y) {
    return (x.tok_end - x.tok_begin) > (y.tok_end - y.tok_begin);
  });

  // A uniform plan (equal lengths, contiguous cache, every item exactly what
  // uniform_item computes, merge jobs in sequence order) lets the kernels
  // compute their item instead of loading it.
  out->uniform_splits = out->uniform_chunk = out->uniform_len = 0;
  const size_t n_items = out->items.size();
  if (page_size != 1 || batch < 1 || lens[0] <= 0 || n_items % static_cast<size_t>(batch) != 0) return;
  for (int b = 0; b < batch; ++b)
    if (lens[b] != lens[0]) return;
  const int splits = static_cast<int>(n_items / static_cast<size_t>(batch));
  const int len = static_cast<int>(lens[0]);
  const int uchunk = splits == 1 ? len : out->items[0].tok_end - out->items[0].tok_begin;
  for (size_t i = 0; i < n_items; ++i) {
    const WorkItem u = uniform_item(static_cast<int>(i), splits, uchunk, len, indptr[0]);
    const WorkItem& w = out->items[i];
    if (w.batch != u.batch || w.tok_begin != u.tok_begin || w.tok_end != u.tok_end || w.slot != u.slot ||
        w.kv_base != u.kv_base || (splits > 1 && (w.merge_job != u.merge_job || w.slot_begin != u.slot_begin ||
                                                  w.nslots != u.nslots)))
      return;
  }
  if (splits > 1) {
    if (out->merge.size() != static_cast<size_t>(batch)) return;
    for (int m = 0; m < batch; ++m) {
      const MergeSeq& j = out->merge[m];
      if (j.batch != m || j.slot_begin != m * splits || j.nslots != splits) return;
    }
  }
  out->uniform_splits = splits;
  out->uniform_chunk = uchunk;
  out->uniform_len = len;
}

// Multi-token decode.  Query token j of sequence b (row qo_indptr[b] + j)
// sits at position n_b - q_b + j and attends to tokens 0 .. n_b - q_b + j.
// The sequences are planned as for single-token decode on 1 / max_b q_b of
// the workgroup slots, and every item becomes q_b items, one per query
// token, over the same tokens clipped to that token's causal end.  The q_b
// copies of an item go to workgroups launched together on one XCD, so that
// they stream the same cache rows at about the same pace through one L2.
static void plan_multi(const std::vector<int64_t>& lens, const std::vector<int32_t>& qlen,
                       const int32_t* qo_indptr, const int32_t* indptr, int split_override, int num_cus,
                       int blocks_per_cu, int page_size, int64_t tile, int64_t min_item, int64_t max_pages,
                       int64_t bin_cost, bool pairs, PlanOut* out) {
  const int batch = static_cast<int>(lens.size());
  int qmax = 0;
  bool single = true;
  for (int b = 0; b < batch; ++b) {
    qmax = std::max(qmax, qlen[b]);
    single = single && qlen[b] == 1;
  }
  if (single) {  // one query token per sequence: rows are sequences
    plan_items(lens, indptr, split_override, num_cus, blocks_per_cu, page_size, tile, min_item, max_pages, bin_cost,
               out);
    out->row_pairs = false;
    return;
  }
  // With pairs (fp8, whose kernel runs two query rows of a sequence over the
  // same tokens together), a parent group's rows take ceil(q / 2) workgroups.
  // Pairs pay where they keep the parents' pieces as long as single rows
  // would: 2 query tokens (bs64 x 8192: 82.5 -> 72.1 us a call).  With 4 the
  // parents are cut twice as fine, and the extra partials cost more than the
  // shared tile reads save (bs16 x 8192: 45.3 -> 48.2 us), so single rows.
  pairs = pairs && bin_cost > 0 && qmax == 2;
  const int lanes = pairs ? (qmax + 1) / 2 : qmax;
  if (pairs) max_pages = std::min<int64_t>(max_pages, kItemPagesFp8Pair);
  std::vector<int64_t> plens(batch);
  for (int b = 0; b < batch; ++b) plens[b] = qlen[b] ? lens[b] : 0;
  const int64_t slots = static_cast<int64_t>(num_cus) * std::max(blocks_per_cu, 1);
  PlanOut par;
  plan_items(plens, indptr, split_override, static_cast<int>(std::max<int64_t>(1, slots / lanes)), 1, page_size,
             tile, min_item, max_pages, bin_cost, &par);

  out->items.clear();
  out->merge.clear();
  out->bins.clear();
  out->num_slots = 0;
  out->max_splits = 0;
  out->uniform_splits = out->uniform_chunk = out->uniform_len = 0;
  out->row_pairs = pairs;
  // Parent group k (a bin, or an item) and query token j (with pairs: tokens
  // 2j and 2j + 1, each parent item's two listed together) become one group of
  // the expanded plan.  Kernels that run bins get bin 8 (q (k / 8) + j) + k % 8
  // (empty where there is nothing to do): workgroup x runs on XCD x mod 8, so
  // the q copies of a parent group share one XCD's L2.  The one-item kernel
  // gets the copies one after another.
  const size_t groups = par.bins.empty() ? par.items.size() : par.bins.size() - 1;
  auto parent_range = [&](size_t k, size_t* i0, size_t* i1) {
    *i0 = par.bins.empty() ? k : static_cast<size_t>(par.bins[k]);
    *i1 = par.bins.empty() ? k + 1 : static_cast<size_t>(par.bins[k + 1]);
  };
  auto emit = [&](size_t i0, size_t i1, int j0, int j1) {
    for (size_t i = i0; i < i1; ++i) {
      const WorkItem& it = par.items[i];
      if (it.slot == WorkItem::kEmpty) continue;  // a sequence without query tokens
      const int b = it.batch;
      for (int j = j0; j < j1 && j < qlen[b]; ++j) {
        const int64_t end = lens[b] - qlen[b] + j + 1;  // this token's causal end
        const int32_t t1 = static_cast<int32_t>(std::min<int64_t>(it.tok_end, end));
        if (it.tok_begin >= t1) continue;
        out->items.push_back(WorkItem{qo_indptr[b] + j, it.tok_begin, t1, 0, indptr[b], -1, 0, 0});
      }
    }
  };
  if (bin_cost > 0) {
    const size_t nbins = 8 * static_cast<size_t>(lanes) * ((groups + 7) / 8);
    for (size_t x = 0; x < nbins; ++x) {
      out->bins.push_back(static_cast<int32_t>(out->items.size()));
      const size_t lane = x % 8, rest = x / 8;
      const int j = static_cast<int>(rest % lanes);
      const size_t k = 8 * (rest / lanes) + lane;
      if (k >= groups) continue;
      size_t i0, i1;
      parent_range(k, &i0, &i1);
      if (pairs)
        emit(i0, i1, 2 * j, 2 * j + 2);
      else
        emit(i0, i1, j, j + 1);
    }
    out->bins.push_back(static_cast<int32_t>(out->items.size()));
  } else {
    for (size_t k = 0; k < groups; ++k) {
      size_t i0, i1;
      parent_range(k, &i0, &i1);
      for (int j = 0; j < qmax; ++j) emit(i0, i1, j, j + 1);
    }
  }

  // slots and merge jobs per row, its items in list order
  const int rows = qo_indptr[batch];
  std::vector<int32_t> npieces(rows, 0), first(rows, 0), job(rows, -1), seen(rows, 0);
  for (const WorkItem& it : out->items) ++npieces[it.batch];
  for (int r = 0; r < rows; ++r) {
    out->max_splits = std::max(out->max_splits, static_cast<int>(npieces[r]));
    if (npieces[r] < 2) continue;
    job[r] = static_cast<int32_t>(out->merge.size());
    first[r] = out->num_slots;
    out->merge.push_back(MergeSeq{r, out->num_slots, npieces[r], 0});
    out->num_slots += npieces[r];
  }
  for (WorkItem& it : out->items) {
    const int r = it.batch;
    if (npieces[r] == 1) {
      it.slot = WorkItem::kWhole;
      continue;
    }
    it.slot = first[r] + seen[r]++;
    it.merge_job = job[r];
    it.slot_begin = first[r];
    it.nslots = npieces[r];
  }
}

}  // namespace mla

extern "C" {

int mla_decode_version(void) { return kVersion; }

const char* mla_status_string(mla_status s) {
  switch (enum_value(s)) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_NOT_PLANNED: return "MLA_ERR_NOT_PLANNED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

mla_status mla_decode_create(mla_decode_t* out, int device, int num_heads, int qk_dim, int v_dim,
                             float sm_scale, mla_kv_dtype kv_dtype, int page_size) {
  if (!out) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (device < 0 || !(sm_scale > 0.f) || !std::isfinite(sm_scale) || page_size < 1)
    return MLA_ERR_INVALID_ARG;
  if (num_heads != mla::kNumHeads || qk_dim != mla::kQkDim || v_dim != mla::kVDim)
    return MLA_ERR_UNSUPPORTED;
  const int fmt = enum_value(kv_dtype);
  if (fmt != MLA_KV_BF16 && fmt != MLA_KV_FP8_E4M3 && fmt != MLA_KV_MXFP4) return MLA_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size > 1024) return MLA_ERR_UNSUPPORTED;
  mla_decode_t h = new (std::nothrow) mla_decode_s();
  if (!h) return MLA_ERR_INVALID_ARG;
  h->device = device;
  h->kv_dtype = fmt;
  h->page_size = page_size;
  while ((1 << h->page_shift) < page_size) ++h->page_shift;
  h->sm_scale = sm_scale;
  *out = h;
  return MLA_OK;
}

namespace {

mla_status plan_impl(mla_decode_t h, int batch, const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                     const int32_t* kv_last_page_len_host, int split_override, size_t* workspace_bytes) {
  if (!h) return MLA_ERR_INVALID_ARG;
  h->last_error.clear();
  if (batch < 1) return fail(h, MLA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (!kv_indptr_host) return fail(h, MLA_ERR_INVALID_ARG, "kv_indptr_host is NULL");
  if (h->page_size > 1 && !kv_last_page_len_host)
    return fail(h, MLA_ERR_INVALID_ARG, "kv_last_page_len_host is NULL with page_size > 1");
  if (split_override < 0) return fail(h, MLA_ERR_INVALID_ARG, "split_override is negative");
  if (!workspace_bytes) return fail(h, MLA_ERR_INVALID_ARG, "workspace_bytes is NULL");
  std::vector<int64_t> lens;
  std::string err;
  if (!mla::seq_lengths(kv_indptr_host, kv_last_page_len_host, batch, h->page_size, &lens, &err))
    return fail(h, MLA_ERR_INVALID_ARG, "%s", err.c_str());
  std::vector<int32_t> qlen(batch, 1), qo_unit;
  if (qo_indptr_host) {
    if (!mla::query_counts(qo_indptr_host, batch, lens, &qlen, &err))
      return fail(h, MLA_ERR_INVALID_ARG, "%s", err.c_str());
  } else {
    qo_unit.resize(batch + 1);
    for (int b = 0; b <= batch; ++b) qo_unit[b] = b;
    qo_indptr_host = qo_unit.data();
  }

  h->planned = false;
  DeviceGuard guard(h->device);
  if (!guard.ok) return fail(h, MLA_ERR_HIP, "cannot select HIP device %d", h->device);
  if (!h->num_cus) {
    int cus = 0, bpc = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess ||
        cus <= 0)
      return fail(h, MLA_ERR_HIP, "cannot read the compute-unit count of device %d", h->device);
    if (mla::stage1_occupancy(h->kv_dtype, h->page_size > 1, &bpc) != hipSuccess || bpc <= 0)
      return fail(h, MLA_ERR_HIP, "cannot read the stage-1 occupancy");
    h->num_cus = cus;
    h->blocks_per_cu = bpc;
  }

  mla::PlanOut plan;
  mla::plan_multi(lens, qlen, qo_indptr_host, kv_indptr_host, split_override, h->num_cus, h->blocks_per_cu,
                  h->page_size, mla::plan_tile(h->kv_dtype), mla::min_item_tokens(h->kv_dtype), mla::item_pages(h->kv_dtype),
                  mla::bin_piece_cost(h->kv_dtype), h->kv_dtype == MLA_KV_FP8_E4M3, &plan);

  const size_t items_bytes = plan.items.size() * sizeof(mla::WorkItem);
  const size_t merge_bytes = plan.merge.size() * sizeof(mla::MergeSeq);
  // completion counters of the fused merge, zero as uploaded
  const size_t counter_bytes = plan.merge.size() * sizeof(int32_t);
  const size_t bins_bytes = plan.bins.size() * sizeof(int32_t);
  const size_t need = items_bytes + merge_bytes + counter_bytes + bins_bytes;

  if (!h->upload_stream) {
    if (hipStreamCreateWithFlags(&h->upload_stream, hipStreamNonBlocking) != hipSuccess) {
      h->upload_stream = nullptr;
      return fail(h, MLA_ERR_HIP, "cannot create the plan upload stream");
    }
    for (int k = 0; k < 2; ++k)
      if (hipEventCreateWithFlags(&h->uploaded[k], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&h->released[k], hipEventDisableTiming) != hipSuccess)
        return fail(h, MLA_ERR_HIP, "hipEventCreate failed");
  }
  // The runs of the current plan have all been enqueued on last_run_stream
  // (runs of a handle do not overlap): its buffer is free once they are done.
  if (h->ran_since_plan) {
    if (hipEventRecord(h->released[h->cur], h->last_run_stream) != hipSuccess)
      return fail(h, MLA_ERR_HIP, "recording the end of the last run failed");
    h->release_pending[h->cur] = true;
  }
  const int b = h->cur ^ 1;
  if (need > h->dev_plan_bytes[b]) {
    if (h->release_pending[b] && hipEventSynchronize(h->released[b]) != hipSuccess)
      return fail(h, MLA_ERR_HIP, "waiting for the runs of an earlier plan failed");
    h->release_pending[b] = false;
    if (h->dev_plan[b]) (void)hipFree(h->dev_plan[b]);
    h->dev_plan[b] = nullptr;
    h->dev_plan_bytes[b] = 0;
    if (hipMalloc(&h->dev_plan[b], need) != hipSuccess)
      return fail(h, MLA_ERR_HIP, "hipMalloc of %zu plan bytes failed", need);
    h->dev_plan_bytes[b] = need;
  }
  // the host copy of buffer b is free again once its last upload is done
  if (h->upload_pending[b] && hipEventSynchronize(h->uploaded[b]) != hipSuccess)
    return fail(h, MLA_ERR_HIP, "waiting for an earlier plan upload failed");
  h->upload_pending[b] = false;
  if (need > h->host_plan_bytes[b]) {
    if (h->host_plan[b]) (void)hipHostFree(h->host_plan[b]);
    h->host_plan[b] = nullptr;
    h->host_plan_bytes[b] = 0;
    if (hipHostMalloc(&h->host_plan[b], need, hipHostMallocDefault) != hipSuccess)
      return fail(h, MLA_ERR_HIP, "hipHostMalloc of %zu plan bytes failed", need);
    h->host_plan_bytes[b] = need;
  }
  unsigned char* blob = static_cast<unsigned char*>(h->host_plan[b]);
  if (items_bytes) std::memcpy(blob, plan.items.data(), items_bytes);
  if (merge_bytes) std::memcpy(blob + items_bytes, plan.merge.data(), merge_bytes);
  if (counter_bytes) std::memset(blob + items_bytes + merge_bytes, 0, counter_bytes);
  if (bins_bytes) std::memcpy(blob + items_bytes + merge_bytes + counter_bytes, plan.bins.data(), bins_bytes);
  if (need) {
    if (h->release_pending[b] && hipStreamWaitEvent(h->upload_stream, h->released[b], 0) != hipSuccess)
      return fail(h, MLA_ERR_HIP, "ordering the plan upload after earlier runs failed");
    if (hipMemcpyAsync(h->dev_plan[b], blob, need, hipMemcpyHostToDevice, h->upload_stream) != hipSuccess ||
        hipEventRecord(h->uploaded[b], h->upload_stream) != hipSuccess)
      return fail(h, MLA_ERR_HIP, "uploading the work list failed");
    h->upload_pending[b] = true;
  }
  h->cur = b;
  h->ran_since_plan = false;
  h->waited = false;

  h->batch = qo_indptr_host[batch];  // output rows
  h->num_items = static_cast<int>(plan.items.size());
  h->num_bins = plan.bins.empty() ? 0 : static_cast<int>(plan.bins.size()) - 1;
  h->row_pairs = plan.row_pairs;
  h->num_slots = plan.num_slots;
  h->max_splits = plan.max_splits;
  h->num_merge = static_cast<int>(plan.merge.size());
  // The fused merge adds the last item's read-back of the other partials to
  // that item, and to every split item a wait for its fp32 partial stores and
  // a counter round trip.  Measured: a uniform plan, whose items all finish
  // together, merges faster in the merge kernel, and so does every ragged
  // fp8 and MXFP4 plan, whose partials go to the merge kernel as bf16
  // (3-4 % per call); ragged bf16 plans, whose partials stay fp32, run about
  // 1 % faster fused.
  h->fused_merge = plan.max_splits <= mla::kFusedMergeMaxSlots && plan.uniform_splits == 0 &&
                   h->kv_dtype == MLA_KV_BF16;
  h->uniform_splits = plan.uniform_splits;
  h->uniform_chunk = plan.uniform_chunk;
  h->uniform_len = plan.uniform_len;
  h->uniform_base = kv_indptr_host[0];
  h->total_tokens = 0;
  for (const mla::WorkItem& it : plan.items) h->total_tokens += it.tok_end - it.tok_begin;
  h->workspace_bytes = static_cast<size_t>(plan.num_slots) * slot_bytes();
  h->planned = true;
  *workspace_bytes = h->workspace_bytes;
  return MLA_OK;
}

mla_status preview_impl(int batch, const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                        const int32_t* kv_last_page_len_host, int page_size, int kv_dtype,
                        int split_override, int num_cus, int blocks_per_cu, int32_t* items_out, int max_items,
                        int* num_items, int* num_slots, size_t* workspace_bytes) {
  if (batch < 1 || !kv_indptr_host || page_size < 1 || !is_pow2(page_size) || split_override < 0 ||
      num_cus < 1 || blocks_per_cu < 1 || max_items < 0 || (max_items > 0 && !items_out) ||
      (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3 && kv_dtype != MLA_KV_MXFP4))
    return MLA_ERR_INVALID_ARG;
  if (page_size > 1 && !kv_last_page_len_host) return MLA_ERR_INVALID_ARG;
  std::vector<int64_t> lens;
  std::string err;
  if (!mla::seq_lengths(kv_indptr_host, kv_last_page_len_host, batch, page_size, &lens, &err))
    return MLA_ERR_INVALID_ARG;
  std::vector<int32_t> qlen(batch, 1), qo_unit;
  if (qo_indptr_host) {
    if (!mla::query_counts(qo_indptr_host, batch, lens, &qlen, &err)) return MLA_ERR_INVALID_ARG;
  } else {
    qo_unit.resize(batch + 1);
    for (int b = 0; b <= batch; ++b) qo_unit[b] = b;
    qo_indptr_host = qo_unit.data();
  }
  mla::PlanOut plan;
  mla::plan_multi(lens, qlen, qo_indptr_host, kv_indptr_host, split_override, num_cus, blocks_per_cu, page_size,
                  mla::plan_tile(kv_dtype), mla::min_item_tokens(kv_dtype), mla::item_pages(kv_dtype), mla::bin_piece_cost(kv_dtype),
                  kv_dtype == MLA_KV_FP8_E4M3, &plan);
  const int n = static_cast<int>(plan.items.size());
  if (num_items) *num_items = n;
  if (num_slots) *num_slots = plan.num_slots;
  if (workspace_bytes) *workspace_bytes = static_cast<size_t>(plan.num_slots) * slot_bytes();
  if (n > max_items) return MLA_ERR_INVALID_ARG;
  int bin = 0;
  for (int i = 0; i < n; ++i) {
    while (!plan.bins.empty() && i >= plan.bins[bin + 1]) ++bin;
    items_out[5 * i + 0] = plan.items[i].batch;
    items_out[5 * i + 1] = plan.items[i].tok_begin;
    items_out[5 * i + 2] = plan.items[i].tok_end;
    items_out[5 * i + 3] = plan.items[i].slot;
    items_out[5 * i + 4] = plan.bins.empty() ? i : bin;
  }
  return MLA_OK;
}

}  // namespace

mla_status mla_decode_plan(mla_decode_t h, int batch, const int32_t* kv_indptr_host,
                           const int32_t* kv_last_page_len_host, int split_override,
                           size_t* workspace_bytes) {
  return plan_impl(h, batch, nullptr, kv_indptr_host, kv_last_page_len_host, split_override, workspace_bytes);
}

mla_status mla_decode_plan_multi(mla_decode_t h, int batch, const int32_t* qo_indptr_host,
                                 const int32_t* kv_indptr_host, const int32_t* kv_last_page_len_host,
                                 int split_override, size_t* workspace_bytes) {
  if (!h) return MLA_ERR_INVALID_ARG;
  if (!qo_indptr_host) return fail(h, MLA_ERR_INVALID_ARG, "qo_indptr_host is NULL");
  return plan_impl(h, batch, qo_indptr_host, kv_indptr_host, kv_last_page_len_host, split_override,
                   workspace_bytes);
}

mla_status mla_decode_plan_preview(int batch, const int32_t* kv_indptr_host,
                                   const int32_t* kv_last_page_len_host, int page_size,
                                   mla_kv_dtype kv_dtype, int split_override, int num_cus,
                                   int blocks_per_cu, int32_t* items_out, int max_items,
                                   int* num_items, int* num_slots, size_t* workspace_bytes) {
  return preview_impl(batch, nullptr, kv_indptr_host, kv_last_page_len_host, page_size, enum_value(kv_dtype),
                      split_override,
                      num_cus, blocks_per_cu, items_out, max_items, num_items, num_slots, workspace_bytes);
}

mla_status mla_decode_plan_preview_multi(int batch, const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                                         const int32_t* kv_last_page_len_host, int page_size,
                                         mla_kv_dtype kv_dtype, int split_override, int num_cus,
                                         int blocks_per_cu, int32_t* items_out, int max_items,
                                         int* num_items, int* num_slots, size_t* workspace_bytes) {
  if (!qo_indptr_host) return MLA_ERR_INVALID_ARG;
  return preview_impl(batch, qo_indptr_host, kv_indptr_host, kv_last_page_len_host, page_size,
                      enum_value(kv_dtype), split_override, num_cus, blocks_per_cu, items_out, max_items, num_items, num_slots,
                      workspace_bytes);
}

mla_status mla_decode_plan_info(mla_decode_t h, int* num_items, int* max_splits,
                                int* num_partials) {
  if (!h) return MLA_ERR_INVALID_ARG;
  if (!h->planned) return fail(h, MLA_ERR_NOT_PLANNED, "no plan");
  if (num_items) *num_items = h->num_items;
  if (max_splits) *max_splits = h->max_splits;
  if (num_partials) *num_partials = h->num_slots;
  return MLA_OK;
}

mla_status mla_decode_run(mla_decode_t h, const void* q, const void* kv, const void* kv_scales,
                          int64_t kv_scale_stride, const int32_t* kv_indptr,
                          const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
                          void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h) return MLA_ERR_INVALID_ARG;
  h->last_error.clear();
  if (!h->planned) return fail(h, MLA_ERR_NOT_PLANNED, "mla_decode_run before a successful plan");
  // With every sequence empty nothing reads the cache, which may then be empty.
  const bool reads_cache = h->total_tokens > 0;
  if (!q || !kv_indptr || !out || (reads_cache && !kv))
    return fail(h, MLA_ERR_INVALID_ARG, "null q/kv/kv_indptr/out");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv)) & 15)
    return fail(h, MLA_ERR_INVALID_ARG, "q and kv must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(out) & 15)
    return fail(h, MLA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (reads_cache && h->kv_dtype != MLA_KV_BF16 && !kv_scales)
    return fail(h, MLA_ERR_INVALID_ARG, "kv_scales is NULL for a scaled cache format");
  if (h->kv_dtype == MLA_KV_MXFP4 && kv_scale_stride < 18)
    return fail(h, MLA_ERR_INVALID_ARG, "MXFP4 kv_scale_stride must be >= 18 (got %lld)",
                static_cast<long long>(kv_scale_stride));
  if (h->page_size > 1 && (!kv_page_indices || !kv_last_page_len))
    return fail(h, MLA_ERR_INVALID_ARG, "page table arrays are NULL with page_size > 1");
  if (workspace_bytes < h->workspace_bytes)
    return fail(h, MLA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, plan needs %zu",
                workspace_bytes, h->workspace_bytes);
  if (h->workspace_bytes && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15)))
    return fail(h, MLA_ERR_INVALID_ARG, "workspace is NULL or not 16-byte aligned");

  DeviceGuard guard(h->device);
  if (!guard.ok) return fail(h, MLA_ERR_HIP, "cannot select HIP device %d", h->device);
  hipStream_t s = static_cast<hipStream_t>(stream);

  mla::Stage1Args a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv);
  a.kv_mx_scales = h->kv_dtype == MLA_KV_MXFP4 ? static_cast<const uint8_t*>(kv_scales) : nullptr;
  a.kv_scale = h->kv_dtype == MLA_KV_FP8_E4M3 ? static_cast<const float*>(kv_scales) : nullptr;
  a.scale_stride = kv_scale_stride;
  a.kv_indptr = kv_indptr;
  a.page_indices = kv_page_indices;
  a.page_shift = h->page_shift;
  // The first run of a plan on a stream waits for the plan's upload.
  if (h->upload_pending[h->cur] && (!h->waited || h->waited_stream != s)) {
    if (hipStreamWaitEvent(s, h->uploaded[h->cur], 0) != hipSuccess)
      return fail(h, MLA_ERR_HIP, "ordering the run after the plan upload failed");
    h->waited = true;
    h->waited_stream = s;
  }
  h->ran_since_plan = true;
  h->last_run_stream = s;
  unsigned char* plan_base = static_cast<unsigned char*>(h->dev_plan[h->cur]);
  const size_t items_bytes = static_cast<size_t>(h->num_items) * sizeof(mla::WorkItem);
  a.items = reinterpret_cast<const mla::WorkItem*>(plan_base);
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = h->num_slots
                   ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                              static_cast<size_t>(h->num_slots) * mla::kNumHeads *
                                                  mla::kVDim * sizeof(float))
                   : nullptr;
  a.out = static_cast<uint16_t*>(out);
  a.score_scale = h->sm_scale * 1.4426950408889634f;
  a.uniform_splits = h->uniform_splits;
  a.uniform_chunk = h->uniform_chunk;
  a.uniform_len = h->uniform_len;
  a.uniform_base = h->uniform_base;
  a.query_e4m3 = h->query_format == MLA_QUERY_E4M3;
  a.part_bf16 = h->kv_dtype != MLA_KV_BF16;
  if (a.query_e4m3 && !mla::stage1_dedicated(h->kv_dtype, a))
    return fail(h, MLA_ERR_UNSUPPORTED,
                "MLA_QUERY_E4M3 needs the MXFP4 split kernel, which needs an even scale stride and scale address");
  const size_t merge_bytes = static_cast<size_t>(h->num_merge) * sizeof(mla::MergeSeq);
  a.counters = h->fused_merge && h->num_merge > 0 && mla::stage1_dedicated(h->kv_dtype, a)
                   ? reinterpret_cast<int*>(plan_base + items_bytes + merge_bytes)
                   : nullptr;

  const bool timed = h->profiling && h->events_ready;
  h->timed_run = false;
  h->merge_timed = false;
  // The fp8 and MXFP4 kernels run a binned plan bin by bin; the generic one
  // (MXFP4 with odd scale addresses) takes its items one per workgroup.
  const bool by_bin = h->num_bins > 0 && mla::stage1_dedicated(h->kv_dtype, a);
  a.bins = by_bin ? reinterpret_cast<const int32_t*>(plan_base + items_bytes + merge_bytes +
                                                     static_cast<size_t>(h->num_merge) * sizeof(int32_t))
                  : nullptr;
  hipError_t e = mla::launch_stage1(h->kv_dtype, h->page_size > 1, by_bin && h->row_pairs, a,
                                     by_bin ? h->num_bins : h->num_items, s,
                                     timed ? h->ev[0] : nullptr, timed ? h->ev[1] : nullptr);
  if (e != hipSuccess) return fail(h, MLA_ERR_HIP, "stage-1 launch: %s", hipGetErrorString(e));
  if (h->num_merge > 0 && !a.counters) {
    mla::MergeArgs m{};
    m.work = reinterpret_cast<const mla::MergeSeq*>(plan_base + items_bytes);
    m.uniform_nslots = h->uniform_splits > 1 ? h->uniform_splits : 0;
    m.part_bf16 = a.part_bf16;
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.out = a.out;
    e = mla::launch_merge(m, h->num_merge, s, timed ? h->ev[2] : nullptr,
                          timed ? h->ev[3] : nullptr);
    if (e != hipSuccess) return fail(h, MLA_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
    h->merge_timed = timed;
  }
  h->timed_run = timed;
  return MLA_OK;
}

mla_status mla_decode_run_noalloc(mla_decode_t h, const void* q, const void* kv, const void* kv_scales,
                                  int64_t kv_scale_stride, const int32_t* kv_indptr,
                                  const int32_t* kv_page_indices, const int32_t* kv_last_page_len, void* out,
                                  void* stream) {
  if (!h) return MLA_ERR_INVALID_ARG;
  h->last_error.clear();
  if (!h->planned) return fail(h, MLA_ERR_NOT_PLANNED, "mla_decode_run_noalloc before a successful plan");
  if (h->workspace_bytes > mla::kScratchBytes)
    return fail(h, MLA_ERR_UNSUPPORTED,
                "the plan needs %zu bytes of partials; the allocation-free run holds at most %zu "
                "(plan with a smaller split_override, or use mla_decode_run with a workspace)",
                h->workspace_bytes, mla::kScratchBytes);
  void* scratch = nullptr;
  if (h->workspace_bytes) {
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(h, MLA_ERR_HIP, "cannot select HIP device %d", h->device);
    const hipError_t e = mla::scratch_address(h->device, &scratch);
    if (e != hipSuccess)
      return fail(h, MLA_ERR_HIP, "device address of the scratch array: %s", hipGetErrorString(e));
  }
  return mla_decode_run(h, q, kv, kv_scales, kv_scale_stride, kv_indptr, kv_page_indices, kv_last_page_len, out,
                        scratch, scratch ? mla::kScratchBytes : 0, stream);
}

mla_status mla_decode_set_query_format(mla_decode_t h, int query_format) {
  if (!h) return MLA_ERR_INVALID_ARG;
  h->last_error.clear();
  if (query_format != MLA_QUERY_EXACT && query_format != MLA_QUERY_E4M3)
    return fail(h, MLA_ERR_INVALID_ARG, "query_format must be MLA_QUERY_EXACT or MLA_QUERY_E4M3 (got %d)",
                query_format);
  if (query_format == MLA_QUERY_E4M3 && h->kv_dtype == MLA_KV_BF16)
    return fail(h, MLA_ERR_UNSUPPORTED, "MLA_QUERY_E4M3 applies to fp8 and MXFP4 caches");
  h->query_format = query_format;
  return MLA_OK;
}

mla_status mla_decode_set_profiling(mla_decode_t h, int enable) {
  if (!h) return MLA_ERR_INVALID_ARG;
  if (enable && !h->events_ready) {
    DeviceGuard guard(h->device);
    if (!guard.ok) return fail(h, MLA_ERR_HIP, "cannot select HIP device %d", h->device);
    for (auto& e : h->ev)
      if (hipEventCreate(&e) != hipSuccess) return fail(h, MLA_ERR_HIP, "hipEventCreate failed");
    h->events_ready = true;
  }
  h->profiling = enable != 0;
  return MLA_OK;
}

mla_status mla_decode_kernel_time_ms(mla_decode_t h, int which, float* ms) {
  if (!h || !ms || (which != 0 && which != 1)) return MLA_ERR_INVALID_ARG;
  if (!h->timed_run) return fail(h, MLA_ERR_NOT_PLANNED, "the last run was not timed");
  *ms = 0.f;
  if (which == 1 && !h->merge_timed) return MLA_OK;
  hipEvent_t e0 = h->ev[which == 0 ? 0 : 2], e1 = h->ev[which == 0 ? 1 : 3];
  if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(ms, e0, e1) != hipSuccess)
    return fail(h, MLA_ERR_HIP, "reading the kernel events failed");
  return MLA_OK;
}

mla_status mla_decode_kernel_resources(mla_decode_t h, int which, int* vgprs, int* lds_bytes,
                                       int* scratch_bytes) {
  if (!h || (which != 0 && which != 1)) return MLA_ERR_INVALID_ARG;
  DeviceGuard guard(h->device);
  if (!guard.ok) return fail(h, MLA_ERR_HIP, "cannot select HIP device %d", h->device);
  hipFuncAttributes attr{};
  if (mla::kernel_attributes(h->kv_dtype, h->page_size > 1, h->planned && h->row_pairs,
                            h->query_format == MLA_QUERY_E4M3, which, &attr) != hipSuccess)
    return fail(h, MLA_ERR_HIP, "hipFuncGetAttributes failed");
  if (vgprs) *vgprs = attr.numRegs;
  if (lds_bytes) *lds_bytes = static_cast<int>(attr.sharedSizeBytes);
  if (scratch_bytes) *scratch_bytes = static_cast<int>(attr.localSizeBytes);
  return MLA_OK;
}

mla_status mla_decode_destroy(mla_decode_t h) {
  if (!h) return MLA_OK;
  {
    DeviceGuard guard(h->device);
    for (int k = 0; k < 2; ++k) {
      if (h->dev_plan[k]) (void)hipFree(h->dev_plan[k]);
      if (h->host_plan[k]) (void)hipHostFree(h->host_plan[k]);
      if (h->uploaded[k]) (void)hipEventDestroy(h->uploaded[k]);
      if (h->released[k]) (void)hipEventDestroy(h->released[k]);
    }
    if (h->upload_stream) (void)hipStreamDestroy(h->upload_stream);
    for (auto& e : h->ev)
      if (e) (void)hipEventDestroy(e);
  }
  delete h;
  return MLA_OK;
}

const char* mla_decode_last_error(mla_decode_t h) {
  if (!h) return "null handle";
  return h->last_error.c_str();
}

}  // extern "C"
