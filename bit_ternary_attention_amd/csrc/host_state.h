// Host-side cache state: configuration checks, page allocator, tier router,
// append planner and decode planner.  Pure C++17, no HIP, so it can be built
// and exercised on a machine without a GPU.
//
// Tiers follow "Minima-KV" (twodots.gr), section "Recent, Anchor and Stale":
// recent pages in FP8, anchor pages (initial attention sinks) at higher
// fidelity, older pages packed, every page addressable through the block table.
#pragma once

#include <cstdint>
#include <deque>
#include <string>
#include <utility>
#include <vector>

#include "vk.h"

namespace vk {

constexpr int kFormats = 4;  // VK_FMT_TERNARY2, FP8E4M3, F16, LOSSLESS
constexpr int kUnit = 16;          // tokens per unit: the decode and pack work granule
constexpr int64_t kAbsBlockElems = 16384;  // elements per absmean block (the write side's pass 1)
constexpr int32_t kNoPage = -1;

inline int32_t make_entry(int fmt, int32_t idx) {
  return static_cast<int32_t>((static_cast<uint32_t>(fmt) << 30) | static_cast<uint32_t>(idx));
}
inline int entry_fmt(int32_t e) { return static_cast<int>(static_cast<uint32_t>(e) >> 30); }
inline int32_t entry_idx(int32_t e) { return e & 0x3FFFFFFF; }

// Returns "" when cfg is usable, else the reason.
std::string validate_config(const vk_cache_config& cfg);
// Bytes of one (K or V, one KV head) tile of a page of `fmt`.
int64_t tile_bytes(const vk_cache_config& cfg, int fmt);
// Bytes of a whole page (K and V, every KV head).
int64_t page_bytes(const vk_cache_config& cfg, int fmt);

// One sequence of an append call, as the device kernels read it.
struct AppendSeqDesc {
  int32_t slot;        // sequence id (block-table row)
  int32_t t0;          // length before the call
  int32_t tern_lo;     // ternary-routed tokens of the call: [tern_lo, tern_hi), call-relative
  int32_t tern_hi;
  int32_t page_first;  // first page the call touches
  int32_t page_off;    // offset of that page's entry in the entry list
  int32_t n_pages;     // pages touched
  int32_t unit_first;  // first 16-token unit touched
  int32_t n_tokens;    // tokens this call adds to the sequence
  int32_t tok_off;     // row of its first token in each layer's input block
  int32_t task_off;    // first pack task of the sequence within a layer (16-token unit, K|V, head)
  int32_t blk_off;     // first absmean block of the sequence within a (layer, K|V)
};
static_assert(sizeof(AppendSeqDesc) == 48, "device layout");

struct AppendPlan {
  std::vector<AppendSeqDesc> seqs;
  std::vector<int32_t> entries;     // block-table entries of every touched page, per seq
  int64_t total_tokens = 0;         // rows of each layer's input block (sum over sequences)
  int64_t total_tasks = 0;          // pack tasks per layer (sum over sequences)
  int64_t total_blk = 0;            // absmean blocks per (layer, K|V) (sum over sequences)
  int32_t max_units = 0;            // most 16-token units touched by one sequence
  int32_t max_tern_tokens = 0;      // most ternary tokens in one sequence
  int64_t new_pages[kFormats] = {0, 0, 0, 0};
  std::vector<int32_t> new_fmt;     // per new page, in order (seq, page)
};

struct SeqState {
  int32_t length = 0;
  std::vector<int32_t> pages;                       // entries of allocated pages
  std::vector<std::pair<int32_t, int32_t>> runs;    // (first page, format) of same-format runs
  int32_t retier_from = 0;                          // pages below were examined by a retier
  int32_t evict_end = 0;                            // pages [sink pages, evict_end) are freed
};

// One page of one sequence moving from the FP8 tier to the ternary tier (all layers).
struct RetierTask {
  int32_t slot;   // sequence id (block-table row)
  int32_t page;   // logical page
  int32_t src;    // FP8 pool index (freed by the commit)
  int32_t dst;    // ternary pool index (taken by the commit)
};
static_assert(sizeof(RetierTask) == 16, "device layout");

struct RetierPlan {
  std::vector<RetierTask> tasks;
  std::vector<int32_t> page_end;   // per listed sequence: pages below are settled
};

// Attended 16-token units of a sequence: [0, a_end) and [b_begin, b_end).
struct UnitRanges {
  int32_t a_end = 0, b_begin = 0, b_end = 0;
  int32_t sinks = 0;       // min(S, L)
  int32_t w0 = 0;          // first window token
  int32_t n_units() const { return a_end + (b_end - b_begin); }
};
UnitRanges attended_units(int32_t length, int32_t sink_tokens, int32_t window);

// Split-K plan of a decode launch: every split holds units_per_split logical units of its
// sequence (the last one fewer), so long sequences get more splits than short ones.
// total_units = attended units summed over the launch's (sequence, KV head) items; the
// split size aims at target_blocks blocks in all, with at least min_units units, and
// n_splits = ceil(max_units / units_per_split) <= max_splits.
struct SplitPlan {
  int32_t n_splits;
  int32_t units_per_split;
};
SplitPlan plan_splits(int64_t total_units, int32_t max_units, int32_t target_blocks, int32_t max_splits,
                      int32_t min_units, int32_t granule = 1);

// A launch whose `items` (sequence, KV head) pairs all attend max_units units runs in
// ceil(items x n_splits / n_cu) blocks on its busiest compute unit, and takes about as long as
// that unit's units (blocks x units_per_split) weighted by how well that many resident blocks
// stream (measured on 32 x 32K tokens at 1, 2 and 3 blocks per CU: 1.18, 1.00, 1.04).  Returns
// the split count (same granule and minimum split size) with the smallest such cost when it
// beats `base` by more than 5%, else `base`.  Only plans that fill every compute unit and keep
// at most max_per_cu (<= 3) blocks per CU, all resident at once, are weighed; `base` outside
// that range is returned as it is.
SplitPlan balance_splits(SplitPlan base, int64_t items, int32_t max_units, int32_t n_cu, int32_t max_per_cu,
                         int32_t max_splits, int32_t min_units, int32_t granule);

// Dispatch order of a matrix-core decode launch over sequences of different lengths: every
// (sequence i, part z) block of the launch once, heaviest first (the longest-processing-time
// rule: the hardware hands the next block to whichever compute-unit slot frees up, so the large
// blocks start first and the small ones fill the tail).  Split z of sequence i weighs the units
// it takes, clamp(units[i] - z * units_per_split, 0, units_per_split); each of the n_mix fp8 /
// fp16 parts weighs mix_weight[i] (0 when the sequence has no such pages).  Equal weights keep
// the default order (part-major, then sequence).  Entries are (part << 8) | i.  Returns false
// (and leaves `order` empty) when the result is the default order or has more than max_entries
// entries: the launch then keeps its plain grid.
bool plan_decode_order(const int32_t* units, const int64_t* mix_weight, int32_t n_seqs, int32_t n_splits,
                       int32_t units_per_split, int32_t n_mix, int32_t max_entries, std::vector<uint16_t>* order);

class HostState {
 public:
  explicit HostState(const vk_cache_config& cfg);

  const vk_cache_config& cfg() const { return cfg_; }
  int32_t max_pages() const { return max_pages_; }
  const SeqState& seq(int32_t s) const { return seqs_[s]; }

  // Format of page `page` when first written by an append ending at new_len.
  int32_t new_page_format(int32_t page, int32_t new_len) const;

  // Checks an append of n_tokens[i] tokens to sequence seq_ids[i] and computes what it needs.
  // Nothing changes.
  vk_status plan_append(int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_tokens, AppendPlan* plan,
                        std::string* err) const;
  // Takes the pages from the free lists, fills plan->entries, advances lengths.
  void commit_append(AppendPlan* plan);

  // Retiering ("Minima-KV", Recent/Anchor/Stale tiers): every FP8 page of the listed
  // sequences that is not a sink page and ends at or before length - recent_tokens.
  // Checks ids and ternary capacity; nothing changes.
  vk_status plan_retier(int32_t n_seqs, const int32_t* seq_ids, RetierPlan* plan, std::string* err) const;
  // Takes ternary pages (fills tasks[].dst), returns the FP8 pages to their free list,
  // flips the host block table.
  void commit_retier(int32_t n_seqs, const int32_t* seq_ids, RetierPlan* plan);

  // Bounded-memory eviction ("Show HN: Vantage-V-AI": max_active_tokens with sink
  // tokens kept): frees every page of the listed sequences past the sink pages that ends
  // at or before length - window; their entries become kNoPage.  Returns the page count.
  vk_status evict(int32_t n_seqs, const int32_t* seq_ids, int32_t window, int64_t* n_pages, std::string* err);

  vk_status check_decode(int32_t n_seqs, const int32_t* seq_ids, int32_t window, std::string* err) const;
  // Attended units of `slot` by page format (route counters).
  void count_units(int32_t slot, int32_t window, int64_t out[kFormats]) const;
  // Two ranges of logical attended units, [out[0], out[1]) and [out[2], out[3]), that hold
  // every attended unit of `slot` whose page is not ternary (split at the widest gap between
  // such units; empty ranges when there are none): the part of the sequence a decode's
  // fp8 / fp16 block has to look at.
  void mixed_ranges(int32_t slot, int32_t window, int32_t out[4]) const;

  vk_status reset_seqs(int32_t n_seqs, const int32_t* seq_ids, std::string* err);

  int64_t pages_used(int fmt) const;
  int64_t tokens_stored(int fmt) const;
  int64_t free_pages(int fmt) const { return static_cast<int64_t>(free_[fmt].size()); }

 private:
  vk_cache_config cfg_;
  int32_t max_pages_;
  std::vector<SeqState> seqs_;
  std::deque<int32_t> free_[kFormats];
};

}  // namespace vk
