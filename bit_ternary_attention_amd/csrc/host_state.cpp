// Host-side cache state (no HIP).  See host_state.h.
#include "host_state.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <unordered_set>

namespace vk {
namespace {

std::string fmt_str(const char* f, long long a, long long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b);
  return buf;
}

bool valid_format(int32_t f) { return f >= VK_FMT_TERNARY2 && f <= VK_FMT_LOSSLESS; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// splitmix64 (Steele, Lea, Flood: "Fast splittable pseudorandom number generators").
struct SplitMix64 {
  uint64_t x;
  uint64_t next() {
    x += 0x9E3779B97F4A7C15ull;
    uint64_t z = x;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

}  // namespace

std::string validate_config(const vk_cache_config& c) {
  if (c.n_layers < 1) return "n_layers must be >= 1";
  if (c.n_kv_heads < 1) return "n_kv_heads must be >= 1";
  if (c.n_q_heads < 1 || c.n_q_heads % c.n_kv_heads) return "n_q_heads must be a positive multiple of n_kv_heads";
  int g = c.n_q_heads / c.n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return "n_q_heads / n_kv_heads must be 1, 2, 4 or 8";
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256) return "head_dim must be 64, 128 or 256";
  if (c.block_size < kUnit || c.block_size > 65536 || (c.block_size & (c.block_size - 1)))
    return "block_size must be a power of two in [16, 65536]";
  if (c.max_seqs < 1) return "max_seqs must be >= 1";
  if (c.max_tokens_per_seq < 1) return "max_tokens_per_seq must be >= 1";
  if (c.sink_tokens < 0) return "sink_tokens must be >= 0";
  if (c.recent_tokens < 0) return "recent_tokens must be >= 0";
  if (!valid_format(c.sink_format) || !valid_format(c.recent_format)) return "unknown page format";
  if (c.decode_kernel < 0 || c.decode_kernel > 2) return "decode_kernel must be 0, 1 or 2";
  if (c.decode_kernel == VK_DECODE_VALU && (c.sink_format == VK_FMT_LOSSLESS || c.recent_format == VK_FMT_LOSSLESS))
    return "lossless pages are read by the matrix-core decode kernel only";
  if (c.head_dim == 256 && (c.sink_format == VK_FMT_LOSSLESS || c.recent_format == VK_FMT_LOSSLESS))
    return "lossless pages take head_dim 64 or 128";
  if (c.fp8_dynamic != 0 && c.fp8_dynamic != 1) return "fp8_dynamic must be 0 or 1";
  if (c.reserved0 != 0) return "reserved0 must be 0";
  if (c.pages_ternary < 0 || c.pages_fp8 < 0 || c.pages_f16 < 0 || c.pages_lossless < 0)
    return "pool capacities must be >= 0";
  if (c.pages_ternary >= (1ll << 30) || c.pages_fp8 >= (1ll << 30) || c.pages_f16 >= (1ll << 30) ||
      c.pages_lossless >= (1ll << 30))
    return "pool capacities must be < 2^30 pages";
  if (!(c.eps >= 0.0f) || !std::isfinite(c.eps)) return "eps must be finite and >= 0";
  if (!(c.fp8_scale > 0.0f) || !std::isfinite(c.fp8_scale)) return "fp8_scale must be finite and > 0";
  int64_t max_pages = cdiv(c.max_tokens_per_seq, c.block_size);
  if (static_cast<int64_t>(c.max_seqs) * max_pages > (1ll << 31) - 1) return "block table too large";
  return "";
}

int64_t tile_bytes(const vk_cache_config& c, int fmt) {
  int64_t elems = static_cast<int64_t>(c.block_size) * c.head_dim;
  switch (fmt) {
    case VK_FMT_TERNARY2: return elems / 4;
    case VK_FMT_FP8E4M3: return elems + (c.fp8_dynamic ? 4ll * c.block_size : 0);  // + token scales
    case VK_FMT_F16: return elems * 2;
    // per 16-token unit: a 16-byte header and room for the raw bfloat16 values
    case VK_FMT_LOSSLESS: return (c.block_size / kUnit) * (kUnit * 2ll * c.head_dim + 16);
  }
  return 0;
}

int64_t page_bytes(const vk_cache_config& c, int fmt) { return 2ll * c.n_kv_heads * tile_bytes(c, fmt); }

UnitRanges attended_units(int32_t length, int32_t sink_tokens, int32_t window) {
  UnitRanges r;
  r.sinks = std::min(sink_tokens, length);
  int32_t all = static_cast<int32_t>(cdiv(length, kUnit));
  if (window < 0 || static_cast<int64_t>(length) - window <= r.sinks) {
    r.a_end = r.b_begin = r.b_end = all;
    r.w0 = 0;
    return r;
  }
  r.w0 = length - window;
  r.a_end = static_cast<int32_t>(cdiv(r.sinks, kUnit));
  if (window == 0) {
    r.b_begin = r.b_end = r.a_end;
  } else {
    r.b_begin = std::max(r.a_end, r.w0 / kUnit);
    r.b_end = all;
  }
  return r;
}

SplitPlan plan_splits(int64_t total_units, int32_t max_units, int32_t target_blocks, int32_t max_splits,
                      int32_t min_units, int32_t granule) {
  if (max_units <= 0) return {1, 1};
  const int64_t want = std::max<int64_t>(std::max(1, min_units), cdiv(total_units, std::max(1, target_blocks)));
  const int64_t n = std::min<int64_t>(std::max<int64_t>(1, cdiv(max_units, want)), std::max(1, max_splits));
  // split size rounded up to the granule (whole kernel steps per wave); fewer splits may then do
  const int64_t g = std::max(1, granule);
  const int64_t ups = cdiv(cdiv(max_units, n), g) * g;
  return {static_cast<int32_t>(cdiv(max_units, ups)), static_cast<int32_t>(ups)};
}

SplitPlan balance_splits(SplitPlan base, int64_t items, int32_t max_units, int32_t n_cu, int32_t max_per_cu,
                         int32_t max_splits, int32_t min_units, int32_t granule) {
  static constexpr int64_t kWeight[4] = {0, 118, 100, 104};  // per resident blocks per CU (1..3)
  const int64_t cap = std::min<int64_t>(3, max_per_cu);
  if (items <= 0 || n_cu <= 0 || max_units <= 0 || base.n_splits < 1 || cap < 1) return base;
  // cost of a plan on its busiest compute unit, or -1 outside the weighed range
  auto cost = [&](int64_t n_splits, int64_t ups) -> int64_t {
    const int64_t blocks = items * n_splits;
    if (blocks < n_cu) return -1;
    const int64_t k = cdiv(blocks, n_cu);
    return k <= cap ? k * ups * kWeight[k] : -1;
  };
  const int64_t base_cost = cost(base.n_splits, base.units_per_split);
  if (base_cost < 0) return base;
  SplitPlan best = base;
  int64_t best_cost = base_cost;
  const int64_t g = std::max(1, granule);
  for (int32_t s = 1; s <= max_splits; ++s) {
    const int64_t ups = cdiv(cdiv(max_units, s), g) * g;
    if (ups < min_units) break;  // ups only shrinks as s grows
    const int64_t n = cdiv(max_units, ups);
    if (n > max_splits) continue;
    const int64_t c = cost(n, ups);
    if (c >= 0 && 100 * c < 95 * base_cost && c < best_cost) {
      best = {static_cast<int32_t>(n), static_cast<int32_t>(ups)};
      best_cost = c;
    }
  }
  return best;
}

bool plan_decode_order(const int32_t* units, const int64_t* mix_weight, int32_t n_seqs, int32_t n_splits,
                       int32_t units_per_split, int32_t n_mix, int32_t max_entries, std::vector<uint16_t>* order) {
  order->clear();
  const int32_t n_parts = n_splits + n_mix;
  const int64_t n = static_cast<int64_t>(n_seqs) * n_parts;
  if (n_seqs < 1 || n_seqs > 256 || n_parts < 1 || n_parts > 255 || n > max_entries) return false;
  std::vector<std::pair<int64_t, uint16_t>> items;  // (weight, entry) in the default order
  items.reserve(static_cast<size_t>(n));
  for (int32_t z = 0; z < n_parts; ++z) {
    for (int32_t i = 0; i < n_seqs; ++i) {
      const int64_t w = z < n_splits ? std::clamp<int64_t>(static_cast<int64_t>(units[i]) -
                                                               static_cast<int64_t>(z) * units_per_split,
                                                           0, units_per_split)
                                     : mix_weight[i];
      items.emplace_back(w, static_cast<uint16_t>((z << 8) | i));
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
  bool same = true;
  for (int64_t k = 0; k < n; ++k) {
    const int32_t z = static_cast<int32_t>(k / n_seqs), i = static_cast<int32_t>(k % n_seqs);
    same &= items[k].second == static_cast<uint16_t>((z << 8) | i);
  }
  if (same) return false;
  for (const auto& it : items) order->push_back(it.second);
  return true;
}

HostState::HostState(const vk_cache_config& cfg) : cfg_(cfg) {
  max_pages_ = static_cast<int32_t>(cdiv(cfg.max_tokens_per_seq, cfg.block_size));
  seqs_.resize(cfg.max_seqs);
  const int64_t caps[kFormats] = {cfg.pages_ternary, cfg.pages_fp8, cfg.pages_f16, cfg.pages_lossless};
  SplitMix64 rng{cfg.page_shuffle_seed};
  for (int f = 0; f < kFormats; ++f) {
    std::vector<int32_t> ids(caps[f]);
    for (int64_t i = 0; i < caps[f]; ++i) ids[i] = static_cast<int32_t>(i);
    if (cfg.page_shuffle_seed != 0) {
      for (int64_t i = caps[f] - 1; i > 0; --i) {
        int64_t j = static_cast<int64_t>(rng.next() % static_cast<uint64_t>(i + 1));
        std::swap(ids[i], ids[j]);
      }
    }
    free_[f].assign(ids.begin(), ids.end());
  }
}

int32_t HostState::new_page_format(int32_t page, int32_t new_len) const {
  const int64_t bs = cfg_.block_size;
  if (page < cdiv(cfg_.sink_tokens, bs)) return cfg_.sink_format;
  const int64_t lo = page * bs, hi = lo + bs;
  if (cfg_.recent_tokens > 0 && lo < new_len && hi > static_cast<int64_t>(new_len) - cfg_.recent_tokens)
    return cfg_.recent_format;
  return VK_FMT_TERNARY2;
}

vk_status HostState::plan_append(int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_tokens, AppendPlan* plan,
                                 std::string* err) const {
  if (n_seqs < 1 || n_seqs > cfg_.max_seqs) {
    *err = fmt_str("n_seqs %lld out of range [1, %lld]", n_seqs, cfg_.max_seqs);
    return VK_ERR_ARG;
  }
  if (!seq_ids) { *err = "seq_ids is NULL"; return VK_ERR_ARG; }
  if (!n_tokens) { *err = "n_tokens is NULL"; return VK_ERR_ARG; }
  std::unordered_set<int32_t> seen;
  const int32_t bs = cfg_.block_size;
  plan->seqs.clear();
  plan->entries.clear();
  plan->new_fmt.clear();
  plan->max_units = 0;
  plan->max_tern_tokens = 0;
  plan->total_tokens = 0;
  plan->total_tasks = 0;
  plan->total_blk = 0;
  for (int f = 0; f < kFormats; ++f) plan->new_pages[f] = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t s = seq_ids[i];
    if (s < 0 || s >= cfg_.max_seqs) { *err = fmt_str("seq id %lld out of range", s); return VK_ERR_ARG; }
    if (!seen.insert(s).second) { *err = fmt_str("seq id %lld repeated", s); return VK_ERR_ARG; }
    if (n_tokens[i] < 1) { *err = fmt_str("n_tokens[%lld] must be >= 1", i); return VK_ERR_ARG; }
    const SeqState& st = seqs_[s];
    const int64_t t0 = st.length, t1 = t0 + n_tokens[i];
    if (t1 > cfg_.max_tokens_per_seq) {
      *err = fmt_str("seq %lld would exceed max_tokens_per_seq (%lld)", s, cfg_.max_tokens_per_seq);
      return VK_ERR_ARG;
    }
    if (t0 % bs) {
      const int32_t e = st.pages[t0 / bs];
      if (e != kNoPage && (entry_fmt(e) == VK_FMT_TERNARY2 || entry_fmt(e) == VK_FMT_LOSSLESS)) {
        *err = fmt_str("seq %lld ends inside a ternary or lossless page (length %lld); such pages are written by "
                       "one append", s, t0);
        return VK_ERR_ALIGN;
      }
    }
    if (plan->total_tokens + n_tokens[i] > (int64_t{1} << 31) - 1) {
      *err = "more than 2^31 - 1 tokens in one call";
      return VK_ERR_ARG;
    }
    AppendSeqDesc d{};
    d.slot = s;
    d.t0 = static_cast<int32_t>(t0);
    d.n_tokens = n_tokens[i];
    d.tok_off = static_cast<int32_t>(plan->total_tokens);
    plan->total_tokens += n_tokens[i];
    d.page_first = static_cast<int32_t>(t0 / bs);
    d.page_off = static_cast<int32_t>(plan->entries.size());
    const int32_t page_end = static_cast<int32_t>(cdiv(t1, bs));
    d.n_pages = page_end - d.page_first;
    d.unit_first = static_cast<int32_t>(t0 / kUnit);
    const int32_t unit_end = static_cast<int32_t>(cdiv(t1, kUnit));
    plan->max_units = std::max(plan->max_units, unit_end - d.unit_first);
    int64_t tlo = t1, thi = t0;  // ternary token range (absolute)
    for (int32_t p = d.page_first; p < page_end; ++p) {
      if (p < static_cast<int32_t>(st.pages.size())) {
        plan->entries.push_back(st.pages[p]);  // existing partly filled page (fp8 / f16)
        continue;
      }
      const int32_t f = new_page_format(p, static_cast<int32_t>(t1));
      plan->new_pages[f] += 1;
      plan->new_fmt.push_back(f);
      plan->entries.push_back(make_entry(f, 0));  // index filled at commit
      if (f == VK_FMT_TERNARY2) {
        tlo = std::min<int64_t>(tlo, std::max<int64_t>(static_cast<int64_t>(p) * bs, t0));
        thi = std::max<int64_t>(thi, std::min<int64_t>(static_cast<int64_t>(p + 1) * bs, t1));
      }
    }
    if (thi > tlo) {
      d.tern_lo = static_cast<int32_t>(tlo - t0);
      d.tern_hi = static_cast<int32_t>(thi - t0);
    } else {
      d.tern_lo = d.tern_hi = 0;
    }
    plan->max_tern_tokens = std::max(plan->max_tern_tokens, d.tern_hi - d.tern_lo);
    // pack tasks: (16-token unit, K|V, KV head); absmean blocks: kAbsBlockElems elements each
    d.task_off = static_cast<int32_t>(plan->total_tasks);
    d.blk_off = static_cast<int32_t>(plan->total_blk);
    plan->total_tasks += static_cast<int64_t>(unit_end - d.unit_first) * 2 * cfg_.n_kv_heads;
    plan->total_blk += cdiv(static_cast<int64_t>(d.tern_hi - d.tern_lo) * cfg_.n_kv_heads * cfg_.head_dim,
                            kAbsBlockElems);
    if (plan->total_tasks > (int64_t{1} << 30) || plan->total_blk > (int64_t{1} << 30)) {
      *err = "append too large for one call; split it";
      return VK_ERR_ARG;
    }
    plan->seqs.push_back(d);
  }
  for (int f = 0; f < kFormats; ++f) {
    if (plan->new_pages[f] > static_cast<int64_t>(free_[f].size())) {
      static const char* names[kFormats] = {"ternary", "fp8", "f16", "lossless"};
      char buf[160];
      std::snprintf(buf, sizeof buf, "pool of %s pages exhausted: need %lld, %lld free", names[f],
                    static_cast<long long>(plan->new_pages[f]), static_cast<long long>(free_[f].size()));
      *err = buf;
      return VK_ERR_CAPACITY;
    }
  }
  return VK_OK;
}

void HostState::commit_append(AppendPlan* plan) {
  const int32_t bs = cfg_.block_size;
  for (AppendSeqDesc& d : plan->seqs) {
    SeqState& st = seqs_[d.slot];
    for (int32_t j = 0; j < d.n_pages; ++j) {
      const int32_t p = d.page_first + j;
      int32_t& e = plan->entries[d.page_off + j];
      if (p < static_cast<int32_t>(st.pages.size())) continue;
      const int f = entry_fmt(e);
      const int32_t idx = free_[f].front();
      free_[f].pop_front();
      e = make_entry(f, idx);
      st.pages.push_back(e);
      if (st.runs.empty() || st.runs.back().second != f) st.runs.emplace_back(p, f);
    }
    st.length += d.n_tokens;
  }
  (void)bs;
}

vk_status HostState::plan_retier(int32_t n_seqs, const int32_t* seq_ids, RetierPlan* plan,
                                 std::string* err) const {
  if (n_seqs < 1 || n_seqs > cfg_.max_seqs) {
    *err = fmt_str("n_seqs %lld out of range [1, %lld]", n_seqs, cfg_.max_seqs);
    return VK_ERR_ARG;
  }
  if (!seq_ids) { *err = "seq_ids is NULL"; return VK_ERR_ARG; }
  std::unordered_set<int32_t> seen;
  plan->tasks.clear();
  plan->page_end.clear();
  const int64_t bs = cfg_.block_size;
  const int32_t first = static_cast<int32_t>(cdiv(cfg_.sink_tokens, bs));
  const bool tiered = cfg_.recent_tokens > 0 && cfg_.recent_format == VK_FMT_FP8E4M3;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t s = seq_ids[i];
    if (s < 0 || s >= cfg_.max_seqs) { *err = fmt_str("seq id %lld out of range", s); return VK_ERR_ARG; }
    if (!seen.insert(s).second) { *err = fmt_str("seq id %lld repeated", s); return VK_ERR_ARG; }
    const SeqState& st = seqs_[s];
    // pages [0, end) end at or before length - R
    const int64_t settled = static_cast<int64_t>(st.length) - cfg_.recent_tokens;
    const int32_t end = tiered && settled > 0 ? static_cast<int32_t>(settled / bs) : st.retier_from;
    for (int32_t p = std::max(st.retier_from, first); p < end; ++p)
      if (st.pages[p] != kNoPage && entry_fmt(st.pages[p]) == VK_FMT_FP8E4M3)
        plan->tasks.push_back({s, p, entry_idx(st.pages[p]), 0});
    plan->page_end.push_back(std::max(end, st.retier_from));
  }
  if (static_cast<int64_t>(plan->tasks.size()) > static_cast<int64_t>(free_[VK_FMT_TERNARY2].size())) {
    *err = fmt_str("pool of ternary pages exhausted: need %lld, %lld free", static_cast<int64_t>(plan->tasks.size()),
                   static_cast<int64_t>(free_[VK_FMT_TERNARY2].size()));
    return VK_ERR_CAPACITY;
  }
  return VK_OK;
}

void HostState::commit_retier(int32_t n_seqs, const int32_t* seq_ids, RetierPlan* plan) {
  for (RetierTask& t : plan->tasks) {
    t.dst = free_[VK_FMT_TERNARY2].front();
    free_[VK_FMT_TERNARY2].pop_front();
    free_[VK_FMT_FP8E4M3].push_back(t.src);
    seqs_[t.slot].pages[t.page] = make_entry(VK_FMT_TERNARY2, t.dst);
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    SeqState& st = seqs_[seq_ids[i]];
    st.retier_from = plan->page_end[i];
  }
  if (plan->tasks.empty()) return;
  for (int32_t i = 0; i < n_seqs; ++i) {  // rebuild the same-format runs of the changed sequences
    SeqState& st = seqs_[seq_ids[i]];
    st.runs.clear();
    for (size_t p = 0; p < st.pages.size(); ++p) {
      const int f = st.pages[p] == kNoPage ? kFormats : entry_fmt(st.pages[p]);
      if (st.runs.empty() || st.runs.back().second != f) st.runs.emplace_back(static_cast<int32_t>(p), f);
    }
  }
}

vk_status HostState::evict(int32_t n_seqs, const int32_t* seq_ids, int32_t window, int64_t* n_pages,
                           std::string* err) {
  if (n_seqs < 1 || n_seqs > cfg_.max_seqs) {
    *err = fmt_str("n_seqs %lld out of range [1, %lld]", n_seqs, cfg_.max_seqs);
    return VK_ERR_ARG;
  }
  if (!seq_ids) { *err = "seq_ids is NULL"; return VK_ERR_ARG; }
  if (window < -1) { *err = "window must be >= -1"; return VK_ERR_ARG; }
  std::unordered_set<int32_t> seen;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t s = seq_ids[i];
    if (s < 0 || s >= cfg_.max_seqs) { *err = fmt_str("seq id %lld out of range", s); return VK_ERR_ARG; }
    if (!seen.insert(s).second) { *err = fmt_str("seq id %lld repeated", s); return VK_ERR_ARG; }
  }
  int64_t freed = 0;
  if (window >= 0) {
    const int64_t bs = cfg_.block_size;
    const int32_t first = static_cast<int32_t>(cdiv(cfg_.sink_tokens, bs));
    for (int32_t i = 0; i < n_seqs; ++i) {
      SeqState& st = seqs_[seq_ids[i]];
      const int64_t edge = static_cast<int64_t>(st.length) - window;  // pages ending by here go
      const int32_t last = edge > 0 ? static_cast<int32_t>(edge / bs) : 0;
      const int32_t from = std::max(st.evict_end, first);
      if (last <= from) continue;
      for (int32_t p = from; p < last; ++p) {
        const int32_t e = st.pages[p];
        free_[entry_fmt(e)].push_back(entry_idx(e));
        st.pages[p] = kNoPage;
        ++freed;
      }
      st.evict_end = last;
      st.runs.clear();
      for (size_t p = 0; p < st.pages.size(); ++p) {
        const int f = st.pages[p] == kNoPage ? kFormats : entry_fmt(st.pages[p]);
        if (st.runs.empty() || st.runs.back().second != f) st.runs.emplace_back(static_cast<int32_t>(p), f);
      }
    }
  }
  if (n_pages) *n_pages = freed;
  return VK_OK;
}

vk_status HostState::check_decode(int32_t n_seqs, const int32_t* seq_ids, int32_t window, std::string* err) const {
  if (n_seqs < 1) { *err = "n_seqs must be >= 1"; return VK_ERR_ARG; }
  if (!seq_ids) { *err = "seq_ids is NULL"; return VK_ERR_ARG; }
  if (window < -1) { *err = "window must be >= -1"; return VK_ERR_ARG; }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t s = seq_ids[i];
    if (s < 0 || s >= cfg_.max_seqs) { *err = fmt_str("seq id %lld out of range", s); return VK_ERR_ARG; }
    const SeqState& st = seqs_[s];
    if (st.length < 1) { *err = fmt_str("seq %lld is empty", s); return VK_ERR_ARG; }
    // tokens [sink pages * Bs, evict_end * Bs) are gone: the window must start at or after them
    const int64_t gone_end = static_cast<int64_t>(st.evict_end) * cfg_.block_size;
    if (gone_end > 0 && (window < 0 || static_cast<int64_t>(st.length) - window < gone_end)) {
      *err = fmt_str("seq %lld: the window reaches tokens freed by eviction (below %lld)", s, gone_end);
      return VK_ERR_ARG;
    }
  }
  return VK_OK;
}

void HostState::count_units(int32_t slot, int32_t window, int64_t out[kFormats]) const {
  const SeqState& st = seqs_[slot];
  const UnitRanges r = attended_units(st.length, cfg_.sink_tokens, window);
  const int64_t upp = cfg_.block_size / kUnit;
  const int64_t n_pages = static_cast<int64_t>(st.pages.size());
  for (size_t k = 0; k < st.runs.size(); ++k) {
    const int64_t p0 = st.runs[k].first;
    const int64_t p1 = k + 1 < st.runs.size() ? st.runs[k + 1].first : n_pages;
    const int64_t u0 = p0 * upp, u1 = p1 * upp;
    int64_t n = std::max<int64_t>(0, std::min<int64_t>(u1, r.a_end) - u0);
    n += std::max<int64_t>(0, std::min<int64_t>(u1, r.b_end) - std::max<int64_t>(u0, r.b_begin));
    if (st.runs[k].second < kFormats) out[st.runs[k].second] += n;  // freed pages are never attended
  }
}

void HostState::mixed_ranges(int32_t slot, int32_t window, int32_t out[4]) const {
  const SeqState& st = seqs_[slot];
  const UnitRanges r = attended_units(st.length, cfg_.sink_tokens, window);
  const int64_t upp = cfg_.block_size / kUnit;
  const int64_t n_pages = static_cast<int64_t>(st.pages.size());
  // logical intervals of the non-ternary runs, in order: the sink range first, then the window
  std::vector<std::pair<int64_t, int64_t>> iv;
  for (int part = 0; part < 2; ++part) {
    const int64_t lo = part == 0 ? 0 : r.b_begin, hi = part == 0 ? r.a_end : r.b_end;
    const int64_t base = part == 0 ? 0 : r.a_end - r.b_begin;  // unit -> logical unit
    for (size_t k = 0; k < st.runs.size(); ++k) {
      const int fmt = st.runs[k].second;
      if (fmt == VK_FMT_TERNARY2 || fmt >= kFormats) continue;  // freed pages are never attended
      const int64_t p0 = st.runs[k].first;
      const int64_t p1 = k + 1 < st.runs.size() ? st.runs[k + 1].first : n_pages;
      const int64_t u0 = std::max(p0 * upp, lo), u1 = std::min(p1 * upp, hi);
      if (u0 < u1) iv.emplace_back(u0 + base, u1 + base);
    }
  }
  out[0] = out[1] = out[2] = out[3] = 0;
  if (iv.empty()) return;
  size_t cut = iv.size() - 1;  // the two ranges are iv[0 .. cut] and iv[cut + 1 ..]
  int64_t widest = -1;
  for (size_t k = 0; k + 1 < iv.size(); ++k)
    if (iv[k + 1].first - iv[k].second > widest) widest = iv[k + 1].first - iv[k].second, cut = k;
  out[0] = static_cast<int32_t>(iv.front().first);
  out[1] = static_cast<int32_t>(iv[cut].second);
  if (cut + 1 < iv.size()) {
    out[2] = static_cast<int32_t>(iv[cut + 1].first);
    out[3] = static_cast<int32_t>(iv.back().second);
  }
}

vk_status HostState::reset_seqs(int32_t n_seqs, const int32_t* seq_ids, std::string* err) {
  if (n_seqs < 0 || (n_seqs > 0 && !seq_ids)) { *err = "bad seq list"; return VK_ERR_ARG; }
  std::unordered_set<int32_t> seen;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (seq_ids[i] < 0 || seq_ids[i] >= cfg_.max_seqs) { *err = fmt_str("seq id %lld out of range", seq_ids[i]); return VK_ERR_ARG; }
    if (!seen.insert(seq_ids[i]).second) { *err = fmt_str("seq id %lld repeated", seq_ids[i]); return VK_ERR_ARG; }
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    SeqState& st = seqs_[seq_ids[i]];
    for (int32_t e : st.pages)
      if (e != kNoPage) free_[entry_fmt(e)].push_back(entry_idx(e));
    st = SeqState();
  }
  return VK_OK;
}

int64_t HostState::pages_used(int fmt) const {
  const int64_t caps[kFormats] = {cfg_.pages_ternary, cfg_.pages_fp8, cfg_.pages_f16, cfg_.pages_lossless};
  return caps[fmt] - static_cast<int64_t>(free_[fmt].size());
}

int64_t HostState::tokens_stored(int fmt) const {
  int64_t n = 0;
  const int64_t bs = cfg_.block_size;
  for (const SeqState& st : seqs_) {
    for (size_t p = 0; p < st.pages.size(); ++p) {
      if (st.pages[p] == kNoPage || entry_fmt(st.pages[p]) != fmt) continue;
      n += std::min<int64_t>(bs, st.length - static_cast<int64_t>(p) * bs);
    }
  }
  return n;
}

}  // namespace vk
