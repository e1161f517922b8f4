// Test-only C shim over the HIP-free host state (page allocator, tier
// router, planners), so the host logic can be checked on a machine without
// a GPU.  Built by the tests with g++; not part of libvk.so.
#include <vector>
#include <cstring>
#include <string>

#include "host_state.h"

extern "C" {

void* hs_create(const vk_cache_config* cfg, char* err, int errlen) {
  const std::string why = vk::validate_config(*cfg);
  if (!why.empty()) {
    std::strncpy(err, why.c_str(), errlen - 1);
    err[errlen - 1] = 0;
    return nullptr;
  }
  return new vk::HostState(*cfg);
}

void hs_destroy(void* h) { delete static_cast<vk::HostState*>(h); }

// Plans and, on success, commits an append.  Returns the status; fills the
// per-seq ternary token ranges (2 ints per seq) and pages taken per format.
int hs_append(void* h, int n_seqs, const int* ids, int n_tokens, int* tern_ranges, long long* new_pages,
              char* err, int errlen) {
  auto* s = static_cast<vk::HostState*>(h);
  vk::AppendPlan plan;
  std::string e;
  std::vector<int> counts(n_seqs > 0 ? n_seqs : 0, n_tokens);
  const vk_status st = s->plan_append(n_seqs, ids, counts.data(), &plan, &e);
  if (st) {
    std::strncpy(err, e.c_str(), errlen - 1);
    err[errlen - 1] = 0;
    return st;
  }
  s->commit_append(&plan);
  for (size_t i = 0; i < plan.seqs.size(); ++i) {
    tern_ranges[2 * i] = plan.seqs[i].tern_lo;
    tern_ranges[2 * i + 1] = plan.seqs[i].tern_hi;
  }
  for (int f = 0; f < 3; ++f) new_pages[f] = plan.new_pages[f];   // (the tests use three formats)
  return 0;
}

// Plans and, on success, commits a retier.  Returns the status; fills up to max_tasks
// (slot, page, src, dst) quadruples and *n_tasks.
int hs_retier(void* h, int n_seqs, const int* ids, int* tasks, int max_tasks, int* n_tasks, char* err, int errlen) {
  auto* s = static_cast<vk::HostState*>(h);
  vk::RetierPlan plan;
  std::string e;
  const vk_status st = s->plan_retier(n_seqs, ids, &plan, &e);
  if (st) {
    std::strncpy(err, e.c_str(), errlen - 1);
    err[errlen - 1] = 0;
    return st;
  }
  s->commit_retier(n_seqs, ids, &plan);
  *n_tasks = static_cast<int>(plan.tasks.size());
  for (int i = 0; i < *n_tasks && i < max_tasks; ++i) {
    tasks[4 * i] = plan.tasks[i].slot;
    tasks[4 * i + 1] = plan.tasks[i].page;
    tasks[4 * i + 2] = plan.tasks[i].src;
    tasks[4 * i + 3] = plan.tasks[i].dst;
  }
  return 0;
}

int hs_evict(void* h, int n_seqs, const int* ids, int window, long long* n_pages) {
  std::string e;
  int64_t n = 0;
  const int st = static_cast<vk::HostState*>(h)->evict(n_seqs, ids, window, &n, &e);
  *n_pages = n;
  return st;
}

int hs_check_decode(void* h, int n_seqs, const int* ids, int window) {
  std::string e;
  return static_cast<vk::HostState*>(h)->check_decode(n_seqs, ids, window, &e);
}

void hs_mixed_ranges(void* h, int seq, int window, int* out4) {
  static_cast<vk::HostState*>(h)->mixed_ranges(seq, window, out4);
}
int hs_length(void* h, int seq) { return static_cast<vk::HostState*>(h)->seq(seq).length; }
int hs_n_pages(void* h, int seq) { return static_cast<int>(static_cast<vk::HostState*>(h)->seq(seq).pages.size()); }
int hs_page_entry(void* h, int seq, int page) { return static_cast<vk::HostState*>(h)->seq(seq).pages[page]; }
long long hs_free_pages(void* h, int fmt) { return static_cast<vk::HostState*>(h)->free_pages(fmt); }
long long hs_tokens_stored(void* h, int fmt) { return static_cast<vk::HostState*>(h)->tokens_stored(fmt); }

void hs_count_units(void* h, int seq, int window, long long* out3) {
  int64_t o[vk::kFormats] = {};
  static_cast<vk::HostState*>(h)->count_units(seq, window, o);
  for (int f = 0; f < 3; ++f) out3[f] = o[f];
}

int hs_reset(void* h, int n, const int* ids) {
  std::string e;
  return static_cast<vk::HostState*>(h)->reset_seqs(n, ids, &e);
}

void hs_attended_units(int length, int sinks, int window, int* out3) {
  const vk::UnitRanges r = vk::attended_units(length, sinks, window);
  out3[0] = r.a_end;
  out3[1] = r.b_begin;
  out3[2] = r.b_end;
}

int hs_plan_splits(long long total_units, int max_units, int target, int max_splits, int min_units, int granule,
                   int* units_per_split) {
  const vk::SplitPlan p = vk::plan_splits(total_units, max_units, target, max_splits, min_units, granule);
  *units_per_split = p.units_per_split;
  return p.n_splits;
}

int hs_balance_splits(int base_splits, int base_ups, long long items, int max_units, int n_cu, int max_per_cu,
                      int max_splits, int min_units, int granule, int* units_per_split) {
  const vk::SplitPlan p = vk::balance_splits({base_splits, base_ups}, items, max_units, n_cu, max_per_cu, max_splits,
                                             min_units, granule);
  *units_per_split = p.units_per_split;
  return p.n_splits;
}

// dispatch order of a decode launch: returns the entry count (0 = the plain grid's order)
int hs_plan_decode_order(const int* units, const long long* mix_weight, int n_seqs, int n_splits,
                         int units_per_split, int n_mix, int max_entries, unsigned short* out) {
  std::vector<int64_t> w(mix_weight, mix_weight + n_seqs);
  std::vector<uint16_t> order;
  if (!vk::plan_decode_order(units, w.data(), n_seqs, n_splits, units_per_split, n_mix, max_entries, &order))
    return 0;
  for (size_t k = 0; k < order.size(); ++k) out[k] = order[k];
  return static_cast<int>(order.size());
}
}
