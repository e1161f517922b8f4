// C ABI of libvk.so (see include/vk.h).  Owns every device buffer; plans on
// the host (host_state.cpp) and launches the HIP kernels (vk_write.hip,
// vk_decode.hip, vk_retier.hip) on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <string>
#include <vector>

#include "host_state.h"
#include "vk.h"
#include "vk_params.h"

namespace {

thread_local std::string g_error;

vk_status fail(vk_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

constexpr int kRingMax = 64;             // append / retier plan staging slots, at most
constexpr int kRingMin = 4;              // ... at least
constexpr int64_t kRingBytes = 64 << 20; // pinned bytes the slots may take together (beyond kRingMin)
constexpr int64_t kPackTargetBlocks = 32768;  // pack blocks per launch, at most
constexpr int64_t kPackPipeMaxTasks = 16;      // pipelined pack: tasks per block, at most
constexpr int64_t kRetierTasksPerLaunch = 65536;  // pages one retier launch converts, at most
constexpr int64_t kMaxPartials = 1 << 20;  // float64 absmean partials per append call
constexpr int kDecodeTargetGroups = 4096;  // work groups a decode launch aims for
constexpr int kDecodeMaxSplits = 64;
constexpr int kDecodeMinUnits = 4;         // 16-token units per split, at least (vector-ALU kernel)
constexpr int kDecodeMaxResidentBlocks = 3;  // matrix-core kernel, head dims 64 / 128: blocks per CU at once
constexpr int kDecodeMinUnitsPerWave = 8;  // matrix-core kernel: units per wave, at least
constexpr int kDecodeUnitsPerStep = 4;     // matrix-core kernel: units per clean step, at most (a wave's
                                           // range is a whole number of them when the split size is)
constexpr int64_t kDecodeScratchItems = 16384;  // (seq, q-head group, split) partial slots
// matrix-core decode blocks per compute unit a launch aims for (3 four-wave blocks fit one at
// the kernel's 3 waves per SIMD; 2 larger ones measured faster than 3 or 4 on 128K-token
// contexts, where each wave's set-up is a larger share of its work, and no slower on 32K ones).
// VK_DECODE_BLOCKS_PER_CU=1..8 overrides.
int decode_blocks_per_cu() {
  const char* e = std::getenv("VK_DECODE_BLOCKS_PER_CU");
  const int v = e ? std::atoi(e) : 0;
  return v >= 1 && v <= 8 ? v : 2;
}
// matrix-core kernel: blocks per (sequence, KV head) for fp8 / fp16 pages (at most kDecodeMixedPartsMax;
// VK_DECODE_MIX_PARTS=1..4 overrides)
constexpr int kDecodeMixedPartsMax = 4;
int decode_mixed_parts() {
  const char* e = std::getenv("VK_DECODE_MIX_PARTS");
  const int v = e ? std::atoi(e) : 0;
  return v >= 1 && v <= kDecodeMixedPartsMax ? v : 1;
}
// Short all-ternary appends at head dims 64 and 128 run the pipelined pack kernel (VK_PACK_PIPE=0:
// k_pack's one-task blocks) with VK_PACK_BLOCKS_PER_CU blocks per compute unit at most (default 16:
// the kernel's 120 registers leave room for 4 waves per SIMD, 16 one-wave blocks per CU).
bool pack_pipelined_on() {
  const char* e = std::getenv("VK_PACK_PIPE");
  return !(e && e[0] == '0');
}
int pack_blocks_per_cu() {
  const char* e = std::getenv("VK_PACK_BLOCKS_PER_CU");
  const int v = e ? std::atoi(e) : 0;
  return v >= 1 && v <= 64 ? v : 16;
}
// Matrix-core launches with several parts (and no lossless pages) merge them in the kernel: the
// last block to finish a (sequence, KV head) combines its parts, and no k_merge launch follows.
// VK_DECODE_FUSED_MERGE=0 keeps the merge launch.
bool decode_fused_merge_on() {
  const char* e = std::getenv("VK_DECODE_FUSED_MERGE");
  return !(e && e[0] == '0');
}
// Launches over sequences of different lengths (or with fp8 / fp16 parts) dispatch their blocks
// heaviest first from an order table.  VK_DECODE_ORDER=0 keeps the plain grid;
// VK_DECODE_BLOCKS_PER_CU_RAGGED=1..8 sets such launches' split target (default: as the others);
// VK_DECODE_MIX_FIXED=n: an fp8 / fp16 part weighs n units beyond its pages' bytes in 1 KB units.
bool decode_order_on() {
  const char* e = std::getenv("VK_DECODE_ORDER");
  return !(e && e[0] == '0');
}
int decode_blocks_per_cu_ragged() {
  const char* e = std::getenv("VK_DECODE_BLOCKS_PER_CU_RAGGED");
  const int v = e ? std::atoi(e) : 0;
  return v >= 1 && v <= 8 ? v : decode_blocks_per_cu();
}
int64_t decode_mix_fixed() {
  const char* e = std::getenv("VK_DECODE_MIX_FIXED");
  const long long v = e ? std::atoll(e) : -1;
  return v >= 0 ? v : 0;
}
// Equal-length all-ternary matrix-core launches re-weigh their split count so that the busiest
// compute unit holds as few units as the blocks' residency allows (balance_splits).
// VK_DECODE_BALANCE=0, or a VK_DECODE_BLOCKS_PER_CU override, keeps the plain plan.
bool decode_balance_on() {
  const char* e = std::getenv("VK_DECODE_BALANCE");
  return !(e && e[0] == '0') && !std::getenv("VK_DECODE_BLOCKS_PER_CU");
}
int decode_units_per_iter() {              // matrix-core prefetch depth in units; VK_DECODE_UPI=4|8 overrides
  const char* e = std::getenv("VK_DECODE_UPI");
  return (e && e[0] == '4') ? 4 : 8;
}
constexpr int32_t kStealPiece = 16;            // units a stealing wave takes at a time
constexpr int64_t kStealMinUnitsPerCu = 256;   // stealing launches: units per compute unit, at least
// Stealing blocks (opt-in: which wave sums which units changes from call to call, so outputs
// repeat only within the decode tolerance).  VK_DECODE_STEAL=1: large launches (by size);
// =2: whenever the launch's shape allows; unset or 0: never.
int decode_steal_mode() {
  const char* e = std::getenv("VK_DECODE_STEAL");
  return (e && e[0] == '1') ? 1 : (e && e[0] == '2') ? 2 : 0;
}

// Per-kind launch timing with HIP event pairs recorded on the launch stream.
class EventTimer : public vk::LaunchTimer {
 public:
  bool on = false;
  int64_t launches[VK_KERNEL_COUNT] = {};
  double ms[VK_KERNEL_COUNT] = {};
  double bytes[VK_KERNEL_COUNT] = {};

  ~EventTimer() override {
    for (Rec& r : pending_) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
    for (hipEvent_t e : pool_) (void)hipEventDestroy(e);
  }
  void reset() {
    flush();
    for (int k = 0; k < VK_KERNEL_COUNT; ++k) launches[k] = 0, ms[k] = 0.0, bytes[k] = 0.0;
  }
  void add_bytes(int kind, double b) {
    if (on) bytes[kind] += b;
  }
  void begin(int kind, hipStream_t s) override {
    if (!on) return;
    open_ = Rec{kind, get(), get()};
    (void)hipEventRecord(open_.a, s);
  }
  void end(int kind, hipStream_t s) override {
    if (!on || open_.kind != kind) return;
    (void)hipEventRecord(open_.b, s);
    pending_.push_back(open_);
    launches[kind] += 1;
    open_.kind = -1;
    if (pending_.size() >= (1u << 16)) flush();  // (a flush waits for the device)
  }
  // Waits for every recorded pair and folds it into the totals.
  void flush() {
    for (Rec& r : pending_) {
      float t = 0.0f;
      if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) ms[r.kind] += t;
      pool_.push_back(r.a);
      pool_.push_back(r.b);
    }
    pending_.clear();
  }

 private:
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  hipEvent_t get() {
    if (!pool_.empty()) {
      hipEvent_t e = pool_.back();
      pool_.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    (void)hipEventCreate(&e);
    return e;
  }
  std::vector<Rec> pending_;
  std::vector<hipEvent_t> pool_;
  Rec open_{-1, nullptr, nullptr};
};

}  // namespace

struct vk_cache {
  vk_cache_config cfg;
  std::unique_ptr<vk::HostState> host;
  int device = 0;
  int n_cu = 0;  // compute units of the device
  bool poisoned = false;
  vk::PoolsView pools{};
  double* partials = nullptr;
  float* dec_partials = nullptr;
  uint32_t* part_count = nullptr;  // decode: parts finished per (sequence, KV head); 0 between launches
  int64_t plan_bytes = 0;
  int n_ring = kRingMin;  // staging slots in use (ring_slots of the config)
  uint8_t* plan_host[kRingMax] = {};
  uint8_t* plan_dev[kRingMax] = {};
  hipEvent_t plan_ev[kRingMax] = {};
  bool plan_ev_used[kRingMax] = {};
  int ring_next = 0;
  int64_t device_bytes = 0;
  std::vector<void*> allocations;
  vk_stats stats{};
  EventTimer timer;
};

namespace {

vk_status hip_fail(vk_cache* c, hipError_t e, const char* what) {
  if (c) c->poisoned = true;
  return fail(VK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t partial_count(const vk_cache_config& cfg) {
  const int g = cfg.n_q_heads / cfg.n_kv_heads;
  return kDecodeScratchItems * g * (cfg.head_dim + 2);
}

int64_t plan_bytes_for(const vk_cache_config& cfg) {
  const int64_t max_pages = (cfg.max_tokens_per_seq + cfg.block_size - 1) / cfg.block_size;
  // descriptors, block-table entries and (with a lossless tier) the call's lossless units: the
  // sink pages and the pages the recent tier can hold, two int32 per 16-token unit
  const int64_t upp = cfg.block_size / vk::kUnit;
  // (and, with an fp8 / fp16 tier, the call's units of those pages: a page is of one format, so
  // both lists together stay within the same bound)
  const bool ll = cfg.sink_format != VK_FMT_TERNARY2 || (cfg.recent_tokens > 0 && cfg.recent_format != VK_FMT_TERNARY2);
  const int64_t ll_pages = ll ? (cfg.sink_tokens + cfg.block_size - 1) / cfg.block_size +
                                    (cfg.recent_tokens + cfg.block_size - 1) / cfg.block_size + 2
                              : 0;
  const int64_t append = static_cast<int64_t>(cfg.max_seqs) *
                         (sizeof(vk::AppendSeqDesc) + 4 * (max_pages + 1) + 8 * upp * std::min(ll_pages, max_pages));
  // a retier of every page of every sequence in one launch, up to kRetierTasksPerLaunch
  const int64_t retier = std::min<int64_t>(static_cast<int64_t>(cfg.max_seqs) * max_pages, kRetierTasksPerLaunch) *
                         static_cast<int64_t>(sizeof(vk::RetierTask));
  const int64_t b = std::max(append, retier);
  return (b + 255) & ~int64_t(255);
}

// Plan staging slots: as many as fit kRingBytes, between kRingMin and kRingMax.  A call waits on
// the host only when every slot still holds a plan the device has not consumed.
int ring_slots(const vk_cache_config& cfg) {
  const int64_t fit = kRingBytes / plan_bytes_for(cfg);
  return static_cast<int>(std::max<int64_t>(kRingMin, std::min<int64_t>(kRingMax, fit)));
}

// Device bytes of every buffer vk_create_cache allocates, in allocation order.
std::vector<int64_t> buffer_sizes(const vk_cache_config& cfg) {
  std::vector<int64_t> s;
  const int64_t caps[3] = {cfg.pages_ternary, cfg.pages_fp8, cfg.pages_f16};
  for (int f = 0; f < 3; ++f) s.push_back(static_cast<int64_t>(cfg.n_layers) * caps[f] * vk::page_bytes(cfg, f));
  s.push_back(static_cast<int64_t>(cfg.n_layers) * caps[0] * 2 * 4);  // gamma
  const int64_t max_pages = (cfg.max_tokens_per_seq + cfg.block_size - 1) / cfg.block_size;
  s.push_back(static_cast<int64_t>(cfg.max_seqs) * max_pages * 4);    // block table
  s.push_back(kMaxPartials * 8);                                      // absmean partials
  s.push_back(partial_count(cfg) * 4);                                // decode split partials
  const int rs = ring_slots(cfg);
  for (int r = 0; r < kRingMax; ++r) s.push_back(r < rs ? plan_bytes_for(cfg) : 0);  // staged plans
  s.push_back(vk::page_bytes(cfg, VK_FMT_TERNARY2));                          // dummy page
  s.push_back(static_cast<int64_t>(cfg.n_layers) * cfg.pages_lossless * vk::page_bytes(cfg, VK_FMT_LOSSLESS));
  s.push_back(kDecodeScratchItems * 4);  // decode part counters, one per (sequence, KV head) of a launch
  return s;
}
constexpr size_t kBufDummy = 7 + kRingMax, kBufLossless = 8 + kRingMax, kBufCount = 9 + kRingMax;  // indices in buffer_sizes

void free_all(vk_cache* c) {
  for (void* p : c->allocations) (void)hipFree(p);
  c->allocations.clear();
  for (int r = 0; r < kRingMax; ++r) {
    if (c->plan_host[r]) (void)hipHostFree(c->plan_host[r]);
    if (c->plan_ev[r]) (void)hipEventDestroy(c->plan_ev[r]);
    c->plan_host[r] = nullptr;
    c->plan_ev[r] = nullptr;
  }
}

vk_status check_handle(vk_cache* c) {
  if (!c) return fail(VK_ERR_ARG, "cache handle is NULL");
  if (c->poisoned) return fail(VK_ERR_STATE, "cache handle poisoned by an earlier HIP failure");
  return VK_OK;
}

vk_status set_device(vk_cache* c) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(c, e, "hipGetDevice");
  if (cur != c->device) {
    e = hipSetDevice(c->device);
    if (e != hipSuccess) return hip_fail(c, e, "hipSetDevice");
  }
  return VK_OK;
}

}  // namespace

extern "C" {

VK_API void vk_config_defaults(vk_cache_config* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof *cfg);
  cfg->sink_tokens = 4;
  cfg->sink_format = VK_FMT_TERNARY2;
  cfg->recent_tokens = 0;
  cfg->recent_format = VK_FMT_FP8E4M3;
  cfg->eps = 1e-5f;
  cfg->fp8_scale = 1.0f;
}

VK_API vk_status vk_cache_device_bytes(const vk_cache_config* cfg, int64_t* bytes) {
  if (!cfg || !bytes) return fail(VK_ERR_ARG, "NULL argument");
  const std::string why = vk::validate_config(*cfg);
  if (!why.empty()) return fail(VK_ERR_ARG, "%s", why.c_str());
  int64_t total = 0;
  for (int64_t s : buffer_sizes(*cfg)) total += s;
  *bytes = total;
  return VK_OK;
}

VK_API int64_t vk_page_bytes(const vk_cache_config* cfg, int32_t fmt) {
  if (!cfg || fmt < 0 || fmt > VK_FMT_LOSSLESS || !vk::validate_config(*cfg).empty()) return 0;
  return vk::page_bytes(*cfg, fmt);
}

VK_API vk_status vk_create_cache(const vk_cache_config* cfg, vk_cache** out) {
  if (!cfg || !out) return fail(VK_ERR_ARG, "NULL argument");
  const std::string why = vk::validate_config(*cfg);
  if (!why.empty()) return fail(VK_ERR_ARG, "%s", why.c_str());
  std::unique_ptr<vk_cache> c(new vk_cache());
  c->cfg = *cfg;
  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) return fail(VK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  e = hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device);
  if (e != hipSuccess) return fail(VK_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  const std::vector<int64_t> sizes = buffer_sizes(*cfg);
  std::vector<void*> ptrs(sizes.size(), nullptr);
  for (size_t i = 0; i < sizes.size(); ++i) {
    if (sizes[i] == 0) continue;
    e = hipMalloc(&ptrs[i], static_cast<size_t>(sizes[i]));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      c->allocations = ptrs;
      free_all(c.get());
      return fail(VK_ERR_OOM, "hipMalloc of %lld bytes failed: %s", static_cast<long long>(sizes[i]),
                  hipGetErrorString(e));
    }
    c->device_bytes += sizes[i];
  }
  c->allocations = ptrs;
  // pools and gamma start zeroed (finite bytes everywhere); the block table starts empty;
  // the dummy page (target of speculative decode loads) is zero too
  for (size_t i : {size_t(0), size_t(1), size_t(2), size_t(3), kBufDummy, kBufLossless, kBufCount})
    if (ptrs[i]) {
      e = hipMemset(ptrs[i], 0, static_cast<size_t>(sizes[i]));
      if (e != hipSuccess) { free_all(c.get()); return fail(VK_ERR_HIP, "hipMemset: %s", hipGetErrorString(e)); }
    }
  e = hipMemset(ptrs[4], 0xFF, static_cast<size_t>(sizes[4]));
  if (e != hipSuccess) { free_all(c.get()); return fail(VK_ERR_HIP, "hipMemset: %s", hipGetErrorString(e)); }
  vk::PoolsView& P = c->pools;
  const int64_t caps[4] = {cfg->pages_ternary, cfg->pages_fp8, cfg->pages_f16, cfg->pages_lossless};
  for (int f = 0; f < 4; ++f) {
    P.pool[f] = static_cast<uint8_t*>(ptrs[f < 3 ? f : kBufLossless]);
    P.cap[f] = caps[f];
    P.tile_bytes[f] = vk::tile_bytes(*cfg, f);
    P.page_bytes[f] = vk::page_bytes(*cfg, f);
  }
  P.gamma = static_cast<float*>(ptrs[3]);
  P.block_table = static_cast<int32_t*>(ptrs[4]);
  P.max_pages = static_cast<int32_t>((cfg->max_tokens_per_seq + cfg->block_size - 1) / cfg->block_size);
  P.n_layers = cfg->n_layers;
  P.hkv = cfg->n_kv_heads;
  P.dim = cfg->head_dim;
  P.bs = cfg->block_size;
  P.bs_shift = 0;
  while ((1 << P.bs_shift) < cfg->block_size) ++P.bs_shift;
  P.fp8_scale = cfg->fp8_scale;
  P.fp8_dynamic = cfg->fp8_dynamic;
  c->partials = static_cast<double*>(ptrs[5]);
  c->dec_partials = static_cast<float*>(ptrs[6]);
  c->part_count = static_cast<uint32_t*>(ptrs[kBufCount]);
  P.dummy_page = static_cast<const uint8_t*>(ptrs[kBufDummy]);
  c->plan_bytes = plan_bytes_for(*cfg);
  c->n_ring = ring_slots(*cfg);
  for (int r = 0; r < c->n_ring; ++r) {
    c->plan_dev[r] = static_cast<uint8_t*>(ptrs[7 + r]);
    e = hipHostMalloc(reinterpret_cast<void**>(&c->plan_host[r]), static_cast<size_t>(c->plan_bytes), 0);
    if (e != hipSuccess) { free_all(c.get()); return fail(VK_ERR_OOM, "hipHostMalloc: %s", hipGetErrorString(e)); }
    e = hipEventCreateWithFlags(&c->plan_ev[r], hipEventDisableTiming);
    if (e != hipSuccess) { free_all(c.get()); return fail(VK_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e)); }
  }
  e = hipDeviceSynchronize();
  if (e != hipSuccess) { free_all(c.get()); return fail(VK_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e)); }
  c->host.reset(new vk::HostState(*cfg));
  c->stats.device_bytes = c->device_bytes;
  for (int f = 0; f < 4; ++f) c->stats.pool_pages[f] = caps[f];
  *out = c.release();
  g_error.clear();
  return VK_OK;
}

namespace {

// vk_append and vk_append_ragged: sequence i gets counts[i] tokens, its rows at tok_off_i of each
// layer's input block (the sequences one after another).
vk_status append_impl(vk_cache* c, int32_t layer_begin, int32_t n_layers, int32_t n_seqs, const int32_t* seq_ids,
                      const int32_t* counts, const void* k, const void* v, int32_t dtype, void* stream) {
  vk_status st = check_handle(c);
  if (st) return st;
  const vk_cache_config& cfg = c->cfg;
  if (n_layers < 1 || layer_begin < 0 || layer_begin + static_cast<int64_t>(n_layers) > cfg.n_layers)
    return fail(VK_ERR_ARG, "layer span [%d, %d) outside [0, %d)", layer_begin, layer_begin + n_layers, cfg.n_layers);
  if (dtype != VK_DTYPE_F16 && dtype != VK_DTYPE_BF16) return fail(VK_ERR_ARG, "dtype must be F16 or BF16");
  if (!k || !v) return fail(VK_ERR_ARG, "k or v is NULL");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(VK_ERR_ARG, "k and v must be 16-byte aligned");
  vk::AppendPlan plan;
  std::string err;
  st = c->host->plan_append(n_seqs, seq_ids, counts, &plan, &err);
  if (st) return fail(st, "%s", err.c_str());
  if (plan.new_pages[VK_FMT_LOSSLESS] > 0 && dtype != VK_DTYPE_BF16)
    return fail(VK_ERR_ARG, "lossless pages hold bfloat16 input");
  const int64_t row = static_cast<int64_t>(cfg.n_kv_heads) * cfg.head_dim;
  if (2 * static_cast<int64_t>(n_layers) * plan.total_blk > kMaxPartials)
    return fail(VK_ERR_ARG, "append too large for one call (%lld absmean blocks per layer); split it",
                static_cast<long long>(plan.total_blk));
  const int64_t total = static_cast<int64_t>(n_layers) * plan.total_tasks;
  // the 16-token units of lossless pages: (sequence index, unit) pairs for the pack kernel that
  // writes them
  std::vector<int32_t> ll_units, ot_units;  // (and the fp8 / fp16 units, likewise)
  int64_t n_units = 0;
  for (size_t i = 0; i < plan.seqs.size(); ++i) {
    const vk::AppendSeqDesc& d = plan.seqs[i];
    const int32_t unit_end = (d.t0 + d.n_tokens + vk::kUnit - 1) / vk::kUnit;
    for (int32_t u = d.unit_first; u < unit_end; ++u) {
      const int32_t page = u * vk::kUnit / cfg.block_size;
      const int f = vk::entry_fmt(plan.entries[d.page_off + page - d.page_first]);
      if (f == VK_FMT_LOSSLESS) {
        ll_units.push_back(static_cast<int32_t>(i));
        ll_units.push_back(u);
      } else if (f != VK_FMT_TERNARY2) {
        ot_units.push_back(static_cast<int32_t>(i));
        ot_units.push_back(u);
      }
      ++n_units;
    }
  }
  int64_t need = static_cast<int64_t>(plan.seqs.size()) * sizeof(vk::AppendSeqDesc) +
                 static_cast<int64_t>(plan.entries.size()) * 4 + static_cast<int64_t>(ll_units.size()) * 4;
  if (need > c->plan_bytes) return fail(VK_ERR_ARG, "append plan too large");
  // A call that is mostly ternary writes its fp8 / fp16 units in a launch of their own, so that
  // the main launch runs the pack kernel's lean ternary instance (fewer registers, more waves);
  // calls made of such units (decode-time appends into the recent tier) keep one launch.
  if (ot_units.empty() || 8 * static_cast<int64_t>(ot_units.size() / 2) > n_units ||
      need + static_cast<int64_t>(ot_units.size()) * 4 > c->plan_bytes)
    ot_units.clear();
  need += static_cast<int64_t>(ot_units.size()) * 4;
  st = set_device(c);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int slot = c->ring_next;
  c->ring_next = (c->ring_next + 1) % c->n_ring;
  hipError_t e = hipSuccess;
  if (c->plan_ev_used[slot]) {  // every slot in flight: wait for the oldest plan's kernels
    e = hipEventSynchronize(c->plan_ev[slot]);
    if (e != hipSuccess) return hip_fail(c, e, "hipEventSynchronize");
  }
  // from here on the host state changes: any failure poisons the handle
  c->host->commit_append(&plan);
  uint8_t* hp = c->plan_host[slot];
  const size_t desc_bytes = plan.seqs.size() * sizeof(vk::AppendSeqDesc);
  std::memcpy(hp, plan.seqs.data(), desc_bytes);
  std::memcpy(hp + desc_bytes, plan.entries.data(), plan.entries.size() * 4);
  const size_t ll_off = desc_bytes + plan.entries.size() * 4;
  if (!ll_units.empty()) std::memcpy(hp + ll_off, ll_units.data(), ll_units.size() * 4);
  const size_t ot_off = ll_off + ll_units.size() * 4;
  if (!ot_units.empty()) std::memcpy(hp + ot_off, ot_units.data(), ot_units.size() * 4);
  e = hipMemcpyAsync(c->plan_dev[slot], hp, static_cast<size_t>(need), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(c, e, "hipMemcpyAsync");
  vk::AppendArgs a{};
  a.P = c->pools;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.descs = reinterpret_cast<const vk::AppendSeqDesc*>(c->plan_dev[slot]);
  a.entries = reinterpret_cast<const int32_t*>(c->plan_dev[slot] + desc_bytes);
  a.partials = c->partials;
  a.dtype = dtype;
  a.layer_begin = layer_begin;
  a.n_layers = n_layers;
  a.n_seqs = n_seqs;
  a.total_tokens = static_cast<int32_t>(plan.total_tokens);
  a.total_blk = static_cast<int32_t>(plan.total_blk);
  a.total_tasks = static_cast<int32_t>(plan.total_tasks);
  // Every touched page ternary, head dim 64 or 128, and a call of at most kPackPipeMaxTasks
  // tasks per block at pack_blocks_per_cu() blocks per compute unit (4096 tokens x 4 sequences
  // x 8 heads, or 36 layers x 4096 tokens x 2 heads): the pipelined pack kernel, with about as
  // many blocks as the GPU holds at once.  Larger calls stream better through the one-task
  // blocks of k_pack (more waves resident: 67 registers against 120).
  const bool only_ternary = std::all_of(plan.entries.begin(), plan.entries.end(),
                                        [](int32_t e) { return vk::entry_fmt(e) == VK_FMT_TERNARY2; });
  const int64_t pipe_blocks = static_cast<int64_t>(std::max(1, c->n_cu)) * pack_blocks_per_cu();
  a.pack_pipelined =
      only_ternary && cfg.head_dim != 256 && total <= pipe_blocks * kPackPipeMaxTasks && pack_pipelined_on() ? 1 : 0;
  const int64_t target = a.pack_pipelined ? pipe_blocks : kPackTargetBlocks;
  const int64_t blocks = std::min<int64_t>(total, target);
  a.tasks_per_blk = static_cast<int32_t>((total + blocks - 1) / blocks);
  a.pack_blocks = static_cast<int32_t>((total + a.tasks_per_blk - 1) / a.tasks_per_blk);
  // sequences with equal task (block) counts: the kernels find a task's sequence by division
  a.seq_tasks = a.seq_blk = 0;
  {
    const int64_t nt0 = (plan.seqs.size() > 1 ? plan.seqs[1].task_off : plan.total_tasks);
    const int64_t nb0 = (plan.seqs.size() > 1 ? plan.seqs[1].blk_off : plan.total_blk);
    bool eq_t = true, eq_b = true;
    for (size_t j = 0; j < plan.seqs.size(); ++j) {
      eq_t &= plan.seqs[j].task_off == static_cast<int64_t>(j) * nt0;
      eq_b &= plan.seqs[j].blk_off == static_cast<int64_t>(j) * nb0;
    }
    eq_t &= plan.total_tasks == static_cast<int64_t>(plan.seqs.size()) * nt0;
    eq_b &= plan.total_blk == static_cast<int64_t>(plan.seqs.size()) * nb0;
    if (eq_t && nt0 > 0) a.seq_tasks = static_cast<int32_t>(nt0);
    if (eq_b && nb0 > 0) a.seq_blk = static_cast<int32_t>(nb0);
  }
  a.eps = cfg.eps;
  a.ll_units = reinterpret_cast<const int32_t*>(c->plan_dev[slot] + ll_off);
  a.n_ll_units = static_cast<int32_t>(ll_units.size() / 2);
  a.ot_units = reinterpret_cast<const int32_t*>(c->plan_dev[slot] + ot_off);
  a.n_ot_units = static_cast<int32_t>(ot_units.size() / 2);
  a.all_ternary = std::all_of(plan.entries.begin(), plan.entries.end(), [](int32_t e) {
    return vk::entry_fmt(e) == VK_FMT_TERNARY2 || vk::entry_fmt(e) == VK_FMT_LOSSLESS;
  });
  if (c->timer.on) {
    // algorithmic bytes: pass 1 reads the ternary-routed input once; pass 2 reads
    // all input once and writes every stored byte once (+ one gamma per ternary page)
    double tern_tokens = 0.0;
    for (const vk::AppendSeqDesc& d : plan.seqs) tern_tokens += d.tern_hi - d.tern_lo;
    const double layers = n_layers;
    c->timer.add_bytes(VK_KERNEL_ABSMEAN, layers * 2.0 * tern_tokens * row * 2.0);
    c->timer.add_bytes(VK_KERNEL_FINALIZE, layers * 2.0 * static_cast<double>(plan.total_blk) * 8.0);
    const double in_bytes = layers * 2.0 * static_cast<double>(plan.total_tokens) * row * 2.0;
    // + token scales; lossless: the coded streams (1.5 bytes per element) and a 16-byte header per
    // 16 tokens (its exceptions, about 0.02% of the values on normal data, are not counted)
    const double per_elem[4] = {0.25, 1.0 + (cfg.fp8_dynamic ? 4.0 / cfg.head_dim : 0.0), 2.0,
                                1.5 + 1.0 / cfg.head_dim};
    double out_bytes = 0.0;
    for (const vk::AppendSeqDesc& d : plan.seqs) {
      for (int32_t j = 0; j < d.n_pages; ++j) {
        const int32_t p = d.page_first + j;
        const int f = vk::entry_fmt(plan.entries[d.page_off + j]);
        const int64_t lo = std::max<int64_t>(static_cast<int64_t>(p) * cfg.block_size, d.t0);
        const int64_t hi = std::min<int64_t>(static_cast<int64_t>(p + 1) * cfg.block_size, d.t0 + d.n_tokens);
        out_bytes += 2.0 * (hi - lo) * row * per_elem[f] + (f == VK_FMT_TERNARY2 && lo % cfg.block_size == 0 ? 8.0 : 0.0);
      }
    }
    c->timer.add_bytes(VK_KERNEL_PACK, in_bytes + layers * out_bytes);
  }
  e = vk::launch_append(a, s, c->timer.on ? &c->timer : nullptr);
  if (e != hipSuccess) return hip_fail(c, e, "append kernels");
  e = hipEventRecord(c->plan_ev[slot], s);
  if (e != hipSuccess) return hip_fail(c, e, "hipEventRecord");
  c->plan_ev_used[slot] = true;
  c->stats.append_calls += 1;
  g_error.clear();
  return VK_OK;
}

}  // namespace

VK_API vk_status vk_append(vk_cache* c, int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                           const int32_t* seq_ids, int32_t n_tokens, const void* k, const void* v,
                           int32_t dtype, void* stream) {
  if (n_tokens < 1) return fail(VK_ERR_ARG, "n_tokens must be >= 1");
  if (n_seqs < 1 || (c && n_seqs > c->cfg.max_seqs)) return fail(VK_ERR_ARG, "n_seqs %d out of range", n_seqs);
  std::vector<int32_t> counts(static_cast<size_t>(n_seqs), n_tokens);
  return append_impl(c, layer_begin, n_layers, n_seqs, seq_ids, counts.data(), k, v, dtype, stream);
}

VK_API vk_status vk_append_ragged(vk_cache* c, int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                  const int32_t* seq_ids, const int32_t* n_tokens, const void* k, const void* v,
                                  int32_t dtype, void* stream) {
  return append_impl(c, layer_begin, n_layers, n_seqs, seq_ids, n_tokens, k, v, dtype, stream);
}

VK_API vk_status vk_retier(vk_cache* c, int32_t n_seqs, const int32_t* seq_ids, int64_t* n_pages, void* stream) {
  vk_status st = check_handle(c);
  if (st) return st;
  vk::RetierPlan plan;
  std::string err;
  st = c->host->plan_retier(n_seqs, seq_ids, &plan, &err);
  if (st) return fail(st, "%s", err.c_str());
  const int64_t n_tasks = static_cast<int64_t>(plan.tasks.size());
  if (n_tasks > 0) {
    st = set_device(c);
    if (st) return st;
  }
  // from here on the host state changes: any failure poisons the handle
  c->host->commit_retier(n_seqs, seq_ids, &plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t per_launch = c->plan_bytes / static_cast<int64_t>(sizeof(vk::RetierTask));
  for (int64_t first = 0; first < n_tasks; first += per_launch) {
    const int64_t cnt = std::min(per_launch, n_tasks - first);
    const int slot = c->ring_next;
    c->ring_next = (c->ring_next + 1) % c->n_ring;
    hipError_t e = hipSuccess;
    if (c->plan_ev_used[slot]) {
      e = hipEventSynchronize(c->plan_ev[slot]);
      if (e != hipSuccess) return hip_fail(c, e, "hipEventSynchronize");
    }
    const size_t bytes = static_cast<size_t>(cnt) * sizeof(vk::RetierTask);
    std::memcpy(c->plan_host[slot], plan.tasks.data() + first, bytes);
    e = hipMemcpyAsync(c->plan_dev[slot], c->plan_host[slot], bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(c, e, "hipMemcpyAsync");
    vk::RetierArgs a{};
    a.P = c->pools;
    a.tasks = reinterpret_cast<const vk::RetierTask*>(c->plan_dev[slot]);
    a.n_tasks = static_cast<int32_t>(cnt);
    a.eps = c->cfg.eps;
    if (c->timer.on) {
      // reads every FP8 page once, writes the ternary page and its two gammas
      const double per_page = static_cast<double>(vk::page_bytes(c->cfg, VK_FMT_FP8E4M3)) +
                              static_cast<double>(vk::page_bytes(c->cfg, VK_FMT_TERNARY2)) + 8.0;
      c->timer.add_bytes(VK_KERNEL_RETIER, static_cast<double>(cnt) * c->cfg.n_layers * per_page);
    }
    e = vk::launch_retier(a, s, c->timer.on ? &c->timer : nullptr);
    if (e != hipSuccess) return hip_fail(c, e, "retier kernel");
    e = hipEventRecord(c->plan_ev[slot], s);
    if (e != hipSuccess) return hip_fail(c, e, "hipEventRecord");
    c->plan_ev_used[slot] = true;
  }
  c->stats.retier_calls += 1;
  c->stats.pages_retiered += n_tasks;
  if (n_pages) *n_pages = n_tasks;
  g_error.clear();
  return VK_OK;
}

VK_API vk_status vk_evict(vk_cache* c, int32_t n_seqs, const int32_t* seq_ids, int32_t window, int64_t* n_pages,
                          void* stream) {
  (void)stream;  // host state only: the freed pages are reused by later appends in stream order
  vk_status st = check_handle(c);
  if (st) return st;
  std::string err;
  int64_t freed = 0;
  st = c->host->evict(n_seqs, seq_ids, window, &freed, &err);
  if (st) return fail(st, "%s", err.c_str());
  c->stats.pages_evicted += freed;
  if (n_pages) *n_pages = freed;
  g_error.clear();
  return VK_OK;
}

VK_API vk_status vk_decode_attn(vk_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const void* q,
                                int32_t q_dtype, int32_t window, float softmax_scale, float* out, void* stream) {
  vk_status st = check_handle(c);
  if (st) return st;
  const vk_cache_config& cfg = c->cfg;
  if (layer < 0 || layer >= cfg.n_layers) return fail(VK_ERR_ARG, "layer %d out of range", layer);
  if (q_dtype != VK_DTYPE_F16 && q_dtype != VK_DTYPE_BF16) return fail(VK_ERR_ARG, "q_dtype must be F16 or BF16");
  if (n_seqs == 0) {  // nothing to attend: no launch (q and out may be NULL)
    g_error.clear();
    return VK_OK;
  }
  if (!q || !out) return fail(VK_ERR_ARG, "q or out is NULL");
  if ((reinterpret_cast<uintptr_t>(q) & 3) || (reinterpret_cast<uintptr_t>(out) & 15))
    return fail(VK_ERR_ARG, "q must be 4-byte and out 16-byte aligned");
  if (!std::isfinite(softmax_scale)) return fail(VK_ERR_ARG, "softmax_scale must be finite");
  if (cfg.sink_tokens == 0 && window == 0) return fail(VK_ERR_ARG, "no sinks and window 0 attend nothing");
  std::string err;
  st = c->host->check_decode(n_seqs, seq_ids, window, &err);
  if (st) return fail(st, "%s", err.c_str());
  st = set_device(c);
  if (st) return st;
  const int g = cfg.n_q_heads / cfg.n_kv_heads;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(cfg.head_dim));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t units[4] = {0, 0, 0, 0};
  int32_t splits_used = 1, steal_used = 0, ordered_used = 0;
  const bool mfma = cfg.decode_kernel != VK_DECODE_VALU;
  const bool d256 = cfg.head_dim == 256;  // matrix-core instances: 4-slot ring, no stealing blocks
  // sequences per launch: every (sequence, KV head) needs room for a split's partial and the
  // fp8 / fp16 blocks' partials
  const int32_t per_launch = static_cast<int32_t>(std::max<int64_t>(
      1, std::min<int64_t>(vk::kDecodeMaxSeqs, kDecodeScratchItems / ((2 + kDecodeMixedPartsMax) * cfg.n_kv_heads))));
  for (int32_t base = 0; base < n_seqs; base += per_launch) {
    const int32_t nb = std::min<int32_t>(per_launch, n_seqs - base);
    vk::DecodeArgs a{};
    a.P = c->pools;
    a.q = static_cast<const uint16_t*>(q) + static_cast<int64_t>(base) * cfg.n_q_heads * cfg.head_dim;
    a.out = out + static_cast<int64_t>(base) * cfg.n_q_heads * cfg.head_dim;
    a.partials = c->dec_partials;
    a.q_dtype = q_dtype;
    a.layer = layer;
    a.n_seqs = nb;
    a.hq = cfg.n_q_heads;
    a.sink_tokens = cfg.sink_tokens;
    a.window = window;
    a.kernel = mfma ? VK_DECODE_MFMA : VK_DECODE_VALU;
    a.units_per_iter = d256 ? 4 : decode_units_per_iter();
    a.scale_log2 = scale * 1.4426950408889634f;
    int32_t max_units = 0, min_units = 0;
    int64_t cu[4] = {0, 0, 0, 0};  // attended units per format in this launch
    int64_t other_kb[vk::kDecodeMaxSeqs];  // fp8 / fp16 units' bytes per head, in ternary units'
    // longest attended ranges first: their blocks are dispatched first, shorter ones fill in
    int32_t order[vk::kDecodeMaxSeqs], units_of[vk::kDecodeMaxSeqs];
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t sid = seq_ids[base + i];
      units_of[i] = vk::attended_units(c->host->seq(sid).length, cfg.sink_tokens, window).n_units();
      order[i] = i;
    }
    std::stable_sort(order, order + nb, [&](int32_t x, int32_t y) { return units_of[x] > units_of[y]; });
    min_units = nb > 0 ? units_of[order[nb - 1]] : 0;
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t sid = seq_ids[base + order[i]];
      a.slots[i] = sid;
      a.lens[i] = c->host->seq(sid).length;
      a.rows[i] = order[i];
      max_units = std::max(max_units, units_of[order[i]]);
      int64_t cs[4] = {0, 0, 0, 0};
      c->host->count_units(sid, window, cs);
      for (int f = 0; f < 4; ++f) cu[f] += cs[f];
      other_kb[i] = cs[1] * 4 + cs[2] * 8;
      c->host->mixed_ranges(sid, window, a.mix[i]);
    }
    for (int f = 0; f < 4; ++f) units[f] += cu[f];
    // matrix-core path: fp8 / fp16 / lossless pages go to one more block per (sequence, KV head),
    // which writes one more partial state
    const bool mixed = mfma && (cu[1] + cu[2] + cu[3]) > 0;
    // fp8 / fp16 pages: n_mix more blocks per (sequence, KV head); lossless pages: one more launch
    // of a block per (sequence, KV head); each writes a partial state of its own
    const int n_ll = mfma && cu[3] > 0 ? 1 : 0;
    const int n_fp = mfma && (cu[1] + cu[2]) > 0 ? decode_mixed_parts() : 0;
    const int n_mix = n_fp + n_ll;
    a.lossless = n_ll;
    a.n_mix_parts = n_fp;
    a.part_base = 0;
    const int64_t items = static_cast<int64_t>(nb) * cfg.n_kv_heads;
    const int32_t max_splits = static_cast<int32_t>(
        std::min<int64_t>(kDecodeMaxSplits - n_mix, kDecodeScratchItems / items - n_mix));
    // Splits hold a fixed number of units, so long sequences get more of them than short
    // ones (a block past a sequence's units writes an empty part).
    const int64_t all_units = (cu[0] + cu[1] + cu[2]) * cfg.n_kv_heads;
    const bool ragged = mfma && (max_units != min_units || n_fp > 0);
    const int32_t target_blocks =
        static_cast<int32_t>(std::max(1, c->n_cu) * (ragged ? decode_blocks_per_cu_ragged() : decode_blocks_per_cu()));
    vk::SplitPlan sp = mfma ? vk::plan_splits(all_units, max_units, target_blocks,
                                              std::max(1, max_splits), 4 * kDecodeMinUnitsPerWave,
                                              4 * kDecodeUnitsPerStep)
                            : vk::plan_splits(all_units, max_units, kDecodeTargetGroups,
                                              std::max(1, max_splits), kDecodeMinUnits);
    // every pair attends the same units: a split count whose blocks spread evenly over the
    // compute units (e.g. 24 sequences x 8 KV heads: 4 splits, 3 blocks on every CU, rather
    // than 3 splits, 3 blocks on some CUs and 2 on others)
    if (mfma && !ragged && !d256 && n_mix == 0 && c->n_cu > 0 && decode_balance_on())
      sp = vk::balance_splits(sp, items, max_units, c->n_cu, kDecodeMaxResidentBlocks, std::max(1, max_splits),
                              4 * kDecodeMinUnitsPerWave, 4 * kDecodeUnitsPerStep);
    a.n_splits = sp.n_splits;
    a.units_per_split = sp.units_per_split;
    // Opted in: all-ternary launches with at most one (sequence, KV head) per compute unit and
    // enough work take one 12-wave block per compute unit whose waves share the block's units
    // piece by piece: the blocks' waves end together, and a block per pair writes its output.
    const int steal_mode = decode_steal_mode();
    if (mfma && !d256 && !mixed && !cfg.fp8_dynamic && a.units_per_iter == 8 && c->n_cu > 0 && items <= c->n_cu &&
        max_units > 0 && (steal_mode == 2 || (steal_mode == 1 && all_units >= kStealMinUnitsPerCu * c->n_cu))) {
      const int32_t ns = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(c->n_cu / items, max_splits)));
      const int32_t ups = (max_units + ns - 1) / ns;
      a.units_per_split = (ups + kStealPiece - 1) / kStealPiece * kStealPiece;
      a.n_splits = (max_units + a.units_per_split - 1) / a.units_per_split;
      a.steal = 1;
    }
    a.n_parts = a.n_splits + n_mix;
    a.part_count = c->part_count;
    a.fused_merge = mfma && a.n_parts > 1 && !n_ll && !a.steal && decode_fused_merge_on() ? 1 : 0;
    a.n_order = 0;
    if (ragged && !a.steal && decode_order_on()) {
      int32_t u_launch[vk::kDecodeMaxSeqs];
      int64_t w_mix[vk::kDecodeMaxSeqs];
      const int64_t fixed = decode_mix_fixed();
      for (int32_t i = 0; i < nb; ++i) {
        u_launch[i] = units_of[order[i]];
        w_mix[i] = other_kb[i] > 0 ? fixed + (other_kb[i] + n_fp - 1) / std::max(1, n_fp) : 0;
      }
      std::vector<uint16_t> ord;
      if (vk::plan_decode_order(u_launch, w_mix, nb, a.n_splits, a.units_per_split, n_fp, vk::kDecodeMaxOrder, &ord)) {
        a.n_order = static_cast<int32_t>(ord.size());
        std::copy(ord.begin(), ord.end(), a.order);
      }
    }
    if (items * a.n_parts > kDecodeScratchItems)  // (only with thousands of KV heads)
      return fail(VK_ERR_CAPACITY, "decode partial states: %lld needed, %lld held", static_cast<long long>(items * a.n_parts),
                  static_cast<long long>(kDecodeScratchItems));
    splits_used = a.n_splits;
    steal_used |= a.steal;
    ordered_used |= a.n_order > 0 ? 1 : 0;
    if (c->timer.on) {
      const double row = cfg.head_dim;
      const double unit_kv = 2.0 * 16.0 * cfg.n_kv_heads;  // K and V, 16 tokens, every KV head
      const double tern_bytes = unit_kv * cu[0] * row / 4.0;
      // lossless units: header and the two coded streams (exceptions not counted)
      const double other_bytes = unit_kv * (cu[1] * (row + (cfg.fp8_dynamic ? 4.0 : 0.0)) + cu[2] * row * 2.0 +
                                            cu[3] * (row * 1.5 + 1.0));
      const double q_bytes = static_cast<double>(nb) * cfg.n_q_heads * cfg.head_dim * 2.0;
      const double out_bytes = static_cast<double>(nb) * cfg.n_q_heads * cfg.head_dim * 4.0;
      const double part1 = static_cast<double>(nb) * cfg.n_q_heads * (cfg.head_dim + 2) * 4.0;  // one part
      const double dec_out = a.n_parts > 1 ? part1 * a.n_splits : out_bytes;
      c->timer.add_bytes(VK_KERNEL_DECODE, tern_bytes + other_bytes + q_bytes + dec_out + n_mix * part1);
      // the parts' combination: read every part, write the output (inside the decode kernel
      // when it merges them itself)
      if (a.n_parts > 1)
        c->timer.add_bytes(a.fused_merge ? VK_KERNEL_DECODE : VK_KERNEL_MERGE, part1 * a.n_parts + out_bytes);
    }
    hipError_t e = vk::launch_decode(a, g, s, c->timer.on ? &c->timer : nullptr);
    if (e != hipSuccess) return hip_fail(c, e, "decode kernels");
  }
  c->stats.decode_calls += 1;
  c->stats.last_decode_splits = splits_used;
  c->stats.last_decode_steal = steal_used;
  c->stats.last_decode_ordered = ordered_used;
  for (int f = 0; f < 4; ++f) {
    c->stats.last_decode_units[f] = units[f];
    c->stats.total_decode_units[f] += units[f];
  }
  g_error.clear();
  return VK_OK;
}

VK_API vk_status vk_reset_seqs(vk_cache* c, int32_t n_seqs, const int32_t* seq_ids, void* stream) {
  vk_status st = check_handle(c);
  if (st) return st;
  std::string err;
  // validate before waiting
  if (n_seqs < 0 || (n_seqs > 0 && !seq_ids)) return fail(VK_ERR_ARG, "bad sequence list");
  for (int32_t i = 0; i < n_seqs; ++i)
    if (seq_ids[i] < 0 || seq_ids[i] >= c->cfg.max_seqs) return fail(VK_ERR_ARG, "seq id %d out of range", seq_ids[i]);
  (void)stream;  // frees are ordered by later appends on the same stream
  st = c->host->reset_seqs(n_seqs, seq_ids, &err);
  if (st) return fail(st, "%s", err.c_str());
  g_error.clear();
  return VK_OK;
}

VK_API vk_status vk_seq_length(vk_cache* c, int32_t seq, int32_t* length) {
  if (!c || !length) return fail(VK_ERR_ARG, "NULL argument");
  if (seq < 0 || seq >= c->cfg.max_seqs) return fail(VK_ERR_ARG, "seq id %d out of range", seq);
  *length = c->host->seq(seq).length;
  return VK_OK;
}

VK_API vk_status vk_read_pages(vk_cache* c, int32_t layer, int32_t seq, int32_t page0, int32_t n_pages,
                               uint8_t* host_bytes, int32_t* host_fmt, float* host_gamma) {
  vk_status st = check_handle(c);
  if (st) return st;
  const vk_cache_config& cfg = c->cfg;
  if (layer < 0 || layer >= cfg.n_layers) return fail(VK_ERR_ARG, "layer out of range");
  if (seq < 0 || seq >= cfg.max_seqs) return fail(VK_ERR_ARG, "seq out of range");
  const vk::SeqState& ss = c->host->seq(seq);
  if (page0 < 0 || n_pages < 0 || page0 + static_cast<int64_t>(n_pages) > static_cast<int64_t>(ss.pages.size()))
    return fail(VK_ERR_ARG, "pages [%d, %d) not allocated", page0, page0 + n_pages);
  if (n_pages > 0 && (!host_bytes || !host_fmt || !host_gamma)) return fail(VK_ERR_ARG, "NULL output");
  st = set_device(c);
  if (st) return st;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(c, e, "hipDeviceSynchronize");
  int64_t stride = 0;  // the largest page of any format
  for (int f = 0; f < 4; ++f) stride = std::max(stride, vk::page_bytes(cfg, f));
  for (int32_t j = 0; j < n_pages; ++j) {
    const int32_t ent = ss.pages[page0 + j];
    if (ent == vk::kNoPage) {  // freed by eviction
      std::memset(host_bytes + j * stride, 0, static_cast<size_t>(stride));
      host_fmt[j] = -1;
      host_gamma[2 * j] = host_gamma[2 * j + 1] = std::nanf("");
      continue;
    }
    const int f = vk::entry_fmt(ent);
    const int64_t idx = vk::entry_idx(ent);
    const uint8_t* src = c->pools.pool[f] + (static_cast<int64_t>(layer) * c->pools.cap[f] + idx) * c->pools.page_bytes[f];
    e = hipMemcpy(host_bytes + j * stride, src, static_cast<size_t>(c->pools.page_bytes[f]), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(c, e, "hipMemcpy");
    host_fmt[j] = f;
    if (f == VK_FMT_TERNARY2) {
      e = hipMemcpy(host_gamma + 2 * j, c->pools.gamma + (static_cast<int64_t>(layer) * c->pools.cap[0] + idx) * 2, 8,
                    hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(c, e, "hipMemcpy");
    } else {
      host_gamma[2 * j] = host_gamma[2 * j + 1] = std::nanf("");
    }
  }
  g_error.clear();
  return VK_OK;
}

VK_API vk_status vk_get_stats(vk_cache* c, vk_stats* out) {
  if (!c || !out) return fail(VK_ERR_ARG, "NULL argument");
  vk_stats s = c->stats;
  for (int f = 0; f < 4; ++f) {
    s.pages_used[f] = c->host->pages_used(f);
    s.tokens_stored[f] = c->host->tokens_stored(f);
  }
  *out = s;
  return VK_OK;
}

VK_API vk_status vk_set_kernel_timing(vk_cache* c, int32_t enable) {
  vk_status st = check_handle(c);
  if (st) return st;
  st = set_device(c);
  if (st) return st;
  if (enable) {
    c->timer.on = true;
    c->timer.reset();
  } else {
    c->timer.flush();
    c->timer.on = false;
  }
  return VK_OK;
}

VK_API vk_status vk_get_kernel_times(vk_cache* c, int64_t* launches, double* milliseconds, double* bytes) {
  vk_status st = check_handle(c);
  if (st) return st;
  st = set_device(c);
  if (st) return st;
  c->timer.flush();
  for (int k = 0; k < VK_KERNEL_COUNT; ++k) {
    if (launches) launches[k] = c->timer.launches[k];
    if (milliseconds) milliseconds[k] = c->timer.ms[k];
    if (bytes) bytes[k] = c->timer.bytes[k];
  }
  return VK_OK;
}

VK_API vk_status vk_release(vk_cache* c) {
  if (!c) return VK_OK;
  vk_status st = VK_OK;
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess && cur != c->device) (void)hipSetDevice(c->device);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) st = fail(VK_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
  free_all(c);
  if (cur >= 0 && cur != c->device) (void)hipSetDevice(cur);
  delete c;
  return st;
}

VK_API int64_t vk_quantize_pack_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  const int64_t n_blk = (n + vk::kAbsElemsPerBlock - 1) / vk::kAbsElemsPerBlock;
  return 256 + ((n_blk * 8 + 255) & ~int64_t(255));
}

namespace {

// Checks shared by the flat entry points; "" when the arguments are usable.
vk_status check_quantize_args(const void* x, int64_t n, int32_t dtype, float eps, const uint8_t* packed,
                              const float* gamma_out) {
  if (!x || !packed || !gamma_out) return fail(VK_ERR_ARG, "NULL argument");
  if (n < 8 || n % 8) return fail(VK_ERR_ARG, "n must be a positive multiple of 8");
  if (dtype != VK_DTYPE_F16 && dtype != VK_DTYPE_BF16) return fail(VK_ERR_ARG, "dtype must be F16 or BF16");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(VK_ERR_ARG, "eps must be finite and >= 0");
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(packed) & 1))
    return fail(VK_ERR_ARG, "x must be 16-byte aligned, packed 2-byte aligned");
  return VK_OK;
}

vk::QuantArgs quantize_args(const void* x, int64_t n, int32_t dtype, float eps, const float* gamma_in,
                            uint8_t* packed, float* gamma_out, uint8_t* scratch) {
  vk::QuantArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.packed = packed;
  a.gamma_in = gamma_in;
  a.gamma_out = gamma_out;
  a.seg = reinterpret_cast<vk::SegInfo*>(scratch);
  a.partials = reinterpret_cast<double*>(scratch + 256);
  a.n = n;
  a.dtype = dtype;
  a.n_blk = static_cast<int32_t>((n + vk::kAbsElemsPerBlock - 1) / vk::kAbsElemsPerBlock);
  a.eps = eps;
  return a;
}

}  // namespace

VK_API vk_status vk_quantize_pack(const void* x, int64_t n, int32_t dtype, float eps, const float* gamma_in,
                                  uint8_t* packed, float* gamma_out, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  vk_status st = check_quantize_args(x, n, dtype, eps, packed, gamma_out);
  if (st) return st;
  if (!workspace) return fail(VK_ERR_ARG, "NULL argument");
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return fail(VK_ERR_ARG, "workspace must be 16-byte aligned");
  if (workspace_bytes < vk_quantize_pack_workspace_bytes(n)) return fail(VK_ERR_ARG, "workspace too small");
  const int64_t n_blk = (n + vk::kAbsElemsPerBlock - 1) / vk::kAbsElemsPerBlock;
  if (n_blk > 0x7FFFFFFF) return fail(VK_ERR_ARG, "tensor too large");
  const vk::QuantArgs a = quantize_args(x, n, dtype, eps, gamma_in, packed, gamma_out, static_cast<uint8_t*>(workspace));
  hipError_t e = vk::launch_quantize(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VK_ERR_HIP, "quantize kernels: %s", hipGetErrorString(e));
  g_error.clear();
  return VK_OK;
}

VK_API int64_t vk_quantize_pack_noalloc_max_elems(void) { return vk::kQuantNoAllocMaxElems; }

VK_API vk_status vk_quantize_pack_noalloc(const void* x, int64_t n, int32_t dtype, float eps, const float* gamma_in,
                                          uint8_t* packed, float* gamma_out, void* stream) {
  vk_status st = check_quantize_args(x, n, dtype, eps, packed, gamma_out);
  if (st) return st;
  if (n > vk::kQuantNoAllocMaxElems)
    return fail(VK_ERR_CAPACITY, "n = %lld exceeds the %lld elements the allocation-free scratch holds; "
                "use vk_quantize_pack with a workspace", static_cast<long long>(n),
                static_cast<long long>(vk::kQuantNoAllocMaxElems));
  void* scratch = nullptr;
  hipError_t e = vk::quantize_noalloc_scratch(&scratch);
  if (e != hipSuccess) return fail(VK_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
  const vk::QuantArgs a = quantize_args(x, n, dtype, eps, gamma_in, packed, gamma_out, static_cast<uint8_t*>(scratch));
  e = vk::launch_quantize(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VK_ERR_HIP, "quantize kernels: %s", hipGetErrorString(e));
  g_error.clear();
  return VK_OK;
}

VK_API const char* vk_last_error(void) { return g_error.c_str(); }

VK_API const char* vk_status_string(vk_status s) {
  switch (s) {
    case VK_OK: return "VK_OK";
    case VK_ERR_ARG: return "VK_ERR_ARG";
    case VK_ERR_OOM: return "VK_ERR_OOM";
    case VK_ERR_CAPACITY: return "VK_ERR_CAPACITY";
    case VK_ERR_ALIGN: return "VK_ERR_ALIGN";
    case VK_ERR_STATE: return "VK_ERR_STATE";
    case VK_ERR_HIP: return "VK_ERR_HIP";
  }
  return "unknown";
}

}  // extern "C"
