// Kernel argument blocks and launchers shared by the host API and the HIP
// kernels.  Everything here is plain data passed by value.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace vk {

struct AppendSeqDesc;  // host_state.h
struct RetierTask;     // host_state.h

// Device view of the paged pools.  Page `idx` of format f in layer `layer`:
//   pool[f] + (layer * cap[f] + idx) * page_bytes[f]
// with the page laid out [K tile head 0..Hkv-1][V tile head 0..Hkv-1].
struct PoolsView {
  uint8_t* pool[4];        // by format (VK_FMT_*)
  float* gamma;            // [n_layers][cap[0]][2]: K and V gamma of ternary pages
  int32_t* block_table;    // [max_seqs][max_pages]: (format << 30) | pool index
  int64_t cap[4];          // pages per layer
  int64_t tile_bytes[4];   // one (K|V, head) tile
  int64_t page_bytes[4];
  int32_t max_pages;
  int32_t n_layers;
  int32_t hkv;
  int32_t dim;
  int32_t bs;              // tokens per page (power of two)
  int32_t bs_shift;        // log2(bs)
  float fp8_scale;
  int32_t fp8_dynamic;     // FP8 tiles end with block_size float32 scales (one per token)
  const uint8_t* dummy_page;  // a zeroed ternary-page-sized buffer: target of speculative loads
};

struct SegInfo {           // per (layer, seq, K|V) of one append call
  float gamma;             // mean |x| of the ternary-routed tokens, float32
  uint32_t thresh;         // smallest 16-bit magnitude whose code is nonzero
};

constexpr int kAbsThreads = 256;
constexpr int kAbsElemsPerThreadIter = 8;       // one 16-byte load
constexpr int kAbsIters = 8;
constexpr int kAbsElemsPerBlock = kAbsThreads * kAbsElemsPerThreadIter * kAbsIters;

struct AppendArgs {
  PoolsView P;
  const uint16_t* k;       // [n_layers][total_tokens][hkv][dim]: sequence i at rows descs[i].tok_off ..
  const uint16_t* v;
  const AppendSeqDesc* descs;
  const int32_t* entries;
  double* partials;        // [n_layers][K|V][total_blk]
  int32_t dtype;           // 0 f16, 1 bf16
  int32_t layer_begin;
  int32_t n_layers;
  int32_t n_seqs;
  int32_t total_tokens;    // input rows per layer (sum of the sequences' token counts)
  int32_t total_blk;       // absmean blocks per (layer, K|V) (sum over the sequences)
  int32_t total_tasks;     // pack tasks per layer (sum over the sequences)
  int32_t tasks_per_blk;   // pack tasks per block
  int32_t pack_blocks;     // pack grid: ceil(n_layers * total_tasks / tasks_per_blk)
  int32_t seq_tasks;       // pack tasks of every sequence when they all have the same count, else 0
  int32_t seq_blk;         // absmean blocks of every sequence when they all have the same count, else 0
  int32_t all_ternary;     // every touched page is ternary or lossless (the pack kernel's lean instance)
  int32_t pack_pipelined;  // every touched page is ternary, head dim 64 or 128: k_pack_tern, whose
                           // blocks keep the next task's loads in flight (tasks_per_blk sized for it)
  const int32_t* ll_units; // [n_ll_units][2]: (sequence index, unit) of every lossless 16-token unit
  int32_t n_ll_units;      // written by a pack launch of their own (the main one skips them)
  const int32_t* ot_units; // [n_ot_units][2]: (sequence index, unit) of every fp8 / fp16 16-token
  int32_t n_ot_units;      // unit, when they get a pack launch of their own (0: the main launch
                           // writes them)
  float eps;
};

constexpr int kDecodeMaxSeqs = 64;    // sequences per decode launch (kernel-argument table)
constexpr int kDecodeMaxOrder = 768;  // entries of a decode launch's dispatch order (kernel arguments)
constexpr int kDecodeUnitsPerIter = 4;

struct DecodeArgs {
  PoolsView P;
  const uint16_t* q;       // [n_seqs][hq][dim]
  float* out;              // [n_seqs][hq][dim]
  float* partials;         // [n_seqs][hq][n_parts][dim + 2]: (o, max, sum) per part
  int32_t q_dtype;
  int32_t layer;
  int32_t n_seqs;          // in this launch (<= kDecodeMaxSeqs)
  int32_t hq;
  int32_t sink_tokens;
  int32_t window;
  int32_t n_splits;        // splits of the attended units (parts 0 .. n_splits-1)
  int32_t units_per_split; // split x takes logical units [x u, (x + 1) u) of its sequence
                           // (none past the sequence's end: an empty part)
  int32_t n_parts;         // n_splits, + n_mix_parts, + 1 with lossless pages (matrix-core path);
                           // 1 = the decode kernel writes out directly
  int32_t kernel;          // VK_DECODE_VALU or VK_DECODE_MFMA
  int32_t units_per_iter;  // matrix-core kernel: prefetch depth in 16-token units (4 or 8)
  int32_t steal;           // matrix-core kernel: 12-wave blocks whose waves take 16-unit pieces of
                           // the block's units from a shared counter
  int32_t lossless;        // the launch attends lossless pages: after the main launch, one more launch
                           // (an instance that reads them) writes part n_splits + n_mix_parts
  int32_t n_mix_parts;     // parts n_splits .. n_splits + n_mix_parts - 1 hold the fp8 / fp16 pages
  int32_t part_base;       // part index of blockIdx.z == 0
  float scale_log2;        // softmax scale * log2(e)
  int32_t slots[kDecodeMaxSeqs];   // launch order: longest attended range first
  int32_t lens[kDecodeMaxSeqs];
  int32_t rows[kDecodeMaxSeqs];    // query / output row (within the launch) of each
  int32_t mix[kDecodeMaxSeqs][4];  // two logical-unit ranges holding every fp8 / fp16 unit
  // Matrix-core path, optional: the launch's blocks in dispatch order, (part << 8) | sequence
  // index per entry, every (sequence, part) once; the grid is then (hkv, n_order).  0 = the
  // grid (hkv, n_seqs, n_parts) in that order.
  uint32_t* part_count;    // [n_seqs][hkv]: parts finished in this launch (0 before and after it)
  int32_t fused_merge;     // matrix-core path with n_parts > 1 and no lossless launch: the last block
                           // of each (sequence, KV head) merges its parts (no k_merge launch)
  int32_t n_order;
  uint16_t order[kDecodeMaxOrder];
};
static_assert(sizeof(DecodeArgs) <= 4096, "decode kernel arguments within 4 KB");

struct QuantArgs {
  const uint16_t* x;
  uint8_t* packed;
  const float* gamma_in;   // NULL: compute
  float* gamma_out;
  double* partials;        // [n_blk]
  SegInfo* seg;            // [1]
  int64_t n;
  int32_t dtype;
  int32_t n_blk;
  float eps;
};

// Allocation-free flat quantise+pack: its scratch is a device array of the library, sized for
// tensors of up to 2^31 elements (one float64 partial per absmean block, after a 256-byte
// finalize record).
constexpr int64_t kQuantNoAllocMaxElems = int64_t(1) << 31;
constexpr int64_t kQuantNoAllocScratchBytes = 256 + (kQuantNoAllocMaxElems / kAbsElemsPerBlock) * 8;

struct RetierArgs {
  PoolsView P;
  const RetierTask* tasks;  // [n_tasks]
  int32_t n_tasks;
  float eps;
};

// Optional per-launch timing: launchers bracket each kernel with begin/end
// (kind = VK_KERNEL_* of vk.h).  nullptr = no timing.
class LaunchTimer {
 public:
  virtual ~LaunchTimer() = default;
  virtual void begin(int kind, hipStream_t s) = 0;
  virtual void end(int kind, hipStream_t s) = 0;
};

// Launchers (vk_write.hip, vk_decode.hip, vk_retier.hip).  Return the first HIP error.
hipError_t launch_append(const AppendArgs& a, hipStream_t s, LaunchTimer* t);
hipError_t launch_decode(const DecodeArgs& a, int32_t group, hipStream_t s, LaunchTimer* t);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_retier(const RetierArgs& a, hipStream_t s, LaunchTimer* t);
// Device address of the allocation-free scratch on the current device (looked up on the first
// call per device, then cached).
hipError_t quantize_noalloc_scratch(void** ptr);

}  // namespace vk
