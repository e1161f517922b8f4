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
  uint8_t* pool[3];
  float* gamma;            // [n_layers][cap[0]][2]: K and V gamma of ternary pages
  int32_t* block_table;    // [max_seqs][max_pages]: (format << 30) | pool index
  int64_t cap[3];          // pages per layer
  int64_t tile_bytes[3];   // one (K|V, head) tile
  int64_t page_bytes[3];
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
  const uint16_t* k;       // [n_layers][n_seqs][n_tokens][hkv][dim]
  const uint16_t* v;
  const AppendSeqDesc* descs;
  const int32_t* entries;
  double* partials;        // [n_seg][n_blk]
  SegInfo* seg;            // [n_seg]
  int32_t dtype;           // 0 f16, 1 bf16
  int32_t layer_begin;
  int32_t n_layers;
  int32_t n_seqs;
  int32_t n_tokens;
  int32_t n_blk;           // absmean blocks per segment
  int32_t max_units;       // most 16-token units touched by one sequence
  int32_t all_ternary;     // every touched page is ternary (the pack kernel's lean instance)
  float eps;
};

constexpr int kDecodeMaxSeqs = 64;    // sequences per decode launch (kernel-argument table)
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
  int32_t n_parts;         // n_splits, or n_splits + 1 when part n_splits holds the fp8 / fp16
                           // pages (matrix-core path); 1 = the decode kernel writes out directly
  int32_t kernel;          // VK_DECODE_VALU or VK_DECODE_MFMA
  int32_t units_per_iter;  // matrix-core kernel: prefetch depth in 16-token units (4 or 8)
  int32_t steal;           // matrix-core kernel: 12-wave blocks whose waves take 16-unit pieces of
                           // the block's units from a shared counter
  float scale_log2;        // softmax scale * log2(e)
  int32_t slots[kDecodeMaxSeqs];   // launch order: longest attended range first
  int32_t lens[kDecodeMaxSeqs];
  int32_t rows[kDecodeMaxSeqs];    // query / output row (within the launch) of each
  int32_t mix[kDecodeMaxSeqs][4];  // two logical-unit ranges holding every fp8 / fp16 unit
};

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
hipError_t launch_append(const AppendArgs& a, int32_t n_seg, hipStream_t s, LaunchTimer* t);
hipError_t launch_decode(const DecodeArgs& a, int32_t group, hipStream_t s, LaunchTimer* t);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_retier(const RetierArgs& a, hipStream_t s, LaunchTimer* t);

}  // namespace vk
