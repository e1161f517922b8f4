/*
 * vk.h - packed 2-bit ternary KV cache with direct decode attention (gfx950).
 *
 * C ABI of libvk.so.  Plain pointers and sizes only.
 *
 * What the library computes follows two pages:
 *   - "Show HN: Vantage-V-AI" (newshot.cc), section "core architecture":
 *     keys and values are quantised to ternary states {-1, 0, +1} with a
 *     per-tensor dynamic scale gamma = mean(|X|), packed four elements per
 *     uint8 (2.0 bits per element); attention-sink tokens (sink_tokens = 4)
 *     are retained beside a bounded recent window (quick start:
 *     max_active_tokens, sink_tokens, quant_mode).
 *   - "Minima-KV" (twodots.gr), sections "Recent, Anchor and Stale" and on
 *     mixed-format attention: recent pages stay FP8, anchor pages (the initial
 *     sinks) keep higher fidelity, older pages are packed; every page stays
 *     addressable through the block table and is read directly by
 *     format-specific branches whose partial softmax states are merged in
 *     logical page order; no dense copy of the cache exists.
 *
 * Conventions for every entry point:
 *   - Device pointers ("device") must be memory of the current HIP device, as
 *     returned by hipMalloc or by torch; host pointers ("host") are read or
 *     written before the call returns.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *     default stream) and reads/writes the caller's device buffers in stream
 *     order: they must stay valid until the stream has passed the call.
 *   - Every argument is checked on the host before anything is enqueued; on
 *     any error the cache is left exactly as it was and a message is available
 *     from vk_last_error() (thread-local).  A HIP failure after enqueueing has
 *     begun poisons the handle: later calls return VK_ERR_STATE.
 *   - No call allocates device memory except vk_create_cache.  Only
 *     vk_read_pages, vk_get_kernel_times and vk_release wait for the device.
 *     vk_append, vk_append_ragged and vk_retier stage their plans (descriptors
 *     and block-table entries) in a ring of pinned slots (up to 64, as many as
 *     fit 64 MiB); a call waits on the host only when every slot holds a plan
 *     that the device has not reached yet (64 calls queued ahead of the
 *     device at the workloads' sizes: back-pressure, as a full launch queue
 *     gives).
 *   - A handle is not thread-safe; distinct handles are independent.  Its calls
 *     share device scratch (the absmean partials of an append, the split partial
 *     states of a decode): calls on one handle that are enqueued on different
 *     streams must be ordered by the caller (an event between them), or they
 *     race on that scratch.
 */
#ifndef VK_H_
#define VK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VK_API __attribute__((visibility("default")))

typedef int32_t vk_status;
enum {
  VK_OK = 0,
  VK_ERR_ARG = 1,       /* an argument is out of range or inconsistent        */
  VK_ERR_OOM = 2,       /* device or pinned host allocation failed (create)   */
  VK_ERR_CAPACITY = 3,  /* not enough free pages of some format               */
  VK_ERR_ALIGN = 4,     /* append into a partly filled ternary page           */
  VK_ERR_STATE = 5,     /* handle poisoned by an earlier HIP failure          */
  VK_ERR_HIP = 6        /* a HIP runtime call failed                          */
};

/* 16-bit input element types */
enum { VK_DTYPE_F16 = 0, VK_DTYPE_BF16 = 1 };

/* page formats (the tiers of Minima-KV, "Recent, Anchor and Stale") */
enum {
  VK_FMT_TERNARY2 = 0,  /* 2-bit codes, 4 per byte, one float32 gamma per page for K and for V */
  VK_FMT_FP8E4M3 = 1,   /* OCP e4m3fn bytes of x / s, round to nearest even, saturating; s =
                           fp8_scale, or with fp8_dynamic s = float32(max|x| / 448) per (token,
                           KV head) vector (0 and codes 0 for a zero vector), stored after each
                           tile as block_size float32 values ("dynamic FP8 streaming mode" of
                           Show HN: Vantage-V-AI)                                              */
  VK_FMT_F16 = 2,       /* IEEE float16, round to nearest even from the input                    */
  VK_FMT_LOSSLESS = 3   /* bfloat16 kept exactly (bfloat16 input only): per 16-token unit and KV
                           head, K and V apart, the exponent fields coded in 4 bits around the
                           group's exponent centre (escapes to an exception list) beside one
                           sign+mantissa byte per value, or the raw values when the exceptions
                           overflow ("ExANS", ainews.dk: exponent / sign+mantissa streams with a
                           per-group exponent centre); a slot of 32 head_dim + 16 bytes per
                           group, of which the decode reads the header, the two streams and the
                           exceptions.  Like ternary pages, a lossless page is written by one
                           append                                                           */
};

/* decode kernels (same results within the decode tolerance; see vk_decode_attn) */
enum {
  VK_DECODE_DEFAULT = 0,  /* the library's choice (currently VK_DECODE_MFMA)                      */
  VK_DECODE_VALU = 1,     /* vector ALU: v_dot2_f32_f16 over unpacked codes, query rows in LDS (no
                             lossless pages: a config with them and this kernel is refused) */
  VK_DECODE_MFMA = 2      /* matrix cores: 16x16x32 f16 scores and P*V, pages staged in LDS by
                             buffer-to-LDS copies, codes unpacked to f16 in registers, query rows
                             resident as the B operand; fp8 / fp16 pages in one extra block per
                             (sequence, KV head) that writes its own partial state.  Opt-in
                             (environment VK_DECODE_STEAL=1: large launches, =2: whenever the
                             shape allows): all-ternary launches with at most one (sequence,
                             KV head) per compute unit run 12-wave blocks whose waves take
                             16-unit pieces from a shared counter; the summation order then
                             varies between calls, so outputs repeat only within the decode
                             tolerance (vk_stats.last_decode_steal reports the choice; never
                             at head_dim 256)                                                 */
};

typedef struct vk_cache vk_cache; /* opaque; owned by the library */

/*
 * Cache geometry and tiering.
 *
 * Page p of a sequence holds tokens [p*block_size, (p+1)*block_size).  When an
 * append brings a sequence to length L', each page it writes for the first
 * time takes: sink_format if p < ceil(sink_tokens / block_size); else
 * recent_format if recent_tokens > 0 and the page meets [L' - recent_tokens,
 * L'); else VK_FMT_TERNARY2.  A page keeps its format.  Pool capacities are per
 * layer; the block table is shared by all layers.
 */
typedef struct vk_cache_config {
  int32_t n_layers;           /* >= 1                                                  */
  int32_t n_kv_heads;         /* >= 1                                                  */
  int32_t n_q_heads;          /* multiple of n_kv_heads; n_q_heads/n_kv_heads in {1,2,4,8} */
  int32_t head_dim;           /* 64, 128 or 256 (256: no lossless pages)               */
  int32_t block_size;         /* tokens per page: power of two in [16, 65536]          */
  int32_t max_seqs;           /* sequence ids are 0 .. max_seqs-1                      */
  int32_t max_tokens_per_seq; /* >= 1                                                  */
  int32_t sink_tokens;        /* S >= 0 (the pages use 4)                              */
  int32_t sink_format;        /* VK_FMT_*                                              */
  int32_t recent_tokens;      /* R >= 0; 0 = no recent tier                            */
  int32_t recent_format;      /* VK_FMT_*                                              */
  int32_t decode_kernel;      /* VK_DECODE_*: which decode kernel reads the pages        */
  int32_t fp8_dynamic;        /* 0: FP8 pages use the static fp8_scale; 1: dynamic FP8, one
                                 float32 scale per (token, KV head) for K and for V       */
  int32_t reserved0;          /* 0                                                     */
  int64_t pages_ternary;      /* pool capacity per layer, pages (>= 0)                 */
  int64_t pages_fp8;
  int64_t pages_f16;
  float eps;                  /* added to gamma before dividing (default 1e-5), >= 0   */
  float fp8_scale;            /* static FP8 scale s > 0 (default 1.0)                  */
  uint64_t page_shuffle_seed; /* 0: pages are handed out in index order; else a seeded
                                 permutation of each free list (splitmix64 Fisher-Yates) */
  int64_t pages_lossless;     /* pool capacity per layer of VK_FMT_LOSSLESS pages (>= 0) */
} vk_cache_config;

/* Fills defaults: sink_tokens 4, sink/recent formats ternary/fp8, recent_tokens 0,
   eps 1e-5, fp8_scale 1; every size field 0 (the caller sets them). */
VK_API void vk_config_defaults(vk_cache_config* cfg);

/* Host only: checks cfg and returns the device bytes vk_create_cache would allocate. */
VK_API vk_status vk_cache_device_bytes(const vk_cache_config* cfg, int64_t* bytes);

/* Bytes of one page of `fmt` (K and V, every KV head) under cfg; 0 if invalid. */
VK_API int64_t vk_page_bytes(const vk_cache_config* cfg, int32_t fmt);

/* Allocates every device buffer (pools, gamma, block table, scratch, staging) on
   the current device.  *out is set only on success. */
VK_API vk_status vk_create_cache(const vk_cache_config* cfg, vk_cache** out);

/*
 * Quantise and pack new tokens into the cache (the write side).
 *
 * k, v: device, contiguous [n_layers][n_seqs][n_tokens][n_kv_heads][head_dim]
 *       of `dtype`, 16-byte aligned; layers layer_begin .. layer_begin+n_layers-1.
 * seq_ids: host, n_seqs distinct ids; each sequence grows by n_tokens.
 *
 * For every (layer, sequence, K|V) the ternary-routed tokens of this call form
 * one tensor whose gamma = mean(|X|) is reduced in float64 and rounded to
 * float32 (Show HN: Vantage-V-AI, core architecture); each element becomes
 * RoundClip(x / (gamma + eps), -1, 1) (ties to even), stored as code+1 in 2
 * bits.  Key tiles are token-major ([block][head_dim/4] bytes, element 4j+i at
 * bits 2i of byte j); value tiles are stored per 16-token unit, 64 chunks of
 * head_dim/16 bytes each, chunk 4c+g holding tokens 4g..4g+3 of the dimensions
 * 16j+c (head_dim 128: two little-endian words, word h with token 4g+2h in its
 * low and 4g+2h+1 in its high 16 bits, dimension 16j+c at bits 2j; head_dim 64:
 * one word, tokens 4g, 4g+2, 4g+1, 4g+3 in bytes 0..3, dimension 16j+c at bits
 * 2j of each byte; head_dim 256: four words, words 0 and 1 as head_dim 128
 * for j < 8, words 2 and 3 the same for j >= 8 at bits 2(j-8)).
 * gamma never returns to the host.
 *
 * Errors: VK_ERR_ARG (ids, sizes, pointers, dtype), VK_ERR_CAPACITY (pool
 * exhausted), VK_ERR_ALIGN (a sequence ends inside a ternary page).
 */
VK_API vk_status vk_append(vk_cache* c, int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                           const int32_t* seq_ids, int32_t n_tokens, const void* k, const void* v,
                           int32_t dtype, void* stream);

/*
 * Ragged append: as vk_append, with its own token count per sequence, so that
 * sequences of different lengths are written by one call (one launch of each
 * write-side kernel).  n_tokens: host, n_seqs counts >= 1.  k, v: device,
 * contiguous [n_layers][sum of n_tokens][n_kv_heads][head_dim]: within each
 * layer, sequence i's tokens follow sequence i-1's.  Each sequence is its own
 * gamma segment, exactly as in vk_append.  Errors as vk_append.
 */
VK_API vk_status vk_append_ragged(vk_cache* c, int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                  const int32_t* seq_ids, const int32_t* n_tokens, const void* k, const void* v,
                                  int32_t dtype, void* stream);

/*
 * One decode step of GQA attention for one layer (the read side).
 *
 * q: device [n_seqs][n_q_heads][head_dim] of q_dtype, any finite values: the
 *    queries of one (sequence, KV head) are scaled by one power of two before
 *    the products and the scores by its inverse, so bf16 queries beyond the f16
 *    range are taken exactly.  f16 operands (the largest magnitude brought to
 *    [2^14, 2^15)) for f16 queries, head_dim 64 and pages other than ternary;
 *    ternary keys at head_dim 128 and 256 with bf16 queries meet the query as the sum of
 *    two e4m3 terms (largest magnitude in [2^6, 2^7)), which hold every element
 *    of at least 2^-12 times the largest exactly and the smaller ones to within
 *    2^-20 times the largest.
 * out: device float32 [n_seqs][n_q_heads][head_dim].
 * Attended tokens of a sequence of length L: [0, min(sink_tokens, L)) and
 * [max(0, L - window), L); window = -1 attends the whole context (the
 * retention-preserving case of Minima-KV).  softmax_scale <= 0 means
 * 1/sqrt(head_dim).  Query head h reads KV head h / (n_q_heads/n_kv_heads).
 * Pages are read in their stored format through the block table; no dense
 * copy is made.  With several parts per (sequence, KV head) (split ranges,
 * fp8 / fp16 blocks) the matrix-core kernel's last block of each pair to finish
 * combines the partial softmax states (device-scope part counters that the
 * merging block sets back to zero); the vector-ALU kernel and launches with
 * lossless pages run a merge launch instead.  Both give the same bits.
 * Every sequence must have L >= 1.  n_seqs = 0 does nothing
 * and returns VK_OK (q and out may then be NULL).
 * The call only enqueues kernel launches on `stream` (no allocation, copy or
 * synchronisation), so it may be captured into a HIP graph.  A replay repeats
 * the launches as planned at capture (sequence lengths, window, split plan,
 * the page-format ranges of each sequence) and reads the pages and block table
 * current when it runs: it is valid while the captured sequences keep the
 * lengths and tier layout they had at capture.
 */
VK_API vk_status vk_decode_attn(vk_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                const void* q, int32_t q_dtype, int32_t window, float softmax_scale,
                                float* out, void* stream);

/*
 * Retiering: moves pages that have left the recent window from the FP8 tier to
 * the ternary tier ("Minima-KV", twodots.gr: section "Recent, Anchor and
 * Stale" names the FP8 recent tier and the packed older pages; the quality
 * section's evaluated profile retiers pages dynamically).
 *
 * For each listed sequence of length L, every page in VK_FMT_FP8E4M3 that is
 * not a sink page (p >= ceil(sink_tokens / block_size)) and ends at or before
 * L - recent_tokens is converted in every layer: x = fp8_scale * v (its
 * dequantised values); gamma = mean(|x|) over the page's block_size *
 * n_kv_heads * head_dim keys (and separately values), float32 of the exact
 * mean; codes RoundClip(x / (gamma + eps), -1, 1) with x in float32, packed
 * as vk_append packs them.  The page takes a ternary pool page, its FP8 page
 * returns to the FP8 free list, and its block-table entry is flipped on the
 * device.  Nothing happens when recent_tokens == 0 or recent_format is not
 * FP8.  Pages already examined are not looked at again, so calling it after
 * every append costs only the new pages.
 *
 * seq_ids: host, n_seqs distinct ids.  *n_pages (host, may be NULL) receives
 * the number of pages converted.  Call on the stream the cache's appends and
 * decodes use: the freed FP8 pages are handed out again by later appends.
 * Errors: VK_ERR_ARG (ids), VK_ERR_CAPACITY (not enough free ternary pages;
 * nothing changes).
 */
VK_API vk_status vk_retier(vk_cache* c, int32_t n_seqs, const int32_t* seq_ids, int64_t* n_pages, void* stream);

/*
 * Bounded-memory eviction ("Show HN: Vantage-V-AI", quick start: max_active_tokens
 * bounds the active attention window while sink_tokens are kept; core
 * architecture: a bounded-memory streaming cache with attention-sink retention).
 *
 * For each listed sequence of length L, frees every page past the sink pages
 * (p >= ceil(sink_tokens / block_size)) that ends at or before L - window, in
 * every layer: the tokens between the sinks and the window.  The pages return
 * to their free lists and are handed out again by later appends; calling it
 * after every append keeps a sequence within ceil(sink_tokens / block_size) +
 * ceil(window / block_size) + 1 pages.  Freed tokens are gone: a later
 * vk_decode_attn of the sequence fails with VK_ERR_ARG unless its window starts
 * at or after them (window >= 0 and L' - window' >= the end of the freed pages),
 * and vk_read_pages reports such pages with format -1.  window = -1 frees
 * nothing.  Host state only: nothing is enqueued and nothing waits; `stream`
 * names the stream of the cache's appends (see vk_reset_seqs for the ordering).
 *
 * seq_ids: host, n_seqs distinct ids.  *n_pages (host, may be NULL) receives
 * the number of pages freed per layer.  Errors: VK_ERR_ARG (ids, window < -1).
 */
VK_API vk_status vk_evict(vk_cache* c, int32_t n_seqs, const int32_t* seq_ids, int32_t window, int64_t* n_pages,
                          void* stream);

/* Frees every page of the given sequences and sets their length to 0 (host
   state only; nothing is enqueued and nothing waits).  Freed pages are handed
   out again by later vk_append calls; work already enqueued that reads them
   stays correct as long as those later appends go to the same stream (stream
   order), so callers that use several streams must order them.  `stream` names
   that stream and is not otherwise used. */
VK_API vk_status vk_reset_seqs(vk_cache* c, int32_t n_seqs, const int32_t* seq_ids, void* stream);

/* Current length of a sequence (host-side state; no device access). */
VK_API vk_status vk_seq_length(vk_cache* c, int32_t seq, int32_t* length);

/*
 * Introspection, synchronous (waits for the device): copies pages
 * [page0, page0+n_pages) of (layer, seq) to host (a page freed by vk_evict
 * reads as zeros with format -1).  Page j lands at
 * host_bytes + j * vk_page_bytes(cfg, VK_FMT_LOSSLESS) (the largest page), laid out
 * [K tile head 0..Hkv-1][V tile head 0..Hkv-1] in its own format.
 * host_fmt[j] receives the format; host_gamma[2j], [2j+1] the K and V gamma
 * of ternary pages (NaN otherwise).  Pages must be allocated.
 */
VK_API vk_status vk_read_pages(vk_cache* c, int32_t layer, int32_t seq, int32_t page0, int32_t n_pages,
                               uint8_t* host_bytes, int32_t* host_fmt, float* host_gamma);

typedef struct vk_stats {
  int64_t device_bytes;             /* all device memory owned by the handle              */
  int64_t pool_pages[4];            /* capacity per layer, by format (VK_FMT_*)           */
  int64_t pages_used[4];            /* allocated pages per layer, by format               */
  int64_t tokens_stored[4];         /* tokens held, by format (per layer)                 */
  int64_t append_calls, decode_calls;
  int64_t last_decode_units[4];     /* 16-token units read by the last decode, by format  */
  int64_t total_decode_units[4];    /* route counters over the handle's life              */
  int32_t last_decode_splits;       /* split-K factor the last decode used                */
  int32_t last_decode_steal;        /* 1 if its matrix-core launches used stealing blocks */
  int64_t retier_calls;             /* vk_retier calls                                    */
  int64_t pages_retiered;           /* pages moved from FP8 to ternary (each in every layer) */
  int64_t pages_evicted;            /* pages freed by vk_evict                            */
  int32_t last_decode_ordered;      /* 1 if its matrix-core launches dispatched their blocks
                                       heaviest first from a host-planned order (sequences of
                                       different lengths, or fp8 / fp16 parts)              */
  int32_t reserved;                 /* 0                                                   */
} vk_stats;

VK_API vk_status vk_get_stats(vk_cache* c, vk_stats* out);

/*
 * Kernel timing (observability).  While enabled, every kernel the handle
 * launches is bracketed by two HIP events on its stream, and the handle
 * accumulates per kernel kind: launches, device milliseconds and algorithmic
 * bytes (the bytes the operation must move: inputs read once per pass,
 * outputs written once; ternary pages D/4 bytes per token and head).
 */
enum {
  VK_KERNEL_ABSMEAN = 0,   /* write side pass 1: mean |x| partial sums        */
  VK_KERNEL_FINALIZE = 1,  /* (unused: the pack kernel derives gamma and the   */
                           /*  code threshold of each segment itself)         */
  VK_KERNEL_PACK = 2,      /* write side pass 2: quantise, pack, scatter      */
  VK_KERNEL_DECODE = 3,    /* paged decode attention (with the split merge     */
                           /*  when the kernel combines the parts itself)     */
  VK_KERNEL_MERGE = 4,     /* split-K online-softmax merge launch             */
  VK_KERNEL_RETIER = 5,    /* FP8 -> ternary page conversion (vk_retier)      */
  VK_KERNEL_COUNT = 6
};
/* enable != 0 starts timing and clears the totals; 0 stops it. */
VK_API vk_status vk_set_kernel_timing(vk_cache* c, int32_t enable);
/* Waits for the device and returns totals per kind (arrays of VK_KERNEL_COUNT);
   any pointer may be NULL. */
VK_API vk_status vk_get_kernel_times(vk_cache* c, int64_t* launches, double* milliseconds, double* bytes);

/* Waits for the device, then frees everything.  NULL is a no-op. */
VK_API vk_status vk_release(vk_cache* c);

/*
 * Flat per-tensor quantise+pack (the write side on a plain tensor).
 *
 * x: device, n elements of dtype (n % 8 == 0, 16-byte aligned).
 * gamma_in: device float32 or NULL.  NULL: gamma = mean(|x|) (float64 sum,
 *           rounded to float32) is computed and written to *gamma_out
 *           (device).  Otherwise *gamma_in is used as gamma and copied to
 *           *gamma_out.
 * packed: device, n/4 bytes; element 4j+i at bits 2i of byte j, code+1.
 * workspace: device scratch of at least vk_quantize_pack_workspace_bytes(n).
 */
VK_API int64_t vk_quantize_pack_workspace_bytes(int64_t n);
VK_API vk_status vk_quantize_pack(const void* x, int64_t n, int32_t dtype, float eps, const float* gamma_in,
                                  uint8_t* packed, float* gamma_out, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/*
 * Allocation-free flat quantise+pack, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments and results as
 * vk_quantize_pack without the workspace: the absmean partials and the
 * finalize record live in a device array of the library, 1 MiB + 256 bytes,
 * held by every device the library runs on until the process ends; its device
 * address is looked up on the first call on each device.  Nothing is
 * allocated and nothing waits.  n <= vk_quantize_pack_noalloc_max_elems()
 * (2^31), else VK_ERR_CAPACITY and nothing is enqueued.  Every call on one
 * device uses the same scratch: calls whose device work may overlap (on
 * different streams of one device, without ordering between them) race and
 * give wrong results; calls ordered on one stream are safe.
 */
VK_API int64_t vk_quantize_pack_noalloc_max_elems(void);
VK_API vk_status vk_quantize_pack_noalloc(const void* x, int64_t n, int32_t dtype, float eps, const float* gamma_in,
                                          uint8_t* packed, float* gamma_out, void* stream);

/* Thread-local text of the last error ("" if none). */
VK_API const char* vk_last_error(void);

/* Name of a status code. */
VK_API const char* vk_status_string(vk_status s);

#ifdef __cplusplus
}
#endif

#endif /* VK_H_ */
