// Retiering for gfx950: FP8 recent pages that have left the recent window are
// re-encoded as ternary pages and their block-table entries flipped.
//
// Follows "Minima-KV" (twodots.gr): section "Recent, Anchor and Stale" (recent
// pages in FP8, older pages packed, all addressable through the block table)
// and the quality section (the evaluated profile retiers pages dynamically).
// The packed encoding is the one of "Show HN: Vantage-V-AI" (newshot.cc),
// section "core architecture": gamma = mean(|X|), codes RoundClip(X / (gamma +
// eps), -1, 1), four per byte; here the tensor is one page's K (or V) over all
// heads, and X are the dequantised FP8 values s * v.
//
// One 256-thread block per (page, layer, K|V):
//   pass 1  sum of |v| over the page part as an exact integer (every e4m3fn
//           magnitude is an integer multiple of 2^-9, at most 448 * 2^9), so
//           gamma = float32(s * sum / N) matches the float64 mean exactly
//           whenever s * sum is exact (s a power of two);
//   pass 2  the same bytes again (from L2): a code is nonzero exactly when the
//           byte's magnitude index reaches a threshold index found from the
//           127 possible float32 values s * v (see vk_write.hip for why the
//           compare |x| > d * (1/2 + 2^-25) in float64 is the RNE float32
//           RoundClip); keys map four FP8 bytes to one packed byte in place
//           order, values are regrouped into per-unit chunks (chunk 4c + g =
//           tokens 4g..4g+3 of dimensions 16j + c) read straight from the FP8
//           value tile's [D][Bs] rows.
#include <hip/hip_runtime.h>

#include "host_state.h"
#include "vk_params.h"

namespace vk {
namespace {

constexpr int kRetierThreads = 256;

// e4m3fn magnitude index m (0..126) times 2^9: an exact integer.
__device__ __forceinline__ uint32_t e4m3_x512(uint32_t m) {
  const uint32_t e = m >> 3, f = m & 7u;
  return e == 0 ? f : (8u + f) << (e - 1);
}

__device__ __forceinline__ uint32_t abs_sum16(uint4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int b = 0; b < 4; ++b) s += e4m3_x512((ws[k] >> (8 * b)) & 0x7Fu);
  return s;
}

// Per byte of w: the 2-bit field u = code + 1 (0, 1 or 2) in the byte's low bits.
// nz = magnitude index >= T (no carry between bytes: index <= 0x7F, 0x80 - T <= 0x80).
__device__ __forceinline__ uint32_t fields4(uint32_t w, uint32_t thresh) {
  const uint32_t y = (w & 0x7F7F7F7Fu) + (0x80u - thresh) * 0x01010101u;
  const uint32_t nz = (y >> 7) & 0x01010101u;
  const uint32_t ng = (w >> 7) & 0x01010101u;
  return 0x01010101u + nz - ((nz & ng) << 1);
}

// Four fields (one per byte) packed into one byte, byte i at bits 2i.
__device__ __forceinline__ uint32_t pack4(uint32_t u) {
  return (u & 3u) | ((u >> 6) & 0xCu) | ((u >> 12) & 0x30u) | ((u >> 18) & 0xC0u);
}

template <int D>
__global__ __launch_bounds__(kRetierThreads) void k_retier(RetierArgs a) {
  __shared__ unsigned long long part[kRetierThreads / 64];
  const RetierTask t = a.tasks[blockIdx.x];
  const int layer = blockIdx.y, kv = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = a.P.hkv, bs = a.P.bs;
  const int64_t n = static_cast<int64_t>(hkv) * bs * D;  // FP8 bytes of this page part
  const uint8_t* src = a.P.pool[VK_FMT_FP8E4M3] +
                       (static_cast<int64_t>(layer) * a.P.cap[VK_FMT_FP8E4M3] + t.src) * a.P.page_bytes[VK_FMT_FP8E4M3] +
                       kv * n;
  uint8_t* dst = a.P.pool[VK_FMT_TERNARY2] +
                 (static_cast<int64_t>(layer) * a.P.cap[VK_FMT_TERNARY2] + t.dst) * a.P.page_bytes[VK_FMT_TERNARY2] +
                 kv * (n / 4);

  // pass 1: exact integer sum of |v| * 2^9
  unsigned long long acc = 0;
  for (int64_t i = tid; i < n / 16; i += kRetierThreads)
    acc += abs_sum16(*reinterpret_cast<const uint4*>(src + 16 * i));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  const unsigned long long total = part[0] + part[1] + part[2] + part[3];

  const float s = a.P.fp8_scale;
  const float gamma =
      static_cast<float>(static_cast<double>(total) * 0x1p-9 * static_cast<double>(s) / static_cast<double>(n));
  const float d = gamma + a.eps;
  uint32_t thresh = 0x80u;  // no index reaches it: every code 0
  if (d > 0.0f) {
    // the values s * v(m) rise with m, so the indices with s * v(m) <= tau form a prefix
    const double tau = static_cast<double>(d) * (0.5 + 0x1p-25);
    const float v0 = s * (static_cast<float>(e4m3_x512(lane)) * 0x1p-9f);
    const float v1 = s * (static_cast<float>(e4m3_x512(lane + 64)) * 0x1p-9f);
    const unsigned long long b0 = __ballot(static_cast<double>(v0) <= tau);
    const unsigned long long b1 = __ballot(lane + 64 < 127 && static_cast<double>(v1) <= tau);
    thresh = static_cast<uint32_t>(__popcll(b0) + __popcll(b1));
  }
  if (tid == 0) {
    a.P.gamma[(static_cast<int64_t>(layer) * a.P.cap[VK_FMT_TERNARY2] + t.dst) * 2 + kv] = gamma;
    if (layer == 0 && kv == 0)
      a.P.block_table[static_cast<int64_t>(t.slot) * a.P.max_pages + t.page] = t.dst;  // format 0 = ternary
  }

  // pass 2
  if (kv == 0) {
    // keys: [head][token][D] bytes -> [head][token][D/4], four bytes to one in order
    for (int64_t i = tid; i < n / 16; i += kRetierThreads) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + 16 * i);
      const uint32_t o = pack4(fields4(w.x, thresh)) | (pack4(fields4(w.y, thresh)) << 8) |
                         (pack4(fields4(w.z, thresh)) << 16) | (pack4(fields4(w.w, thresh)) << 24);
      *reinterpret_cast<uint32_t*>(dst + 4 * i) = o;
    }
  } else {
    // values: FP8 tile [D][Bs] per head -> per 16-token unit, 64 chunks of D/16 bytes;
    // lane = chunk 4c + g holds tokens 4g..4g+3 of dimensions 16j + c
    const int c = lane >> 2, g = lane & 3;
    const int units = bs >> 4;
    for (int pair = wave; pair < hkv * units; pair += kRetierThreads / 64) {
      const int h = pair / units, u = pair - h * units;
      const uint8_t* tile = src + static_cast<int64_t>(h) * bs * D + 16 * u + 4 * g;
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const uint32_t f = fields4(*reinterpret_cast<const uint32_t*>(tile + static_cast<int64_t>(16 * j + c) * bs),
                                   thresh);
        const uint32_t r0 = f & 3u, r1 = (f >> 8) & 3u, r2 = (f >> 16) & 3u, r3 = f >> 24;
        if (D == 128) {
          // word 0: token 4g at bits 2j, 4g+1 at bits 16+2j; word 1: tokens 4g+2, 4g+3
          w0 |= (r0 << (2 * j)) | (r1 << (16 + 2 * j));
          w1 |= (r2 << (2 * j)) | (r3 << (16 + 2 * j));
        } else {
          // one word: token 4g at bits 2j, 4g+2 at 8+2j, 4g+1 at 16+2j, 4g+3 at 24+2j
          w0 |= (r0 << (2 * j)) | (r2 << (8 + 2 * j)) | (r1 << (16 + 2 * j)) | (r3 << (24 + 2 * j));
        }
      }
      uint8_t* out = dst + static_cast<int64_t>(h) * bs * (D / 4) + u * 4 * D + lane * (D / 16);
      if (D == 128) *reinterpret_cast<uint2*>(out) = make_uint2(w0, w1);
      else *reinterpret_cast<uint32_t*>(out) = w0;
    }
  }
}

}  // namespace

hipError_t launch_retier(const RetierArgs& a, hipStream_t s, LaunchTimer* t) {
  if (a.n_tasks <= 0) return hipSuccess;
  const dim3 grid(a.n_tasks, a.P.n_layers, 2);
  if (t) t->begin(VK_KERNEL_RETIER, s);
  if (a.P.dim == 128) k_retier<128><<<grid, kRetierThreads, 0, s>>>(a);
  else k_retier<64><<<grid, kRetierThreads, 0, s>>>(a);
  if (t) t->end(VK_KERNEL_RETIER, s);
  return hipGetLastError();
}

}  // namespace vk
