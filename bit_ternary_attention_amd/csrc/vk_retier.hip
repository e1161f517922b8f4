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
//   sum     of |v| over the page part as an exact integer (every e4m3fn
//           magnitude is an integer multiple of 2^-9, at most 448 * 2^9), so
//           gamma = float32(s * sum / N) matches the float64 mean exactly
//           whenever s * sum is exact (s a power of two);
//   codes   a code is nonzero exactly when the byte's magnitude index reaches
//           a threshold index found from the 127 possible float32 values s * v
//           (see vk_write.hip for why the compare |x| > d * (1/2 + 2^-25) in
//           float64 is the RNE float32 RoundClip); keys map four FP8 bytes to
//           one packed byte in place order, values are regrouped into per-unit
//           chunks (chunk 4c + g = tokens 4g..4g+3 of dimensions 16j + c) read
//           straight from the FP8 value tile's [D][Bs] rows.
// A page part of up to 16 KiB (block 16, 8 heads of 128) is read once, in the
// layout the codes need, and kept in registers; larger ones are read twice.
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

typedef float f2_t __attribute__((ext_vector_type(2)));

// Sum of |v| * 2^9 over the four e4m3fn bytes of w, exact: the hardware conversion gives
// each value exactly; their float32 sum (a multiple of 2^-9 below 2^11) is exact.
__device__ __forceinline__ float abs_sum4f(uint32_t w) {
  const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  return (fabsf(lo.x) + fabsf(lo.y)) + (fabsf(hi.x) + fabsf(hi.y));
}

// Same over sixteen bytes, as an integer (at most 16 * 448 * 2^9 < 2^24: exact in float32).
__device__ __forceinline__ uint32_t abs_sum16(uint4 w) {
  const float s = (abs_sum4f(w.x) + abs_sum4f(w.y)) + (abs_sum4f(w.z) + abs_sum4f(w.w));
  return static_cast<uint32_t>(s * 512.0f);
}

// Per byte of w: the 2-bit field u = code + 1 (0, 1 or 2) in the byte's low bits, with
// nz = (magnitude index >= T) and ng = sign: u = 1 + nz - 2 nz ng.  Adding 0x80 - T to
// the index sets bit 7 exactly when index >= T (no carry between bytes: index <= 0x7F,
// 0x80 - T <= 0x80).
__device__ __forceinline__ uint32_t fields4(uint32_t w, uint32_t add) {
  const uint32_t nzb = ((w & 0x7F7F7F7Fu) + add) & 0x80808080u;  // nz in bit 7 of each byte
  return 0x01010101u + (nzb >> 7) - ((nzb & w) >> 6);
}

// The four fields of w's bytes packed into one byte, byte i at bits 2i:
// 0x55 + sum_i nz_i 4^i - 2 sum_i nz_i ng_i 4^i, as two byte dot products.
__device__ __forceinline__ uint32_t key_byte(uint32_t w, uint32_t add) {
  const uint32_t nzb = ((w & 0x7F7F7F7Fu) + add) & 0x80808080u;
  const uint32_t pos = __builtin_amdgcn_udot4(nzb >> 7, 0x40100401u, 0x55u, false);
  return static_cast<uint32_t>(
      __builtin_amdgcn_sdot4(static_cast<int>((nzb & w) >> 7), static_cast<int>(0x80E0F8FEu),  // -2, -8, -32, -128
                             static_cast<int>(pos), false));
}

// Fixed-order block sum of the per-thread integer sums.
__device__ __forceinline__ unsigned long long block_sum(unsigned long long x, unsigned long long* part) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  return part[0] + part[1] + part[2] + part[3];
}

struct Scale {
  float gamma;
  uint32_t add;  // (0x80 - T) in every byte: magnitude indices >= T have a nonzero code
};

// gamma = float32(s * sum / n) from the exact integer sum of |v| * 2^9, and the index threshold.
__device__ __forceinline__ Scale page_scale(unsigned long long total, int64_t n, float s, float eps) {
  Scale r;
  r.gamma = static_cast<float>(static_cast<double>(total) * 0x1p-9 * static_cast<double>(s) / static_cast<double>(n));
  const float d = r.gamma + eps;
  uint32_t thresh = 0x80u;  // no index reaches it: every code 0
  if (d > 0.0f) {
    // the values s * v(m) rise with m, so the indices with s * v(m) <= tau form a prefix
    const int lane = threadIdx.x & 63;
    const double tau = static_cast<double>(d) * (0.5 + 0x1p-25);
    const float v0 = s * (static_cast<float>(e4m3_x512(lane)) * 0x1p-9f);
    const float v1 = s * (static_cast<float>(e4m3_x512(lane + 64)) * 0x1p-9f);
    const unsigned long long b0 = __ballot(static_cast<double>(v0) <= tau);
    const unsigned long long b1 = __ballot(lane + 64 < 127 && static_cast<double>(v1) <= tau);
    thresh = static_cast<uint32_t>(__popcll(b0) + __popcll(b1));
  }
  r.add = (0x80u - thresh) * 0x01010101u;
  return r;
}

__device__ __forceinline__ uint32_t key_word(uint4 w, uint32_t add) {
  return key_byte(w.x, add) | (key_byte(w.y, add) << 8) | (key_byte(w.z, add) << 16) | (key_byte(w.w, add) << 24);
}

// One value chunk: x[j] = FP8 bytes of tokens 4g..4g+3 (little-endian) of dimension 16j + c;
// byte r of `add` belongs to token 4g + r.  Dimensions are taken two at a time: one byte
// permute puts bytes (b0, b1) of x[j] and x[j+1] side by side, so their fields land two
// bits apart (the add bytes are permuted the same way).
template <int D>
__device__ __forceinline__ void store_chunk(const uint32_t* x, uint32_t add, uint8_t* out) {
  const uint32_t add01 = __builtin_amdgcn_perm(add, add, 0x01010000u);  // tokens 0, 0, 1, 1
  const uint32_t add23 = __builtin_amdgcn_perm(add, add, 0x03030202u);  // tokens 2, 2, 3, 3
  uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
  for (int j = 0; j < D / 16; j += 2) {
    // [x_j.b0, x_j+1.b0, x_j.b1, x_j+1.b1] and the same of bytes 2, 3
    const uint32_t f01 = fields4(__builtin_amdgcn_perm(x[j + 1], x[j], 0x05010400u), add01);
    const uint32_t f23 = fields4(__builtin_amdgcn_perm(x[j + 1], x[j], 0x07030602u), add23);
    const uint32_t t01 = (f01 & 0x00030003u) | ((f01 >> 6) & 0x000C000Cu);  // bits 0-3, 16-19
    const uint32_t t23 = (f23 & 0x00030003u) | ((f23 >> 6) & 0x000C000Cu);
    if (D == 64) {
      // one word: token 4g at bits 2j, 4g+2 at 8+2j, 4g+1 at 16+2j, 4g+3 at 24+2j
      w0 |= (t01 << (2 * j)) | (t23 << (8 + 2 * j));
    } else if (j < 8) {
      // word 0: token 4g at bits 2j, 4g+1 at bits 16+2j; word 1: tokens 4g+2, 4g+3
      w0 |= t01 << (2 * j);
      w1 |= t23 << (2 * j);
    } else {
      // head dim 256: words 2 and 3 the same for dimensions 16j + c with j >= 8
      w2 |= t01 << (2 * (j - 8));
      w3 |= t23 << (2 * (j - 8));
    }
  }
  if (D == 256) *reinterpret_cast<uint4*>(out) = make_uint4(w0, w1, w2, w3);
  else if (D == 128) *reinterpret_cast<uint2*>(out) = make_uint2(w0, w1);
  else *reinterpret_cast<uint32_t*>(out) = w0;
}

constexpr int kRegBytes = kRetierThreads * 64;  // page parts up to this size stay in registers

template <int D>
__global__ __launch_bounds__(kRetierThreads) void k_retier(RetierArgs a) {
  __shared__ unsigned long long part[kRetierThreads / 64];
  const RetierTask t = a.tasks[blockIdx.x];
  const int layer = blockIdx.y, kv = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = a.P.hkv, bs = a.P.bs, units = bs >> 4;
  const int64_t n = static_cast<int64_t>(hkv) * bs * D;  // FP8 bytes of this page part
  const uint8_t* src = a.P.pool[VK_FMT_FP8E4M3] +
                       (static_cast<int64_t>(layer) * a.P.cap[VK_FMT_FP8E4M3] + t.src) * a.P.page_bytes[VK_FMT_FP8E4M3] +
                       kv * n;
  uint8_t* dst = a.P.pool[VK_FMT_TERNARY2] +
                 (static_cast<int64_t>(layer) * a.P.cap[VK_FMT_TERNARY2] + t.dst) * a.P.page_bytes[VK_FMT_TERNARY2] +
                 kv * (n / 4);
  // value chunks: lane = chunk 4c + g holds tokens 4g..4g+3 of dimensions 16j + c of one
  // (head, 16-token unit) pair; its FP8 bytes are one 32-bit word per dimension row
  const int c = lane >> 2, g = lane & 3;
  auto vsrc = [&](int pair) {
    const int h = pair / units, u = pair - h * units;
    return src + static_cast<int64_t>(h) * bs * D + 16 * u + 4 * g;
  };
  auto vdst = [&](int pair) {
    const int h = pair / units, u = pair - h * units;
    return dst + static_cast<int64_t>(h) * bs * (D / 4) + u * 4 * D + lane * (D / 16);
  };
  Scale sc;

  if (n <= kRegBytes) {
    // the whole part in registers: one read, the integer sum, then the codes
    if (kv == 0) {
      // keys: [head][token][D] bytes -> [head][token][D/4], four bytes to one in order
      uint4 w[4];
      unsigned long long acc = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = tid + r * kRetierThreads;
        w[r] = i < n / 16 ? *reinterpret_cast<const uint4*>(src + 16 * i) : make_uint4(0, 0, 0, 0);
        acc += abs_sum16(w[r]);
      }
      sc = page_scale(block_sum(acc, part), n, a.P.fp8_scale, a.eps);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t i = tid + r * kRetierThreads;
        if (i < n / 16) *reinterpret_cast<uint32_t*>(dst + 4 * i) = key_word(w[r], sc.add);
      }
    } else {
      constexpr int NJ = D / 16, NP = 16 / NJ;  // rows per chunk; pairs per wave, at most
      const int pairs = hkv * units;
      uint32_t x[NP][NJ];
      float accf = 0.0f;  // at most 64 values, each a multiple of 2^-9 below 2^9: exact
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pair = wave + 4 * p;
        const uint8_t* vs = vsrc(pair < pairs ? pair : 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          x[p][j] = pair < pairs ? *reinterpret_cast<const uint32_t*>(vs + static_cast<int64_t>(16 * j + c) * bs) : 0u;
          accf += abs_sum4f(x[p][j]);
        }
      }
      const unsigned long long acc = static_cast<unsigned long long>(accf * 512.0f);
      sc = page_scale(block_sum(acc, part), n, a.P.fp8_scale, a.eps);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pair = wave + 4 * p;
        if (pair < pairs) store_chunk<D>(x[p], sc.add, vdst(pair));
      }
    }
  } else {
    // large pages: sum, then read the part again (mostly from L2) for the codes
    unsigned long long acc = 0;
    for (int64_t i = tid; i < n / 16; i += kRetierThreads)
      acc += abs_sum16(*reinterpret_cast<const uint4*>(src + 16 * i));
    sc = page_scale(block_sum(acc, part), n, a.P.fp8_scale, a.eps);
    if (kv == 0) {
      for (int64_t i = tid; i < n / 16; i += kRetierThreads)
        *reinterpret_cast<uint32_t*>(dst + 4 * i) = key_word(*reinterpret_cast<const uint4*>(src + 16 * i), sc.add);
    } else {
      for (int pair = wave; pair < hkv * units; pair += kRetierThreads / 64) {
        const uint8_t* vs = vsrc(pair);
        uint32_t x[D / 16];
#pragma unroll
        for (int j = 0; j < D / 16; ++j) x[j] = *reinterpret_cast<const uint32_t*>(vs + static_cast<int64_t>(16 * j + c) * bs);
        store_chunk<D>(x, sc.add, vdst(pair));
      }
    }
  }
  if (tid == 0) {
    a.P.gamma[(static_cast<int64_t>(layer) * a.P.cap[VK_FMT_TERNARY2] + t.dst) * 2 + kv] = sc.gamma;
    if (layer == 0 && kv == 0)
      a.P.block_table[static_cast<int64_t>(t.slot) * a.P.max_pages + t.page] = t.dst;  // format 0 = ternary
  }
}

// Dynamic FP8 pages: every token has its own scale s_t (stored after each tile's codes),
// so x = s_t v.  Sum in float64: per token the float32 sum of |v| is exact, times s_t.
// A code is nonzero when float32(s_t v) > tau, i.e. when the byte's magnitude index reaches
// the token's own threshold index (a 7-step search over the 127 magnitudes).  Two passes.
__device__ __forceinline__ uint32_t thresh_index(float s, double tau) {
  uint32_t lo = 0, hi = 127;  // count of indices m with float32(s * v(m)) <= tau (a prefix)
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    const uint32_t mid = (lo + hi) >> 1;
    const bool le = static_cast<double>(s * (static_cast<float>(e4m3_x512(mid)) * 0x1p-9f)) <= tau;
    lo = le ? mid + 1 : lo;
    hi = le ? hi : mid;
  }
  return lo;
}

__device__ __forceinline__ double block_sum_f64(double x, double* part) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  return ((part[0] + part[1]) + part[2]) + part[3];
}

template <int D>
__global__ __launch_bounds__(kRetierThreads) void k_retier_dyn(RetierArgs a) {
  __shared__ double part[kRetierThreads / 64];
  const RetierTask t = a.tasks[blockIdx.x];
  const int layer = blockIdx.y, kv = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = a.P.hkv, bs = a.P.bs, units = bs >> 4;
  const int64_t tile = a.P.tile_bytes[VK_FMT_FP8E4M3];  // bs * D codes, then bs float32 scales
  const int64_t n = static_cast<int64_t>(hkv) * bs * D;
  const int64_t per_head = static_cast<int64_t>(bs) * D / 16;  // 16-byte key pieces per head
  const uint8_t* src = a.P.pool[VK_FMT_FP8E4M3] +
                       (static_cast<int64_t>(layer) * a.P.cap[VK_FMT_FP8E4M3] + t.src) * a.P.page_bytes[VK_FMT_FP8E4M3] +
                       kv * hkv * tile;
  uint8_t* dst = a.P.pool[VK_FMT_TERNARY2] +
                 (static_cast<int64_t>(layer) * a.P.cap[VK_FMT_TERNARY2] + t.dst) * a.P.page_bytes[VK_FMT_TERNARY2] +
                 kv * (n / 4);
  auto scale_of = [&](int h, int tok) {
    return *reinterpret_cast<const float*>(src + h * tile + static_cast<int64_t>(bs) * D + 4 * tok);
  };
  const int c = lane >> 2, g = lane & 3;

  double acc = 0.0;
  if (kv == 0) {
    for (int64_t i = tid; i < hkv * per_head; i += kRetierThreads) {
      const int h = static_cast<int>(i / per_head);
      const int64_t rem = i - h * per_head;
      const uint4 w = *reinterpret_cast<const uint4*>(src + h * tile + 16 * rem);
      const float s16 = (abs_sum4f(w.x) + abs_sum4f(w.y)) + (abs_sum4f(w.z) + abs_sum4f(w.w));
      acc += static_cast<double>(s16) * static_cast<double>(scale_of(h, static_cast<int>(16 * rem / D)));
    }
  } else {
    for (int pair = wave; pair < hkv * units; pair += kRetierThreads / 64) {
      const int h = pair / units, u = pair - h * units;
      const uint8_t* vs = src + h * tile + 16 * u + 4 * g;
      float tok[4] = {0.f, 0.f, 0.f, 0.f};  // per token: at most D / 16 values, exact
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(vs + static_cast<int64_t>(16 * j + c) * bs);
        const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(x), false);
        const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(x), true);
        tok[0] += fabsf(lo.x); tok[1] += fabsf(lo.y); tok[2] += fabsf(hi.x); tok[3] += fabsf(hi.y);
      }
      const float4 s4 = *reinterpret_cast<const float4*>(src + h * tile + static_cast<int64_t>(bs) * D + 4 * (16 * u + 4 * g));
      acc += static_cast<double>(tok[0]) * s4.x + static_cast<double>(tok[1]) * s4.y +
             static_cast<double>(tok[2]) * s4.z + static_cast<double>(tok[3]) * s4.w;
    }
  }
  const double total = block_sum_f64(acc, part);
  const float gamma = static_cast<float>(total / static_cast<double>(n));
  const float d = gamma + a.eps;
  const double tau = static_cast<double>(d) * (0.5 + 0x1p-25);
  auto add_of = [&](float sc) { return d > 0.0f ? 0x80u - thresh_index(sc, tau) : 0u; };  // per byte

  if (kv == 0) {
    for (int64_t i = tid; i < hkv * per_head; i += kRetierThreads) {
      const int h = static_cast<int>(i / per_head);
      const int64_t rem = i - h * per_head;
      const uint4 w = *reinterpret_cast<const uint4*>(src + h * tile + 16 * rem);
      const uint32_t add = add_of(scale_of(h, static_cast<int>(16 * rem / D))) * 0x01010101u;
      *reinterpret_cast<uint32_t*>(dst + h * (per_head * 4) + 4 * rem) = key_word(w, add);
    }
  } else {
    for (int pair = wave; pair < hkv * units; pair += kRetierThreads / 64) {
      const int h = pair / units, u = pair - h * units;
      const uint8_t* vs = src + h * tile + 16 * u + 4 * g;
      const float4 s4 = *reinterpret_cast<const float4*>(src + h * tile + static_cast<int64_t>(bs) * D + 4 * (16 * u + 4 * g));
      const uint32_t add = add_of(s4.x) | (add_of(s4.y) << 8) | (add_of(s4.z) << 16) | (add_of(s4.w) << 24);
      uint32_t x[D / 16];
#pragma unroll
      for (int j = 0; j < D / 16; ++j) x[j] = *reinterpret_cast<const uint32_t*>(vs + static_cast<int64_t>(16 * j + c) * bs);
      store_chunk<D>(x, add, dst + static_cast<int64_t>(h) * bs * (D / 4) + u * 4 * D + lane * (D / 16));
    }
  }
  if (tid == 0) {
    a.P.gamma[(static_cast<int64_t>(layer) * a.P.cap[VK_FMT_TERNARY2] + t.dst) * 2 + kv] = gamma;
    if (layer == 0 && kv == 0)
      a.P.block_table[static_cast<int64_t>(t.slot) * a.P.max_pages + t.page] = t.dst;  // format 0 = ternary
  }
}

}  // namespace

hipError_t launch_retier(const RetierArgs& a, hipStream_t s, LaunchTimer* t) {
  if (a.n_tasks <= 0) return hipSuccess;
  const dim3 grid(a.n_tasks, a.P.n_layers, 2);
  if (t) t->begin(VK_KERNEL_RETIER, s);
  if (a.P.fp8_dynamic) {
    if (a.P.dim == 256) k_retier_dyn<256><<<grid, kRetierThreads, 0, s>>>(a);
    else if (a.P.dim == 128) k_retier_dyn<128><<<grid, kRetierThreads, 0, s>>>(a);
    else k_retier_dyn<64><<<grid, kRetierThreads, 0, s>>>(a);
  } else {
    if (a.P.dim == 256) k_retier<256><<<grid, kRetierThreads, 0, s>>>(a);
    else if (a.P.dim == 128) k_retier<128><<<grid, kRetierThreads, 0, s>>>(a);
    else k_retier<64><<<grid, kRetierThreads, 0, s>>>(a);
  }
  if (t) t->end(VK_KERNEL_RETIER, s);
  return hipGetLastError();
}

}  // namespace vk
