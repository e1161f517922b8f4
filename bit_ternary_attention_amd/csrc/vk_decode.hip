// Read side: paged GQA decode attention directly over packed ternary, FP8
// and FP16 pages, for gfx950.
//
// Follows "Minima-KV" (twodots.gr), section on mixed-format attention: each
// page is read in its own format as it is loaded (no dense copy), every
// branch produces a partial state (max score, sum of exponentials, output),
// and partial states are merged with one online-softmax normalisation in
// logical page order.  The attended set (first sink_tokens plus the recent
// window, or the whole context) follows "Show HN: Vantage-V-AI", quick start
// and core architecture.
//
// One wave per (sequence, KV head, split).  A split walks its attended
// 16-token units four at a time:
//   scores  lane = token: the key row's 2-bit codes are unpacked to f16
//           {-1, 0, +1} in registers (OR into the mantissa of 1024.0, then
//           subtract 1025) and dotted with the g query rows kept in LDS,
//           two dimensions per v_dot2_f32_f16, accumulated in float32;
//   softmax the reference max is shared by the wave (cross-lane max), so
//           probabilities of all four units are comparable; they go to LDS
//           as f16 (scaled by 2^14 to stay clear of f16 subnormals);
//   PV      lane = head dimension: the value tile is stored dimension-major,
//           so one 32-bit word holds 16 tokens of one dimension; pairs of
//           tokens are unpacked the same way and dotted with the matching
//           probability pairs; gamma_V (or the fp8 scale) is applied per unit.
// Splits write (o, max, sum) partials that k_merge combines; with one split
// the kernel writes the normalised output.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "host_state.h"
#include "vk_params.h"

namespace vk {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t x) { return __builtin_bit_cast(h2_t, x); }

__device__ __forceinline__ float dot2(uint32_t a, h2_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), b, c, false);
}

// Codes of bits [2i, 2i+1] of each 16-bit half of w, as f16 {-1, 0, +1}.
__device__ __forceinline__ h2_t tern2(uint32_t w, int i) {
  const uint32_t x = ((w >> (2 * i)) & 0x00030003u) | 0x64006400u;  // f16 1024 + u
  const h2_t off = {static_cast<_Float16>(1025.0f), static_cast<_Float16>(1025.0f)};
  return as_h2(x) - off;
}

// Two e4m3fn bytes (in the low byte of each 16-bit half) as exact f16 values.
__device__ __forceinline__ h2_t fp8x2(uint32_t x) {
  const uint32_t f = ((x & 0x007F007Fu) << 7) | ((x & 0x00800080u) << 8);  // value * 2^-8
  const h2_t k256 = {static_cast<_Float16>(256.0f), static_cast<_Float16>(256.0f)};
  return as_h2(f) * k256;
}

template <int QDT>
__device__ __forceinline__ uint32_t q_f16(uint16_t h) {
  if (QDT == 0) return h;
  return static_cast<uint32_t>(__half_as_ushort(__float2half_rn(__uint_as_float(static_cast<uint32_t>(h) << 16))));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

struct Units {
  int a_end, b_begin, b_end, sinks, w0;
  bool single;
};

// Same arithmetic as the host planner (attended_units in host_state.cpp).
__device__ __forceinline__ Units attended(int L, int S, int W) {
  Units r;
  r.sinks = min(S, L);
  const int all = (L + 15) >> 4;
  if (W < 0 || L - W <= r.sinks) {
    r.single = true;
    r.a_end = r.b_begin = r.b_end = all;
    r.w0 = 0;
    return r;
  }
  r.single = false;
  r.w0 = L - W;
  r.a_end = (r.sinks + 15) >> 4;
  if (W == 0) {
    r.b_begin = r.b_end = r.a_end;
  } else {
    r.b_begin = max(r.a_end, r.w0 >> 4);
    r.b_end = all;
  }
  return r;
}

template <int D, int G, int QDT>
__global__ __launch_bounds__(64) void k_decode(DecodeArgs a) {
  constexpr int DW = D / 16;   // 32-bit code words per key row
  constexpr int QP = D / 2;    // f16 pairs per query row
  constexpr int DPL = D / 64;  // value dimensions per lane
  constexpr int UPI = kDecodeUnitsPerIter;
  __shared__ uint32_t q2[G * QP];
  __shared__ uint32_t pbuf[UPI * G * 8];

  const int lane = threadIdx.x;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int slot = a.slots[b], L = a.lens[b];
  const PoolsView& P = a.P;
  const Units R = attended(L, a.sink_tokens, a.window);
  const int n_a = R.a_end;
  const int U = R.a_end + (R.b_end - R.b_begin);
  const int u_begin = static_cast<int>((static_cast<int64_t>(split) * U) / a.n_splits);
  const int u_end = static_cast<int>((static_cast<int64_t>(split + 1) * U) / a.n_splits);

  // query rows of this KV head's group, as f16 pairs (d, d+8) within each 16-dim block
  for (int j = lane; j < G * QP; j += 64) {
    const int hh = j / QP, jj = j % QP, w = jj >> 3, ii = jj & 7;
    const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * a.hq + kvh * G + hh) * D;
    q2[j] = q_f16<QDT>(qrow[16 * w + ii]) | (q_f16<QDT>(qrow[16 * w + 8 + ii]) << 16);
  }
  __syncthreads();

  float o[G][DPL];
  float m[G], lsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    lsum[hh] = 0.0f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[hh][j] = 0.0f;
  }
  const int64_t layer = a.layer;
  const int32_t* bt = P.block_table + static_cast<int64_t>(slot) * P.max_pages;
  const int us = lane >> 4, r = lane & 15;
  uint16_t* pb16 = reinterpret_cast<uint16_t*>(pbuf);

  for (int ub = u_begin; ub < u_end; ub += UPI) {
    // ---------------- scores: lane = token ----------------
    const int lu = ub + us;
    const bool uv = lu < u_end;
    const int u = lu < n_a ? lu : R.b_begin + (lu - n_a);
    const int t = u * 16 + r;
    const bool att = uv && (R.single ? t < L : (t < R.sinks || (t >= R.w0 && t < L)));
    float logit[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) logit[hh] = -INFINITY;
    if (uv) {
      const int page = (u * 16) >> P.bs_shift;
      const int upi = ((u * 16) & (P.bs - 1)) >> 4;
      const int32_t entry = bt[page];
      const int fmt = static_cast<int>(static_cast<uint32_t>(entry) >> 30);
      const int64_t idx = entry & 0x3FFFFFFF;
      const uint8_t* pg = P.pool[fmt] + (layer * P.cap[fmt] + idx) * P.page_bytes[fmt];
      float acc[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) acc[hh] = 0.0f;
      float kscale;
      if (fmt == VK_FMT_TERNARY2) {
        const uint4* krow = reinterpret_cast<const uint4*>(pg + kvh * P.tile_bytes[0] + (upi * 16 + r) * (D / 4));
        uint32_t kw[DW];
#pragma unroll
        for (int q4 = 0; q4 < DW / 4; ++q4) {
          const uint4 x = krow[q4];
          kw[4 * q4] = x.x; kw[4 * q4 + 1] = x.y; kw[4 * q4 + 2] = x.z; kw[4 * q4 + 3] = x.w;
        }
#pragma unroll
        for (int w = 0; w < DW; ++w) {
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const h2_t c2 = tern2(kw[w], ii);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) acc[hh] = dot2(q2[hh * QP + w * 8 + ii], c2, acc[hh]);
          }
        }
        kscale = P.gamma[(layer * P.cap[0] + idx) * 2];
      } else if (fmt == VK_FMT_FP8E4M3) {
        const uint4* krow = reinterpret_cast<const uint4*>(pg + kvh * P.tile_bytes[1] + (upi * 16 + r) * D);
#pragma unroll
        for (int w = 0; w < DW; ++w) {
          const uint4 x = krow[w];  // bytes 16w .. 16w+15
          const uint32_t lo[2] = {x.x, x.y}, hi[2] = {x.z, x.w};
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const uint32_t bl = (lo[ii >> 2] >> (8 * (ii & 3))) & 0xFFu;
            const uint32_t bh = (hi[ii >> 2] >> (8 * (ii & 3))) & 0xFFu;
            const h2_t c2 = fp8x2(bl | (bh << 16));
#pragma unroll
            for (int hh = 0; hh < G; ++hh) acc[hh] = dot2(q2[hh * QP + w * 8 + ii], c2, acc[hh]);
          }
        }
        kscale = P.fp8_scale;
      } else {
        const uint4* krow = reinterpret_cast<const uint4*>(pg + kvh * P.tile_bytes[2] + (upi * 16 + r) * D * 2);
#pragma unroll
        for (int w = 0; w < DW; ++w) {
          const uint4 x0 = krow[2 * w], x1 = krow[2 * w + 1];  // elements 16w..+7, 16w+8..+15
          const uint32_t lo[4] = {x0.x, x0.y, x0.z, x0.w}, hi[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const uint32_t a16 = (lo[ii >> 1] >> (16 * (ii & 1))) & 0xFFFFu;
            const uint32_t b16 = (hi[ii >> 1] >> (16 * (ii & 1))) & 0xFFFFu;
            const h2_t c2 = as_h2(a16 | (b16 << 16));
#pragma unroll
            for (int hh = 0; hh < G; ++hh) acc[hh] = dot2(q2[hh * QP + w * 8 + ii], c2, acc[hh]);
          }
        }
        kscale = 1.0f;
      }
      if (att) {
        const float ks = kscale * a.scale_log2;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) logit[hh] = acc[hh] * ks;
      }
    }

    // ---------------- online softmax, wave-wide reference ----------------
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mx = wave_max(logit[hh]);
      if (mx > m[hh]) {
        const float corr = exp2f(m[hh] - mx);  // 0 when m was -inf
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[hh][j] *= corr;
        lsum[hh] *= corr;
        m[hh] = mx;
      }
      const float p = (logit[hh] == -INFINITY) ? 0.0f : exp2f(logit[hh] - m[hh]);
      lsum[hh] += p;
      pb16[(us * G + hh) * 16 + r] = __half_as_ushort(__float2half_rn(p * 16384.0f));
    }
    __syncthreads();

    // ---------------- PV: lane = head dimension ----------------
#pragma unroll
    for (int us2 = 0; us2 < UPI; ++us2) {
      const int lu2 = ub + us2;
      if (lu2 >= u_end) break;
      const int u2 = lu2 < n_a ? lu2 : R.b_begin + (lu2 - n_a);
      const int page = (u2 * 16) >> P.bs_shift;
      const int upi = ((u2 * 16) & (P.bs - 1)) >> 4;
      const int32_t entry = __builtin_amdgcn_readfirstlane(bt[page]);
      const int fmt = static_cast<int>(static_cast<uint32_t>(entry) >> 30);
      const int64_t idx = entry & 0x3FFFFFFF;
      const uint8_t* vt = P.pool[fmt] + (layer * P.cap[fmt] + idx) * P.page_bytes[fmt] +
                          (P.hkv + kvh) * P.tile_bytes[fmt];
      const uint32_t* pp = pbuf + us2 * G * 8;
      float tmp[G][DPL];
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int j = 0; j < DPL; ++j) tmp[hh][j] = 0.0f;
      float vscale;
      if (fmt == VK_FMT_TERNARY2) {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int dd = lane * DPL + j;
          const uint32_t wv = reinterpret_cast<const uint32_t*>(vt)[dd * (P.bs >> 4) + upi];
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const h2_t c2 = tern2(wv, ii);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) tmp[hh][j] = dot2(pp[hh * 8 + ii], c2, tmp[hh][j]);
          }
        }
        vscale = P.gamma[(layer * P.cap[0] + idx) * 2 + 1];
      } else if (fmt == VK_FMT_FP8E4M3) {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int dd = lane * DPL + j;
          const uint4 x = *reinterpret_cast<const uint4*>(vt + static_cast<int64_t>(dd) * P.bs + upi * 16);
          const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const uint32_t wd = xs[ii >> 1] >> (16 * (ii & 1));  // tokens 2ii, 2ii+1 in bytes 0, 1
            const h2_t c2 = fp8x2((wd & 0xFFu) | ((wd & 0xFF00u) << 8));
#pragma unroll
            for (int hh = 0; hh < G; ++hh) tmp[hh][j] = dot2(pp[hh * 8 + ii], c2, tmp[hh][j]);
          }
        }
        vscale = P.fp8_scale;
      } else {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int dd = lane * DPL + j;
          const uint4* v4 = reinterpret_cast<const uint4*>(vt + (static_cast<int64_t>(dd) * P.bs + upi * 16) * 2);
          const uint4 x0 = v4[0], x1 = v4[1];
          const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) tmp[hh][j] = dot2(pp[hh * 8 + ii], as_h2(xs[ii]), tmp[hh][j]);
          }
        }
        vscale = 1.0f;
      }
      const float vs = vscale * (1.0f / 16384.0f);
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[hh][j] = fmaf(tmp[hh][j], vs, o[hh][j]);
    }
    __syncthreads();
  }

  // ---------------- write ----------------
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float l = wave_sum(lsum[hh]);
    const int64_t qh = static_cast<int64_t>(b) * a.hq + kvh * G + hh;
    if (a.n_splits == 1) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int j = 0; j < DPL; ++j) a.out[qh * D + lane * DPL + j] = o[hh][j] * inv;
    } else {
      float* part = a.partials + (qh * a.n_splits + split) * (D + 2);
#pragma unroll
      for (int j = 0; j < DPL; ++j) part[lane * DPL + j] = o[hh][j];
      if (lane == 0) {
        part[D] = m[hh];
        part[D + 1] = l;
      }
    }
  }
}

// Combines split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(D) void k_merge(DecodeArgs a) {
  const int64_t qh = static_cast<int64_t>(blockIdx.y) * a.hq + blockIdx.x;
  const int dd = threadIdx.x;
  const float* base = a.partials + qh * a.n_splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, base[s * (D + 2) + D]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float ls = base[s * (D + 2) + D + 1];
    if (ls > 0.0f) {
      const float w = exp2f(base[s * (D + 2) + D] - M);
      num = fmaf(w, base[s * (D + 2) + dd], num);
      den = fmaf(w, ls, den);
    }
  }
  a.out[qh * D + dd] = num / den;
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t s, LaunchTimer* t) {
  const dim3 grid(a.n_splits, a.P.hkv, a.n_seqs);
  if (t) t->begin(VK_KERNEL_DECODE, s);
  if (a.q_dtype == VK_DTYPE_BF16) k_decode<D, G, 1><<<grid, 64, 0, s>>>(a);
  else k_decode<D, G, 0><<<grid, 64, 0, s>>>(a);
  if (t) t->end(VK_KERNEL_DECODE, s);
  if (a.n_splits > 1) {
    if (t) t->begin(VK_KERNEL_MERGE, s);
    k_merge<D><<<dim3(a.hq, a.n_seqs), D, 0, s>>>(a);
    if (t) t->end(VK_KERNEL_MERGE, s);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int32_t group, hipStream_t s, LaunchTimer* t) {
  switch (group) {
    case 1: return launch_dg<D, 1>(a, s, t);
    case 2: return launch_dg<D, 2>(a, s, t);
    case 4: return launch_dg<D, 4>(a, s, t);
    case 8: return launch_dg<D, 8>(a, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int32_t group, hipStream_t s, LaunchTimer* t) {
  if (a.P.dim == 128) return launch_d<128>(a, group, s, t);
  if (a.P.dim == 64) return launch_d<64>(a, group, s, t);
  return hipErrorInvalidValue;
}

}  // namespace vk
