// Read side: paged GQA decode attention directly over packed ternary, FP8
// and FP16 pages, for gfx950.
//
// Follows "Minima-KV" (twodots.gr), section on mixed-format attention: each
// page is read in its own format as it is loaded (no dense copy), every
// branch produces a partial state (max score, sum of exponentials, output),
// and partial states are merged with one online-softmax normalisation.  The
// attended set (first sink_tokens plus the recent window, or the whole
// context) follows "Show HN: Vantage-V-AI", quick start and core architecture.
//
// Two kernels compute the same thing:
//   k_decode_mfma (default): scores and P*V on the matrix cores (the g query
//     heads of a KV head share every unpacked code), pages staged in LDS by
//     buffer-to-LDS copies; see the section comment further down;
//   k_decode (vector ALU): one wave per (sequence, KV head, split), codes
//     unpacked to f16 {-1, 0, +1} pairs and dotted with v_dot2_f32_f16 against
//     the query rows in LDS (scores, lane = token) and the probabilities
//     (P*V, lane = head dimension).
// Splits write (o, max, sum) partials that k_merge combines; with a single
// part the kernel writes the normalised output.
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

// Query elements enter the products as f16.  bf16 queries reach 2^128, beyond f16, so every
// query of a (sequence, KV head) is first scaled by one power of two 2^sh that puts its
// largest magnitude in [2^14, 2^15) (exact: a power-of-two product of a 16-bit value), and the
// scores are multiplied back by 2^-sh.  Every element within 2^-28 of the largest stays exact
// in f16 (a normal f16 value); smaller ones round to the f16 subnormal grid.
template <int QDT>
__device__ __forceinline__ float q_value(uint16_t h) {
  if (QDT == 0) return static_cast<float>(__builtin_bit_cast(_Float16, h));
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return static_cast<uint32_t>(__half_as_ushort(__float2half_rn(x)));
}

// Exponent shift sh for a largest magnitude qmax (clamped to [-126, 126], where 2^sh and 2^-sh
// are normal floats; 0 for qmax = 0).
// TOP: the exponent the largest magnitude is brought to (14 for f16 operands).
template <int TOP = 14>
__device__ __forceinline__ int q_shift(float qmax) {
  if (!(qmax > 0.0f)) return 0;
  const int e = static_cast<int>((__float_as_uint(qmax) >> 23) & 0xFFu) - 127;  // floor(log2 qmax) for normals
  const int sh = TOP - e;
  return sh < -126 ? -126 : (sh > 126 ? 126 : sh);
}
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float(static_cast<uint32_t>(k + 127) << 23); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// max over the four 16-lane rows of each lane column (lanes l, l^16, l^32, l^48), with the
// gfx950 row-swap permutes (VALU only, no LDS round trip).  permlane16_swap(x, x) returns
// rows (0, 0, 2, 2) and (1, 1, 3, 3); permlane32_swap(x, x) returns halves (lo, lo), (hi, hi).
// (The swap results are copied to scalars before reinterpretation: a bit cast applied to a
// vector element directly reads element 0 with this compiler.)
__device__ __forceinline__ float max_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = r16[0], a1 = r16[1];
  x = fmaxf(__uint_as_float(a0), __uint_as_float(a1));
  const uint32_t v = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const uint32_t b0 = r32[0], b1 = r32[1];
  return fmaxf(__uint_as_float(b0), __uint_as_float(b1));
}

// sum over the four 16-lane rows of each lane column, with the same row-swap permutes
__device__ __forceinline__ float sum_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = r16[0], a1 = r16[1];
  x = __uint_as_float(a0) + __uint_as_float(a1);
  const uint32_t v = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  const uint32_t b0 = r32[0], b1 = r32[1];
  return __uint_as_float(b0) + __uint_as_float(b1);
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

// Same arithmetic as the host planner (attended_units in host_state.cpp), written with
// selects: no branch stands between a kernel's set-up loads.
__device__ __forceinline__ Units attended(int L, int S, int W) {
  Units r;
  r.sinks = min(S, L);
  const int all = (L + 15) >> 4;
  const int a_end = (r.sinks + 15) >> 4;
  r.single = W < 0 || L - W <= r.sinks;  // one range: the whole context
  r.w0 = r.single ? 0 : L - W;
  r.a_end = r.single ? all : a_end;
  r.b_begin = r.single ? all : (W == 0 ? a_end : max(a_end, (L - W) >> 4));
  r.b_end = r.single ? all : (W == 0 ? a_end : all);
  return r;
}

template <int D, int G, int QDT>
__global__ __launch_bounds__(64) void k_decode(DecodeArgs a) {
  constexpr int DW = D / 16;   // 32-bit code words per key row
  constexpr int QP = D / 2;    // f16 pairs per query row
  constexpr int DPL = D / 64;  // value dimensions per lane
  constexpr int UPI = kDecodeUnitsPerIter;
  // key words per pass of the score loop: head dim 256 takes its row in four passes that stay
  // a loop (their query reads from LDS are not hoisted into registers), the others in one
  constexpr int KW = D == 256 ? 4 : DW;
  __shared__ uint32_t q2[G * QP];
  __shared__ uint32_t pbuf[UPI * G * 8];
  __shared__ float vmax_s[UPI];  // dynamic FP8: largest value scale of each unit's 16 tokens

  const int lane = threadIdx.x;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int slot = a.slots[b], L = a.lens[b];
  const PoolsView& P = a.P;
  const Units R = attended(L, a.sink_tokens, a.window);
  const int n_a = R.a_end;
  const int U = R.a_end + (R.b_end - R.b_begin);
  const int u_begin = min(split * a.units_per_split, U);
  const int u_end = min(u_begin + a.units_per_split, U);

  // query rows of this KV head's group, as f16 pairs (d, d+8) within each 16-dim block, scaled
  // by 2^sh (q_shift); qsl = softmax scale * log2(e) * 2^-sh multiplies the scores
  const uint16_t* qgrp = a.q + (static_cast<int64_t>(a.rows[b]) * a.hq + kvh * G) * D;
  float qmax = 0.0f;
  for (int j = lane; j < G * D; j += 64) qmax = fmaxf(qmax, fabsf(q_value<QDT>(qgrp[j])));
  const int qsh = __builtin_amdgcn_readfirstlane(q_shift(wave_max(qmax)));
  const float qmul = pow2i(qsh), qsl = a.scale_log2 * pow2i(-qsh);
  for (int j = lane; j < G * QP; j += 64) {
    const int hh = j / QP, jj = j % QP, w = jj >> 3, ii = jj & 7;
    const uint16_t* qrow = qgrp + hh * D;
    q2[j] = f16_bits(q_value<QDT>(qrow[16 * w + ii]) * qmul) | (f16_bits(q_value<QDT>(qrow[16 * w + 8 + ii]) * qmul) << 16);
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
    float vsc = 1.0f;  // dynamic FP8: this token's value scale (1 elsewhere)
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
#pragma unroll 1
        for (int p0 = 0; p0 < DW; p0 += KW) {
          uint32_t kw[KW];
#pragma unroll
          for (int q4 = 0; q4 < KW / 4; ++q4) {
            const uint4 x = krow[p0 / 4 + q4];
            kw[4 * q4] = x.x; kw[4 * q4 + 1] = x.y; kw[4 * q4 + 2] = x.z; kw[4 * q4 + 3] = x.w;
          }
#pragma unroll
          for (int w = 0; w < KW; ++w) {
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
              const h2_t c2 = tern2(kw[w], ii);
#pragma unroll
              for (int hh = 0; hh < G; ++hh) acc[hh] = dot2(q2[hh * QP + (p0 + w) * 8 + ii], c2, acc[hh]);
            }
          }
        }
        kscale = P.gamma[(layer * P.cap[0] + idx) * 2];
      } else if (fmt == VK_FMT_FP8E4M3) {
        const uint4* krow = reinterpret_cast<const uint4*>(pg + kvh * P.tile_bytes[1] + (upi * 16 + r) * D);
#pragma unroll 1
        for (int p0 = 0; p0 < DW; p0 += KW) {
#pragma unroll
          for (int w = p0; w < p0 + KW; ++w) {
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
        }
        kscale = P.fp8_scale;
        if (P.fp8_dynamic) {  // the tiles' token scales follow their codes
          const int64_t so = static_cast<int64_t>(P.bs) * D + 4 * (upi * 16 + r);
          kscale = *reinterpret_cast<const float*>(pg + kvh * P.tile_bytes[1] + so);
          // a token slot past the sequence may hold a stale scale of a recycled page
          vsc = att ? *reinterpret_cast<const float*>(pg + (P.hkv + kvh) * P.tile_bytes[1] + so) : 0.0f;
        }
      } else {
        const uint4* krow = reinterpret_cast<const uint4*>(pg + kvh * P.tile_bytes[2] + (upi * 16 + r) * D * 2);
#pragma unroll 1
        for (int p0 = 0; p0 < DW; p0 += KW) {
#pragma unroll
          for (int w = p0; w < p0 + KW; ++w) {
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
        }
        kscale = 1.0f;
      }
      if (att) {
        const float ks = kscale * qsl;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) logit[hh] = acc[hh] * ks;
      }
    }

    // dynamic FP8 values enter P*V as v * (s_t / s_max) with s_max the unit's largest scale
    // (no overflow in f16), and the unit's sum is multiplied by s_max
    float vmax = vsc;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    const float vratio = vmax > 0.0f ? vsc / vmax : 0.0f;
    if (r == 0) vmax_s[us] = vmax;

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
      // the sum takes each weight as P*V will see it: the f16 product, divided back by the
      // value ratio (numerator and denominator then round alike)
      const __half ph = __float2half_rn(p * vratio * 16384.0f);
      const float pr = __half2float(ph);  // below the f16 normal range the ratio is not kept
      lsum[hh] += pr >= 0x1p-14f ? pr * (1.0f / 16384.0f) / vratio : p;
      pb16[(us * G + hh) * 16 + r] = __half_as_ushort(ph);
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
        // value chunks of this unit: chunk 4*(d%16) + g holds tokens 4g..4g+3 of dimension d
        const uint8_t* vu = vt + upi * 4 * D;
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int dd = lane * DPL + j;
          const int cq = dd & 15, jj = dd >> 4;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            h2_t c01, c23;  // tokens (4g, 4g+1) and (4g+2, 4g+3)
            if (D == 256) {  // two head-dim-128 chunks: dimensions with jj < 8, then jj >= 8
              const uint4 x = *reinterpret_cast<const uint4*>(vu + (cq * 4 + g) * (D / 16));
              c01 = tern2(jj < 8 ? x.x : x.z, jj & 7);
              c23 = tern2(jj < 8 ? x.y : x.w, jj & 7);
            } else if (D == 128) {
              const uint2 x = *reinterpret_cast<const uint2*>(vu + (cq * 4 + g) * (D / 16));
              c01 = tern2(x.x, jj);
              c23 = tern2(x.y, jj);
            } else {
              const uint32_t x = *reinterpret_cast<const uint32_t*>(vu + (cq * 4 + g) * (D / 16));
              c01 = tern2(x, jj);
              c23 = tern2(x, jj + 4);
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              tmp[hh][j] = dot2(pp[hh * 8 + 2 * g], c01, tmp[hh][j]);
              tmp[hh][j] = dot2(pp[hh * 8 + 2 * g + 1], c23, tmp[hh][j]);
            }
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
        vscale = P.fp8_dynamic ? vmax_s[us2] : P.fp8_scale;
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
    const int64_t qh = static_cast<int64_t>(b) * a.hq + kvh * G + hh;  // partial slot
    if (a.n_parts == 1) {
      const float inv = 1.0f / l;
      const int64_t qo = static_cast<int64_t>(a.rows[b]) * a.hq + kvh * G + hh;
#pragma unroll
      for (int j = 0; j < DPL; ++j) a.out[qo * D + lane * DPL + j] = o[hh][j] * inv;
    } else {
      float* part = a.partials + (qh * a.n_parts + split) * (D + 2);
#pragma unroll
      for (int j = 0; j < DPL; ++j) part[lane * DPL + j] = o[hh][j];
      if (lane == 0) {
        part[D] = m[hh];
        part[D + 1] = l;
      }
    }
  }
}

// ------------------------------------------------------------------------
// Matrix-core variant.  Per 16-token unit:
//   S^T[16 tok x 16 heads] = K[16 x D] * Q^T[D x 16]   (D/32 x v_mfma_f32_16x16x32_f16)
//   O^T[D x 16 heads]     += V^T[D x 32] * P[32 x 16]   (per two units, D/16 x 16x16x32)
// Lane l holds token/dimension row l%16 of the A operands and query head l%16
// of the B operands; the score output (lane l: tokens 4(l/16)+r, head l%16) is
// exactly the P operand layout of the second product, so probabilities never
// leave registers.  With g < 16 the query heads repeat over the 16 columns (slots of
// max(g, 4) columns); clean steps give each slot its own unit (see "Column slots" below).
//
// Codes enter the products as u = code + 1 in {0, 1, 2}, as f16 values off + u 2^-14
// (offset form below: one v_and_or_b32 per pair of codes); the constant parts are
// removed once per head: sum_d q_d (u_d - 1) follows from the score product and
// sum_d (off_d + 2^-14) q_d, and sum_t p_t (u_t - 1) from the P*V product and
// sum_t p_t (off_j + 2^-14) per 16-dimension block j.
//
// Head dim 128 scores ternary keys with one fp4 x fp8 product per unit and query term
// (v_mfma_scale_f32_16x16x128_f8f6f4): a 2-bit field u with two zero bits above it is the
// e2m1 value u / 2, so a key code word becomes two fp4 operand words with an AND and a
// shift-AND.  A bfloat16 query, scaled so its largest magnitude lies in [2^6, 2^7), is held
// as the sum of two e4m3 terms, the second stored at 2^4 its value and weighted 2^-4 by the
// product's scale operand: each term takes four significant bits, so the two hold every
// element of at least 2^-12 times the largest exactly (e4m3 steps reach 2^-9) and the smaller
// ones to within 2^-20 times the largest.  Then
// sum_d q_d (u_d - 1) = 2 acc - sum_d q_d, with q the sum of the terms.
//
// Four waves share one (sequence, KV head, split): each walks a quarter of the
// split's units.  A unit's key and value tiles of the head (8 D bytes) are copied
// into the wave's LDS ring by one buffer-to-LDS load, NR units ahead; the page
// addresses come from the block table, one entry per lane for 64 units at a time.
// The four partial states are merged through LDS; global splits by k_merge.
// Split n_splits (when the attended set has fp8 / fp16 pages) handles those pages
// and writes one more partial state.  The grid is (KV head, sequence, split).
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr int kMfmaWaves = 4;
constexpr int kStealWaves = 12;  // a whole CU at 3 waves per SIMD
constexpr int kPiece = 16;       // units per piece a stealing wave takes
// Fourth word of a raw buffer descriptor on gfx9-family parts (32-bit data format; byte
// offsets checked against the record count, reads past it return 0).
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0), the others at their maximum
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0), the others at their maximum
constexpr int wait_vm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }  // vmcnt(n) only

__device__ __forceinline__ uint32_t h2u(h2_t x) { return __builtin_bit_cast(uint32_t, x); }

// 2-bit fields at bit s of each 16-bit half, as f16 u * 2^-14 (bit pattern u << 10).
template <int S>
__device__ __forceinline__ uint32_t ucode2(uint32_t w) {
  if constexpr (S <= 10) return (w << (10 - S)) & 0x0C000C00u;
  else return (w >> (S - 10)) & 0x0C000C00u;
}

template <int NC, int NV>
struct UnitRaw {
  uint32_t k[NC];  // key codes of token l%16, dims of lane group l/16
  uint32_t v[NV];  // value chunk 4(l%16) + l/16: tokens 4(l/16)..+3 of dims 16j + l%16
};

// Offset form of a code pair, one AND-OR per pair for most positions: the 2-bit fields at
// bits (P, P+16) of w become, in each 16-bit half, the f16 value 2^(-4-pe) + u * 2^-14,
// i.e. the field sits in mantissa bits [pe, pe+1] under the exponent 11 - pe.  Fields at
// P = 4, 6, 8 are used in place (pe = P); P = 10, 12, 14 come from w >> 6 and P = 0, 2 from
// w << 4 (pe = 4, 6, 8 and 4, 6), so every value is a normal f16 and the constant part is
// at most 64 times the code step.  The constant parts are removed once per head (keys) or
// once per output block (values).
template <int P>
struct OPos {
  static constexpr int pe = P < 4 ? P + 4 : (P <= 8 ? P : P - 6);
  static constexpr float off = 1.0f / static_cast<float>(1u << (4 + pe));  // 2^(-4-pe)
};
__device__ __forceinline__ float ocode_off(int p) {  // same as OPos<p>::off, for loops
  const int pe = p < 4 ? p + 4 : (p <= 8 ? p : p - 6);
  return 1.0f / static_cast<float>(1u << (4 + pe));
}
// The masks (scalar registers) and exponent words (vector registers) of pe = 4, 6, 8, made
// opaque so that each pair compiles to a single v_and_or_b32 (a VOP3 encoding takes no
// literal constants and at most one scalar operand).
struct OConst {
  uint32_t m[3], e[3];
};
__device__ __forceinline__ OConst oconst() {
  OConst c;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int pe = 4 + 2 * i;
    c.m[i] = 0x00030003u << pe;
    c.e[i] = ((11u - pe) << 10) * 0x00010001u;
    asm volatile("" : "+s"(c.m[i]));
    asm volatile("" : "+v"(c.e[i]));
  }
  return c;
}
template <int P>
__device__ __forceinline__ uint32_t ocode2(uint32_t w, uint32_t wl4, uint32_t wr6, const OConst& c) {
  constexpr int i = (OPos<P>::pe - 4) / 2;
  const uint32_t src = P < 4 ? wl4 : (P <= 8 ? w : wr6);
  return (src & c.m[i]) | c.e[i];
}

// A operands of the score product: pairs (d, d+8) of each 16-dimension code word.
template <int NS, int NC>
__device__ __forceinline__ void ka_ternary(const uint32_t (&k)[NC], h8_t (&ka)[NS], const OConst& o) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t w = k[c], l4 = w << 4, r6 = w >> 6;
    ka[2 * c] = __builtin_bit_cast(h8_t, u4_t{ocode2<0>(w, l4, r6, o), ocode2<2>(w, l4, r6, o),
                                              ocode2<4>(w, l4, r6, o), ocode2<6>(w, l4, r6, o)});
    ka[2 * c + 1] = __builtin_bit_cast(h8_t, u4_t{ocode2<8>(w, l4, r6, o), ocode2<10>(w, l4, r6, o),
                                                  ocode2<12>(w, l4, r6, o), ocode2<14>(w, l4, r6, o)});
  }
}

// Value chunk words with their shifted copies (offset form, head_dim 128).
template <int NV>
struct VWords {
  uint32_t w[NV], l4[NV], r6[NV];
};
template <int NV>
__device__ __forceinline__ VWords<NV> vwords(const uint32_t (&v)[NV]) {
  VWords<NV> r;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    r.w[i] = v[i];
    r.l4[i] = v[i] << 4;
    r.r6[i] = v[i] >> 6;
  }
  return r;
}

// A operand of block j of the value product: tokens (4g, 4g+1), (4g+2, 4g+3) of dim 16j + l%16.
// Head dim 128 (two words, block j at bits 2j of each): offset form, constant OPos<2j>::off.
// Head dim 64 (one word, bits 2j and 8 + 2j): plain form u * 2^-14 (bit pattern u << 10).
// Head dim 256 (four words): blocks j < 8 as head dim 128 in words 0 and 1, blocks j >= 8 the
// same in words 2 and 3 (at bits 2 (j - 8)), constant OPos<2 (j % 8)>::off.
template <int NV, int J>
__device__ __forceinline__ h4_t va_ternary(const VWords<NV>& v, const OConst& o) {
  if constexpr (NV == 4) {
    constexpr int w = 2 * (J / 8), p = 2 * (J % 8);
    return __builtin_bit_cast(h4_t, u2_t{ocode2<p>(v.w[w], v.l4[w], v.r6[w], o),
                                         ocode2<p>(v.w[w + 1], v.l4[w + 1], v.r6[w + 1], o)});
  } else if constexpr (NV == 2) {
    return __builtin_bit_cast(h4_t, u2_t{ocode2<2 * J>(v.w[0], v.l4[0], v.r6[0], o),
                                         ocode2<2 * J>(v.w[NV - 1], v.l4[NV - 1], v.r6[NV - 1], o)});
  } else {
    return __builtin_bit_cast(h4_t, u2_t{ucode2<2 * J>(v.w[0]), ucode2<2 * J + 8>(v.w[0])});
  }
}
template <int NV>
__device__ __forceinline__ float va_off(int j) {
  return NV == 4 ? ocode_off(2 * (j & 7)) : NV == 2 ? ocode_off(2 * j) : 0.0f;
}

template <int NV, int NB, int J = 0>
__device__ __forceinline__ void va_all(const VWords<NV>& v, h4_t (&va)[NB], const OConst& o) {
  if constexpr (J < NB) {
    va[J] = va_ternary<NV, J>(v, o);
    va_all<NV, NB, J + 1>(v, va, o);
  }
}

// Head dim 256: the value product of two units (16x16x32) or of one (16x16x16), one word pair
// (8 blocks) at a time, each operand built just before its product: the shifted copies and the
// operands of all 16 blocks would not fit beside the other state.
template <int H, int J = 8 * H>
__device__ __forceinline__ void pv2_half(const uint32_t (&a)[4], const uint32_t (&b)[4], h8_t pb, f4_t (&oacc)[16],
                                         const OConst& o) {
  if constexpr (J < 8 * H + 8) {
    constexpr int p = 2 * (J % 8), w = 2 * H;
    const uint32_t x0 = ocode2<p>(a[w], a[w] << 4, a[w] >> 6, o), x1 = ocode2<p>(a[w + 1], a[w + 1] << 4, a[w + 1] >> 6, o);
    const uint32_t y0 = ocode2<p>(b[w], b[w] << 4, b[w] >> 6, o), y1 = ocode2<p>(b[w + 1], b[w + 1] << 4, b[w + 1] >> 6, o);
    oacc[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, u4_t{x0, x1, y0, y1}), pb, oacc[J], 0, 0, 0);
    pv2_half<H, J + 1>(a, b, pb, oacc, o);
  }
}
template <int H, int J = 8 * H>
__device__ __forceinline__ void pv1_half(const uint32_t (&a)[4], h4_t pb, f4_t (&oacc)[16], const OConst& o) {
  if constexpr (J < 8 * H + 8) {
    constexpr int p = 2 * (J % 8), w = 2 * H;
    const uint32_t x0 = ocode2<p>(a[w], a[w] << 4, a[w] >> 6, o), x1 = ocode2<p>(a[w + 1], a[w + 1] << 4, a[w + 1] >> 6, o);
    oacc[J] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, u2_t{x0, x1}), pb, oacc[J], 0, 0, 0);
    pv1_half<H, J + 1>(a, pb, oacc, o);
  }
}

// STEAL: one 12-wave block per (sequence, KV head, split) whose waves take pieces of the
// block's units from a shared counter (launches of all-ternary pages with a block per CU).
// LL: the fp8 / fp16 blocks also read lossless pages (an instance of its own, launched only when
// a launch attends lossless units: their decode needs registers the other instances keep).
// Fused split merge (matrix-core launches with several parts and no lossless launch): every
// block of a (sequence, KV head) has stored its part with device-coherent stores; once they have
// completed, one thread adds 1 to the pair's part counter (a device-scope atomic).  The block that
// brings it to n_parts is the last, so every other part is stored: it resets the counter for the
// next launch and combines the parts as k_merge does, in the same order with the same arithmetic
// (one wave per query head: lane s holds part s's (max, sum) for the butterflies, then every lane
// sums its dimensions over the parts in part order), so outputs equal the two-launch path bit for
// bit.  No block waits for another: the ones that finish earlier just leave.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_parts_last_block(const DecodeArgs& a, int b, int kvh, int64_t qh0, int64_t qo0) {
  __shared__ int last_s;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's part stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = a.part_count + static_cast<int64_t>(b) * a.P.hkv + kvh;
    const uint32_t done = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    last_s = done == static_cast<uint32_t>(a.n_parts);
    if (done == static_cast<uint32_t>(a.n_parts)) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last_s) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ns = a.n_parts;  // <= 64
  auto ld = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  for (int hh = wave; hh < G; hh += NW) {
    const float* base = a.partials + (qh0 + hh) * ns * (D + 2);
    const float ms = lane < ns ? ld(base + lane * (D + 2) + D) : -INFINITY;
    const float ls = lane < ns ? ld(base + lane * (D + 2) + D + 1) : 0.0f;
    float M = ms;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float wgt = ls > 0.0f ? exp2f(ms - M) : 0.0f;
    float den = wgt * ls;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
    for (int dd = lane; dd < D; dd += 64) {
      float num = 0.0f;
      for (int s0 = 0; s0 < ns; s0 += 8) {
        float o8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o8[k] = s0 + k < ns ? ld(base + (s0 + k) * (D + 2) + dd) : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float w = __shfl(wgt, (s0 + k) & 63, 64);
          num = s0 + k < ns ? fmaf(w, o8[k], num) : num;
        }
      }
      a.out[(qo0 + hh) * D + dd] = num / den;
    }
  }
}

template <int D, int G, int QDT, int PF, bool DYN, bool STEAL, bool LL = false>
__global__ __launch_bounds__(64 * (STEAL ? kStealWaves : kMfmaWaves))
__attribute__((amdgpu_waves_per_eu(D == 256 ? 2 : 3, 8)))  // head dim 256: twice the state per lane
void k_decode_mfma(DecodeArgs a) {
  constexpr int NW = STEAL ? kStealWaves : kMfmaWaves;  // waves per block
  constexpr int NC = D / 64;   // 32-bit key code words per lane per unit
  constexpr int NV = D / 64;   // 32-bit value chunk words per lane per unit
  constexpr int NS = D / 32;   // 16x16x32 steps per unit of the score product
  constexpr int NB = D / 16;   // 16-dimension output blocks
  constexpr int CH = 64;       // units per metadata chunk (one per lane)
  constexpr int UG = 2;        // units sharing one online-softmax update and one P*V product
  // ternary scores on the fp4 x fp8 product: head dims 128 and 256, bfloat16 queries (two e4m3
  // terms hold one exactly; f16 queries would need a third term's registers and keep the f16
  // product)
  constexpr bool F4 = (D == 128 || D == 256) && QDT == 1;
  constexpr int NQ = 2;       // e4m3 terms of the query
  constexpr int NH = D >= 128 ? D / 128 : 1;  // fp4 products per term (128 dimensions each)
  // ternary logit = ks (kmul acc - qoff): kmul 2 for the fp4 product, 2^14 for the f16 one
  using ProdF4 = std::integral_constant<bool, F4>;  // long ranges: the fp4 product where built
  using ProdF16 = std::false_type;                  // short ranges: the f16 product, whose
                                                    // query set-up is shorter (latency-bound)
  static_assert(G <= 16, "one query head per lane column");
  static_assert(D != 256 || (!STEAL && !LL), "head dim 256: no stealing blocks and no lossless pages");
  // Column slots: the query heads are repeated over the 16 columns of the score product, in
  // NSL slots of W columns.  A clean step puts one unit's scores in each slot, so its softmax
  // steps cover NSL units at once; the other paths keep their sums in slot 0 only.
  constexpr int W = G < 4 ? 4 : G;       // columns per slot
  constexpr int NSL = 16 / W;            // 4 (G <= 4), 2 (G = 8) or 1 (G = 16)
  constexpr int SU = NSL == 4 ? 4 : 2;   // units per clean step
  // clean steps may hold partly attended units (masked) where the registers allow it; at head
  // dim 128 with g <= 4 the masking would spill, and such steps take the general path
  constexpr bool PCLEAN = D == 64 || (D == 128 && G == 8);
  static_assert(CH % PF == 0 && PF % UG == 0 && PF % SU == 0, "chunks hold whole prefetch rounds and groups");
  __shared__ float lds_m[NW][G], lds_l[NW][G];
  __shared__ int lds_next;  // stealing blocks: the next piece to hand out
  if constexpr (STEAL) {
    if (threadIdx.x == 0) lds_next = 0;
    __syncthreads();
  }
  // LDS ring: NR slots per wave, each one unit's key tile then value tile (8 D bytes), filled
  // by buffer-to-LDS loads.  One array per slot, so the compiler's wait counting can tell
  // the slots apart and waits only for the load of the slot it reads.
  constexpr int UB = 8 * D;     // bytes of one unit's tiles of one head
  // ring row: one 16-byte piece per lane (head dim 64 fills half); head dim 256: two pieces per
  // lane, the key tile and then the value tile, by two copies
  constexpr int NCP = D == 256 ? 2 : 1;  // copies per unit
  constexpr int RB = 64 * 16 * NCP;
  constexpr int NR = PF;
  static_assert(NR == 8 || NR == 4, "ring of 4 or 8 slots");
  __shared__ __attribute__((aligned(16))) uint8_t ring0[NW][RB], ring1[NW][RB],
      ring2[NW][RB], ring3[NW][RB], ring4[NR == 8 ? NW : 1][RB],
      ring5[NR == 8 ? NW : 1][RB], ring6[NR == 8 ? NW : 1][RB], ring7[NR == 8 ? NW : 1][RB];

  // wave-uniform indices live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63, grp = lane >> 4, c16 = lane & 15;
  const int cslot = c16 / W;  // this lane's column slot
  // grid (KV head, sequence, split): blocks dispatched together read the heads' slices of the
  // same pages.  With a dispatch order (launches of sequences of different lengths) the grid is
  // (KV head, order index) and entry y of the order names the sequence and the part.
  const uint32_t ord = a.n_order > 0 ? static_cast<uint32_t>(a.order[blockIdx.y]) : 0u;
  const int kvh = blockIdx.x;
  const int b = a.n_order > 0 ? static_cast<int>(ord & 0xFFu) : static_cast<int>(blockIdx.y);
  const int split = (a.n_order > 0 ? static_cast<int>(ord >> 8) : static_cast<int>(blockIdx.z)) + a.part_base;
  const int slot = a.slots[b], L = a.lens[b];
  const PoolsView& P = a.P;
  // The kernel arguments the set-up reads, loaded in one batch: left to the compiler, the
  // scalar loads go out in rounds, each waiting for the one before (a launch that moves a
  // few tens of KB pays for every round).
  {
    const void* ptrs[5] = {P.block_table, P.gamma, P.pool[0], P.dummy_page, a.q};
    asm volatile("" ::"s"(slot), "s"(L), "s"(a.sink_tokens), "s"(a.window), "s"(a.n_splits),
                 "s"(a.units_per_split), "s"(a.rows[b]), "s"(a.hq), "s"(a.layer), "s"(P.max_pages),
                 "s"(P.bs_shift), "s"(P.bs), "s"(P.hkv), "s"(P.cap[0]), "s"(P.page_bytes[0]),
                 "s"(P.tile_bytes[0]), "s"(ptrs[0]), "s"(ptrs[1]), "s"(ptrs[2]), "s"(ptrs[3]), "s"(ptrs[4]));
  }
  const Units R = attended(L, a.sink_tokens, a.window);
  const int n_a = R.a_end;
  const int U = R.a_end + (R.b_end - R.b_begin);
  // one of the extra blocks: fp8 / fp16 pages, or (LL) the lossless pages
  const bool mixed_part = LL || split >= a.n_splits;
  const int s_begin = min(split * a.units_per_split, U);  // empty past the sequence's units
  const int s_end = min(s_begin + a.units_per_split, U);
  // a wave's share of the split (stealing waves: the whole split, taken piece by piece)
  const int u_begin = STEAL ? s_begin : s_begin + ((s_end - s_begin) * wave) / NW;
  const int u_end = STEAL ? s_end : s_begin + ((s_end - s_begin) * (wave + 1)) / NW;
  const int u_last = max(u_end - 1, 0);
  const int dbase = grp * (D / 4);  // first head dimension of this lane group's key slice
  const int64_t layer = a.layer;
  const int32_t* bt = P.block_table + static_cast<int64_t>(slot) * P.max_pages;
  const int tile0 = static_cast<int>(P.tile_bytes[0]);
  const int page_bytes0 = static_cast<int>(P.page_bytes[0]);
  const int64_t qh0 = static_cast<int64_t>(b) * a.hq + kvh * G;          // partial slots
  const int64_t qo0 = static_cast<int64_t>(a.rows[b]) * a.hq + kvh * G;  // query / output rows
  // Lane (c16, grp) needs bytes [32 c16 + 8 grp, +8) of the unit's key tile (row c16, dims
  // 32 grp ..) and the same bytes of its value tile (chunk 4 c16 + grp); head dim 64: 4 bytes
  // at 16 c16 + 4 grp.  The copy moves 16-byte pieces, lane i to ring offset 16 i.  Head dim
  // 128 places piece (row r, half h) at 16 (16 h + r): then the 8-byte reads of lanes
  // 0..31 (and of 32..63) cover 256 contiguous bytes, free of bank conflicts.
  // Head dim 256: 16 bytes at 64 c16 + 16 grp of each tile, whose copies place every piece
  // in order.
  // lane_k = this lane's read offset in the key half of a ring row (+ UB / 2: value half).
  const uint32_t lane_k = D == 128 ? 256 * (grp >> 1) + 16 * c16 + 8 * (grp & 1) : c16 * (D / 4) + grp * (D / 16);
  // piece fetched by this lane: lanes [0, D/4) the key tile, [D/4, D/2) the value tile; with
  // head dim 64 lanes [32, 64) repeat lanes [0, 32) (every lane issues the copy: no branch)
  const int hkv_tile = P.hkv * tile0;
  const int dl = lane % (D / 2), dp = dl % (D / 4);
  const uint32_t piece = D == 128 ? 32 * (dp % 16) + 16 * (dp / 16) : 16 * dp;
  const uint32_t dma_off = dl < D / 4 ? piece : hkv_tile + piece;
  auto ring_row = [&](auto I) -> uint8_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return ring0[wave];
    else if constexpr (i == 1) return ring1[wave];
    else if constexpr (i == 2) return ring2[wave];
    else if constexpr (i == 3) return ring3[wave];
    else if constexpr (i == 4) return ring4[wave];
    else if constexpr (i == 5) return ring5[wave];
    else if constexpr (i == 6) return ring6[wave];
    else return ring7[wave];
  };

  auto unit_of = [&](int lu) { return lu < n_a ? lu : R.b_begin + (lu - n_a); };
  auto attended_tok = [&](int t) { return R.single ? t < L : (t < R.sinks || (t >= R.w0 && t < L)); };
  // every token of logical units [lu, lu + n) is attended
  auto fully_attended = [&](int lu, int n) {
    if (lu + n > u_end) return false;
    const int u0 = unit_of(lu), u1 = unit_of(lu + n - 1);
    if (u1 - u0 != n - 1) return false;
    if (R.single) return (u1 * 16 + 16) <= L;
    return (u1 * 16 + 16 <= R.sinks) || (u0 * 16 >= R.w0 && u1 * 16 + 16 <= L);
  };
  // Per-chunk unit metadata, one unit per lane (lanes past the end repeat the last unit):
  // block-table entry, the K and V gamma of ternary pages, and the address of the page the
  // codes are read from (the zeroed dummy page for other formats).  Page addresses are
  // computed here, per lane, once per 64 units; a unit takes them with readlane.  The copies
  // need only the addresses; the gamma values are first waited for by chunk_flags.
  struct Chunk {
    int32_t ent;
    float gk, gv;
    uint32_t plo, phi;
    uint64_t cmask;  // bit i: unit c0 + i is ternary with the gamma pair below
    uint64_t fmask;  // bit i: every token of unit c0 + i is attended
    float gk0, gv0;  // the gamma pair of the chunk's first ternary unit (uniform)
  };
  auto lane_f = [](float x, int k) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), k));
  };
  auto load_chunk = [&](int c0) -> Chunk {
    // (a piece needs kPiece lanes; the others repeat its first unit: no extra memory traffic)
    const int lu = min(c0 + (STEAL && lane >= kPiece ? 0 : lane), u_last);
    Chunk c;
    c.ent = bt[(unit_of(lu) * 16) >> P.bs_shift];
    const bool tern = (static_cast<uint32_t>(c.ent) >> 30) == VK_FMT_TERNARY2;
    const int64_t gi = layer * P.cap[0] + (tern ? (c.ent & 0x3FFFFFFF) : 0);
    const float2 gg = *reinterpret_cast<const float2*>(P.gamma + gi * 2);
    c.gk = gg.x;
    c.gv = gg.y;
    const uint64_t pg = tern ? reinterpret_cast<uint64_t>(P.pool[0] + gi * P.page_bytes[0])
                             : reinterpret_cast<uint64_t>(P.dummy_page);
    c.plo = static_cast<uint32_t>(pg);
    c.phi = static_cast<uint32_t>(pg >> 32);
    return c;
  };
  auto chunk_flags = [&](Chunk& c, int c0) {
    const int lu = min(c0 + lane, u_last);
    const bool tern = (static_cast<uint32_t>(c.ent) >> 30) == VK_FMT_TERNARY2;
    const uint64_t tm = __ballot(tern);
    const int l0 = tm ? static_cast<int>(__builtin_ctzll(tm)) : 0;
    c.gk0 = lane_f(c.gk, l0);
    c.gv0 = lane_f(c.gv, l0);
    const int u = unit_of(lu);
    const bool full = R.single ? u * 16 + 16 <= L : (u * 16 + 16 <= R.sinks || (u * 16 >= R.w0 && u * 16 + 16 <= L));
    c.cmask = __ballot(tern && c.gk == c.gk0 && c.gv == c.gv0);
    c.fmask = __ballot(full);
  };

  // Query head c16 mod G as the B operand of the score product: f16 pairs (d, d+8) of each
  // 16-dimension block.  For ternary codes in offset form the logit
  // is ks (2^14 acc - qoff), qoff = 2^14 sum_d off(d) q_d + sum_d q_d.
  h8_t qb[NS];
  float qsum = 0.0f, qoff = 0.0f;
  float qsl = a.scale_log2;  // softmax scale * log2(e) * 2^-sh for the query scaled by 2^sh
  const uint16_t* qhead = a.q + (qo0 + (c16 & (G - 1))) * D;
  auto make_qb = [&]() {
    // (the memory clobber keeps the query's loads, and the wait for them, after the page
    // copies issued before this call: the compiler would otherwise hoist them to the top)
    asm volatile("" ::: "memory");
    const uint16_t* qrow = qhead + dbase;
    uint32_t w[NS][4];
    float sum = 0.0f;
    uint4 x[NC][2];
    float qmax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      x[c][0] = reinterpret_cast<const uint4*>(qrow + 16 * c)[0];  // dims 16c .. 16c+7
      x[c][1] = reinterpret_cast<const uint4*>(qrow + 16 * c)[1];  // dims 16c+8 .. 16c+15
      const uint32_t all[8] = {x[c][0].x, x[c][0].y, x[c][0].z, x[c][0].w, x[c][1].x, x[c][1].y, x[c][1].z, x[c][1].w};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        qmax = fmaxf(qmax, fabsf(q_value<QDT>(static_cast<uint16_t>((all[i >> 1] >> (16 * (i & 1))) & 0xFFFFu))));
    }
    // one power of two for the whole group (every lane holds one of its query heads)
    const int qsh = __builtin_amdgcn_readfirstlane(q_shift(wave_max(qmax)));
    const float qmul = pow2i(qsh);
    qsl = a.scale_log2 * pow2i(-qsh);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t lo[4] = {x[c][0].x, x[c][0].y, x[c][0].z, x[c][0].w}, hi[4] = {x[c][1].x, x[c][1].y, x[c][1].z, x[c][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t e0 = (lo[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const uint32_t e1 = (hi[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const uint32_t pr = f16_bits(q_value<QDT>(static_cast<uint16_t>(e0)) * qmul) |
                            (f16_bits(q_value<QDT>(static_cast<uint16_t>(e1)) * qmul) << 16);
        w[2 * c + (i >> 2)][i & 3] = pr;
        const h2_t hp = as_h2(pr);
        sum += static_cast<float>(hp[0]) + static_cast<float>(hp[1]);
      }
    }
    float koff = 0.0f;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      qb[st] = __builtin_bit_cast(h8_t, u4_t{w[st][0], w[st][1], w[st][2], w[st][3]});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2_t hp = as_h2(w[st][i]);
        koff += ocode_off(2 * (4 * (st & 1) + i)) * (static_cast<float>(hp[0]) + static_cast<float>(hp[1]));
      }
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    koff += __shfl_xor(koff, 16, 64);
    koff += __shfl_xor(koff, 32, 64);
    qsum = sum;
    qoff = 16384.0f * koff + sum;  // logit = ks (2^14 acc - qoff) for offset-form codes
  };
  // The query as NQ e4m3 terms, the B operands of the fp4 x fp8 score product (ternary
  // blocks).  The product pairs nibble n of word v of an A lane of group g (product dimension
  // 32 g + 16 (v / 2) + 2 n + v % 2, from tern_score) with byte 16 (g / 2) + 8 (v % 2) + n of a
  // B lane of group 2 (g % 2) + v / 2; so B lane group g holds, in bytes jb and 16 + jb
  // (jb < 16), product dimensions 16 g + e(jb) and 64 + 16 g + e(jb), e(jb) = 2 (jb % 8) +
  // jb / 8.  Head dim 128: product dimension = head dimension.  Head dim 256 takes two
  // products; product h pairs each A lane's words 2h, 2h + 1, so its dimension p is head
  // dimension 64 (p / 32) + 32 h + p % 32, and the 16 dimensions 64 c + 16 g + [0, 16) of B
  // lane group g are head dimensions 128 c + 64 (g / 2) + 32 h + 16 (g % 2) + [0, 16).
  v8i_t qf[NH][NQ];
  auto make_qf = [&]() {
    asm volatile("" ::: "memory");  // (as in make_qb)
    uint32_t x[NH][2][8];
    float qmax = 0.0f;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint16_t* qrow =
            qhead + (NH == 1 ? 64 * c + 16 * grp : 128 * c + 64 * (grp >> 1) + 32 * h + 16 * (grp & 1));
        const uint4 lo = reinterpret_cast<const uint4*>(qrow)[0];  // dims +0 .. +7
        const uint4 hi = reinterpret_cast<const uint4*>(qrow)[1];  // dims +8 .. +15
        const uint32_t all[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[h][c][i] = all[i];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          qmax = fmaxf(qmax, fabsf(q_value<QDT>(static_cast<uint16_t>((all[i >> 1] >> (16 * (i & 1))) & 0xFFFFu))));
      }
    const int qsh = __builtin_amdgcn_readfirstlane(q_shift<6>(wave_max(qmax)));
    const float qmul = pow2i(qsh);
    qsl = a.scale_log2 * pow2i(-qsh);
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      uint32_t w[NQ][8];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {  // operand word t8: bytes (slots) 4 t8 .. 4 t8 + 3
        float r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = 4 * t8 + k, c = j >> 4, i = 2 * (j & 7) + ((j >> 3) & 1);  // product dimension 64 c + 16 grp + i
          r[k] = q_value<QDT>(static_cast<uint16_t>((x[h][c][i >> 1] >> (16 * (i & 1))) & 0xFFFFu)) * qmul;
        }
#pragma unroll
        for (int t = 0; t < NQ; ++t) {  // term t, stored at 2^(4 t): four bytes by two packed converts
          const float up = pow2i(4 * t), down = pow2i(-4 * t);
          int e = __builtin_amdgcn_cvt_pk_fp8_f32(r[0] * up, r[1] * up, 0, false);
          e = __builtin_amdgcn_cvt_pk_fp8_f32(r[2] * up, r[3] * up, e, true);
          const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(e, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(e, true);
          const float back[4] = {lo[0] * down, lo[1] * down, hi[0] * down, hi[1] * down};  // the term's values
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            r[k] -= back[k];
            sum += back[k];
          }
          w[t][t8] = static_cast<uint32_t>(e);
        }
      }
#pragma unroll
      for (int t = 0; t < NQ; ++t)
        qf[h][t] = v8i_t{static_cast<int>(w[t][0]), static_cast<int>(w[t][1]), static_cast<int>(w[t][2]),
                         static_cast<int>(w[t][3]), static_cast<int>(w[t][4]), static_cast<int>(w[t][5]),
                         static_cast<int>(w[t][6]), static_cast<int>(w[t][7])};
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    qsum = sum;
    qoff = sum;  // logit = ks (2 acc - qoff)
  };
  // query operands of the ternary blocks
  auto make_qt = [&]() {
    if constexpr (F4) make_qf();
    else make_qb();
  };

  f4_t oacc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) oacc[j] = f4_t{0.f, 0.f, 0.f, 0.f};
  // p' = f16(2^14 p).  oacc = sum p' u 2^-14 (ternary) or sum p' v 2^-14 (other formats) and
  // tsum = sum p' over ternary tokens, both in units of vcur; lsum = sum p' over all tokens.
  float m = -INFINITY, lsum = 0.0f, tsum = 0.0f, vcur = 0.0f;
  const h2_t ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  const OConst oc = oconst();
  // raw score accumulator of one ternary unit (logit = ks (kmul acc - qoff)); PRD: ProdF4 or
  // ProdF16, the product the wave's query operands were built for (make_qt or make_qb)
  auto tern_score = [&](const uint32_t (&k)[NC], auto PRD) -> f4_t {
    f4_t s4 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (decltype(PRD)::value) {
      constexpr uint32_t M = 0x33333333u;  // the even 2-bit fields, one per nibble
#pragma unroll
      for (int h = 0; h < NH; ++h) {  // product h: words 2h, 2h + 1 of the lane's key slice
        const uint32_t k0 = k[2 * h], k1 = k[2 * h + 1];
        const v8i_t ak = {static_cast<int>(k0 & M), static_cast<int>((k0 >> 2) & M),
                          static_cast<int>(k1 & M), static_cast<int>((k1 >> 2) & M), 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < NQ; ++t)
          s4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ak, qf[h][t], s4, 4, 0, 0, 127, 0, 127 - 4 * t);
      }
    } else {
      h8_t ka[NS];
      ka_ternary<NS, NC>(k, ka, oc);
#pragma unroll
      for (int st = 0; st < NS; ++st) s4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[st], qb[st], s4, 0, 0, 0);
    }
    return s4;
  };

  // Starts the copy of logical unit lu's key and value tiles of this head into a ring row.
  // Always issued (a fixed number of loads per unit keeps the waits exact): other formats
  // read the zeroed dummy page, units past the end re-read the last unit (masked).
  auto dma_unit = [&](int lu, const Chunk& cc, const Chunk& cn, int c0, uint8_t* row) {
    const int lc = min(lu, u_last);
    const int k = lc - c0;
    const bool in_cur = k < CH;
    const uint32_t lo = __builtin_amdgcn_readlane(in_cur ? cc.plo : cn.plo, in_cur ? k : k - CH);
    const uint32_t hi = __builtin_amdgcn_readlane(in_cur ? cc.phi : cn.phi, in_cur ? k : k - CH);
    const uint8_t* pg = reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
    const int upi = ((unit_of(lc) * 16) & (P.bs - 1)) >> 4;  // the dummy page takes any unit offset
    // A copy for a unit past the wave's range is still issued (the ring's waits count on a
    // fixed number of copies), with an empty record range: out of range, it reads no memory.
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pg), 0, lu < u_end ? page_bytes0 : 0, kBufferWord3);
    const int soff = kvh * tile0 + upi * 4 * D;  // unit offset within the key (and value) tile
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)row, 16, dma_off, soff, 0, 0);
    if constexpr (NCP == 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(row + UB / 2), 16,
                                               dma_off + hkv_tile, soff, 0, 0);
  };
  auto read_unit = [&](const uint8_t* row, UnitRaw<NC, NV>& r) {
    if constexpr (NC == 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(row + lane_k);
      const uint4 y = *reinterpret_cast<const uint4*>(row + UB / 2 + lane_k);
      r.k[0] = x.x; r.k[1] = x.y; r.k[2] = x.z; r.k[3] = x.w;
      r.v[0] = y.x; r.v[1] = y.y; r.v[2] = y.z; r.v[3] = y.w;
    } else if (NC == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(row + lane_k);
      const uint2 y = *reinterpret_cast<const uint2*>(row + UB / 2 + lane_k);
      r.k[0] = x.x;
      r.k[NC - 1] = x.y;
      r.v[0] = y.x;
      r.v[NV - 1] = y.y;
    } else {
      r.k[0] = *reinterpret_cast<const uint32_t*>(row + lane_k);
      r.v[0] = *reinterpret_cast<const uint32_t*>(row + UB / 2 + lane_k);
    }
  };

  // keep oacc and tsum in units of vs (uniform; rare: gamma_V changes between append calls)
  auto set_value_scale = [&](float vs) {
    if (vs != vcur) {
      const float ratio = vcur / vs;
#pragma unroll
      for (int j = 0; j < NB; ++j) oacc[j] *= ratio;
      tsum *= ratio;
      vcur = vs;
    }
  };

  // max over the slots of each head (lanes c16, c16 ^ W, ...; the rows are already merged)
  auto max_slots = [&](float x) {
#pragma unroll
    for (int o = W; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
  };
  // probabilities of the general paths count in slot 0 only (the other slots repeat its heads)
  auto slot0 = [&](uint32_t p) { return NSL == 1 || cslot == 0 ? p : 0u; };

  // One clean step: SU units that are ternary with the chunk's reference gamma pair gk0, gv0,
  // with the steps of process_group below and no per-unit checks.  A partial step (a unit
  // with tokens outside the attended set, or units past the end of the range, whose slots
  // hold copies of nothing) masks those tokens' scores.  With NSL > 1
  // the score tiles of NSL units merge into one, unit i in slot i, so the softmax runs once
  // for them; P*V then gives each unit's probabilities only to its own slot's columns (a
  // block-diagonal B operand) and the slots are summed when the wave ends.
  auto process_clean = [&](const Chunk& cc, const UnitRaw<NC, NV> (&r)[SU], bool partial, int lu0, int lu_end,
                           auto PRD) {
    constexpr float kmul = decltype(PRD)::value ? 2.0f : 16384.0f;
    constexpr int UT = NSL == 1 ? 1 : NSL;  // units per score tile
    constexpr int NT = SU / UT;             // score tiles
    const float ks = cc.gk0 * qsl;
    const float a0 = ks * kmul, a1 = -qoff * ks;  // logit (log2 units) = a0 * acc + a1
    float sc[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f4_t tile;
#pragma unroll
      for (int i = 0; i < UT; ++i) {
        const f4_t s4 = tern_score(r[t * UT + i].k, PRD);
        if (i == 0) {
          tile = s4;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) tile[q] = cslot == i ? s4[q] : tile[q];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sc[t][q] = fmaf(tile[q], a0, a1);
    }
    if (PCLEAN && partial) {  // this lane's rows of tile t are tokens 4 grp .. 4 grp + 3 of one unit
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int lu = lu0 + t * UT + (UT == 1 ? 0 : cslot);
        const int t0 = unit_of(lu) * 16 + 4 * grp;
#pragma unroll
        for (int q = 0; q < 4; ++q) sc[t][q] = lu < lu_end && attended_tok(t0 + q) ? sc[t][q] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t) mx = fmaxf(mx, fmaxf(fmaxf(sc[t][0], sc[t][1]), fmaxf(sc[t][2], sc[t][3])));
    if (__ballot(mx > m + 1.0f) != 0) {  // lazy running max, as in process_group
      mx = max_slots(max_rows(mx));
      const float mn = fmaxf(m, mx);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int j = 0; j < NB; ++j) oacc[j] *= corr;
      lsum *= corr;
      tsum *= corr;
      m = mn;
    }
    const float ms = m - 14.0f;
    uint32_t pk[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const h2_t p2 = {static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[t][2 * h] - ms)),
                         static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[t][2 * h + 1] - ms))};
        pk[t][h] = h2u(p2);
        lsum = __builtin_amdgcn_fdot2(p2, ones, lsum, false);
      }
    if (cc.gv0 == 0.0f) return;  // every value of these pages is 0
    set_value_scale(cc.gv0);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) tsum = __builtin_amdgcn_fdot2(as_h2(pk[t][h]), ones, tsum, false);
    // P*V, two units per 16x16x32 product: unit u's probabilities sit in tile u / UT, and
    // with slots only the lanes of slot u % UT pass them on
    auto pvals = [&](int u, int h) {
      const uint32_t x = pk[u / UT][h];
      return UT == 1 || cslot == u % UT ? x : 0u;
    };
#pragma unroll
    for (int s2 = 0; s2 < SU / 2; ++s2) {
      const h8_t pb = __builtin_bit_cast(
          h8_t, u4_t{pvals(2 * s2, 0), pvals(2 * s2, 1), pvals(2 * s2 + 1, 0), pvals(2 * s2 + 1, 1)});
      if constexpr (NV == 4) {
        pv2_half<0>(r[2 * s2].v, r[2 * s2 + 1].v, pb, oacc, oc);
        pv2_half<1>(r[2 * s2].v, r[2 * s2 + 1].v, pb, oacc, oc);
        continue;
      }
      h4_t v0[NB], v1[NB];
      va_all<NV, NB>(vwords<NV>(r[2 * s2].v), v0, oc);
      va_all<NV, NB>(vwords<NV>(r[2 * s2 + 1].v), v1, oc);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const u2_t x0 = __builtin_bit_cast(u2_t, v0[j]), x1 = __builtin_bit_cast(u2_t, v1[j]);
        const h8_t av = __builtin_bit_cast(h8_t, u4_t{x0[0], x0[1], x1[0], x1[1]});
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb, oacc[j], 0, 0, 0);
      }
    }
  };

  // Two consecutive units: scores, one online-softmax update, then P*V (one 16x16x32
  // product per 16-dimension block when both units are ternary with one gamma_V).
  auto process_group = [&](int lu0, const Chunk& cc, int c0, const UnitRaw<NC, NV>& r0,
                           const UnitRaw<NC, NV>& r1, auto PRD) {
    constexpr float kmul = decltype(PRD)::value ? 2.0f : 16384.0f;
    if (lu0 >= u_end) return;
    const bool have1 = lu0 + 1 < u_end;
    const int k0 = lu0 - c0;
    const int32_t e0 = __builtin_amdgcn_readlane(cc.ent, k0);
    const int32_t e1 = have1 ? __builtin_amdgcn_readlane(cc.ent, k0 + 1) : e0;
    // fp8 / fp16 units are left to the mixed-format kernel: here they count as masked
    bool tern[UG];
    tern[0] = (static_cast<uint32_t>(e0) >> 30) == VK_FMT_TERNARY2;
    tern[1] = have1 && (static_cast<uint32_t>(e1) >> 30) == VK_FMT_TERNARY2;
    if (!tern[0] && !tern[1]) return;
    const bool full = tern[0] && tern[1] && fully_attended(lu0, UG);
    float sc[UG][4], vs[UG];
#pragma unroll
    for (int g = 0; g < UG; ++g) {
      const int lu = lu0 + g;
      vs[g] = 0.0f;
      if (!tern[g]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[g][r] = -INFINITY;
        continue;
      }
      const UnitRaw<NC, NV>& raw = g == 0 ? r0 : r1;
      const float ks = lane_f(cc.gk, k0 + g) * qsl;
      vs[g] = lane_f(cc.gv, k0 + g);
      const f4_t s4 = tern_score(raw.k, PRD);
      const float a0 = ks * kmul, a1 = -qoff * ks;  // logit (log2 units) = a0 * acc + a1
      if (full) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[g][r] = fmaf(s4[r], a0, a1);
      } else {
        const int u = unit_of(lu);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = u * 16 + 4 * grp + r;
          const bool att = R.single ? t < L : (t < R.sinks || (t >= R.w0 && t < L));
          sc[g][r] = att ? fmaf(s4[r], a0, a1) : -INFINITY;
        }
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    // Lazy running max: m only has to stay within 1 (log2 units) of every score seen, so that
    // p' = 2^(s - m + 14) <= 2^15 fits f16.  The max across the lane rows and the rescale run
    // only when a score exceeds m + 1 (a uniform branch; m = -inf takes it for any score).
    if (__ballot(mx > m + 1.0f) != 0) {
      mx = max_rows(mx);
      const float mn = fmaxf(m, mx);
      const float corr = __builtin_amdgcn_exp2f(m - mn);  // m = -inf gives 0
#pragma unroll
      for (int j = 0; j < NB; ++j) oacc[j] *= corr;
      lsum *= corr;
      tsum *= corr;
      m = mn;
    }
    // nothing attended yet (this group included): it adds nothing, and m - 14 is not finite
    if (__builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, m)) == __builtin_bit_cast(int, -INFINITY)) return;
    const float ms = m - 14.0f;  // p' = 2^(s - m + 14), at most 2^15
    uint32_t pk[UG][2];
#pragma unroll
    for (int g = 0; g < UG; ++g) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const h2_t p2 = {static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[g][2 * h] - ms)),
                         static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[g][2 * h + 1] - ms))};
        pk[g][h] = slot0(h2u(p2));
        lsum = __builtin_amdgcn_fdot2(as_h2(pk[g][h]), ones, lsum, false);
      }
    }
    if (tern[0] && tern[1] && vs[0] == vs[1]) {
      if (vs[0] == 0.0f) return;  // every value of these pages is 0
      set_value_scale(vs[0]);
#pragma unroll
      for (int g = 0; g < UG; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) tsum = __builtin_amdgcn_fdot2(as_h2(pk[g][h]), ones, tsum, false);
      const h8_t pb = __builtin_bit_cast(h8_t, u4_t{pk[0][0], pk[0][1], pk[1][0], pk[1][1]});
      if constexpr (NV == 4) {
        pv2_half<0>(r0.v, r1.v, pb, oacc, oc);
        pv2_half<1>(r0.v, r1.v, pb, oacc, oc);
        return;
      }
      h4_t v0[NB], v1[NB];
      va_all<NV, NB>(vwords<NV>(r0.v), v0, oc);
      va_all<NV, NB>(vwords<NV>(r1.v), v1, oc);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const u2_t x0 = __builtin_bit_cast(u2_t, v0[j]), x1 = __builtin_bit_cast(u2_t, v1[j]);
        const h8_t av = __builtin_bit_cast(h8_t, u4_t{x0[0], x0[1], x1[0], x1[1]});
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb, oacc[j], 0, 0, 0);
      }
      return;
    }
    // one ternary unit (the other masked or non-ternary), or two gamma values: one at a time
#pragma unroll
    for (int g = 0; g < UG; ++g) {
      if (!tern[g] || vs[g] == 0.0f) continue;
      set_value_scale(vs[g]);
      const h4_t pb = __builtin_bit_cast(h4_t, u2_t{pk[g][0], pk[g][1]});
      tsum = __builtin_amdgcn_fdot2(as_h2(pk[g][0]), ones, tsum, false);
      tsum = __builtin_amdgcn_fdot2(as_h2(pk[g][1]), ones, tsum, false);
      if constexpr (NV == 4) {
        pv1_half<0>(g == 0 ? r0.v : r1.v, pb, oacc, oc);
        pv1_half<1>(g == 0 ? r0.v : r1.v, pb, oacc, oc);
        continue;
      }
      h4_t vt[NB];
      va_all<NV, NB>(vwords<NV>(g == 0 ? r0.v : r1.v), vt, oc);
#pragma unroll
      for (int j = 0; j < NB; ++j) oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(vt[j], pb, oacc[j], 0, 0, 0);
    }
  };

  // Raw words of one fp8 / fp16 unit as loaded, before any conversion, so that a wave can have
  // the next unit's loads in flight while it computes one (fp8: k[0, NC) and v[j].x).
  struct OtherRaw {
    uint4 k[2 * NC];
    uint2 v[NB];
    float4 ks4, vs4;  // dynamic FP8: the token scales of this lane's score and value rows
  };
  auto load_other = [&](int lu, int32_t entry, OtherRaw& r) {
    const int fmt = static_cast<int>(static_cast<uint32_t>(entry) >> 30);
    const int64_t idx = entry & 0x3FFFFFFF;
    const int upi = ((unit_of(lu) * 16) & (P.bs - 1)) >> 4;
    if (fmt != VK_FMT_F16) {  // fp8 (the words fp8 units use of OtherRaw: 16 registers, + 8 dynamic)
      const uint8_t* pg = P.pool[1] + (layer * P.cap[1] + idx) * P.page_bytes[1];
      const uint4* kp = reinterpret_cast<const uint4*>(pg + kvh * P.tile_bytes[1] + (upi * 16 + c16) * D + dbase);
#pragma unroll
      for (int c = 0; c < NC; ++c) r.k[c] = kp[c];
      const uint8_t* vt = pg + (P.hkv + kvh) * P.tile_bytes[1];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        r.v[j].x = *reinterpret_cast<const uint32_t*>(vt + static_cast<int64_t>(16 * j + c16) * P.bs + upi * 16 + 4 * grp);
      if constexpr (DYN) {
        // token scales after each tile's codes; this lane's score and value rows are tokens
        // 4 grp .. 4 grp + 3
        const int64_t so = static_cast<int64_t>(P.bs) * D + 4 * (upi * 16 + 4 * grp);
        r.ks4 = *reinterpret_cast<const float4*>(pg + kvh * P.tile_bytes[1] + so);
        r.vs4 = *reinterpret_cast<const float4*>(vt + so);
      }
    } else {
      const uint8_t* pg = P.pool[2] + (layer * P.cap[2] + idx) * P.page_bytes[2];
      const uint4* kp =
          reinterpret_cast<const uint4*>(pg + kvh * P.tile_bytes[2] + ((upi * 16 + c16) * D + dbase) * 2);
#pragma unroll
      for (int c = 0; c < 2 * NC; ++c) r.k[c] = kp[c];
      const uint8_t* vt = pg + (P.hkv + kvh) * P.tile_bytes[2];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        r.v[j] = *reinterpret_cast<const uint2*>(vt + (static_cast<int64_t>(16 * j + c16) * P.bs + upi * 16 + 4 * grp) * 2);
    }
  };
  // The A operands and scales of an fp8 / fp16 unit from its raw words (f16 values, not
  // u * 2^-14).  ks[r]: factor of the score of token 4 grp + r (applied to the float32 product);
  // rt[r]: factor of that token's probability in P*V; vscale: factor of the unit's P*V sum.
  // Dynamic FP8 gives every token its own scales: ks = s_t, rt = s_t / s_max (at most 1: no f16
  // overflow) and vscale = s_max for the values.  Only attended tokens count towards s_max: a
  // slot past the sequence may hold a stale scale of a recycled page.
  auto convert_other = [&](int lu, int32_t entry, const OtherRaw& r, h8_t (&ka)[NS], h4_t (&va)[NB],
                           float (&ks)[4], float (&rt)[4], float& vscale) {
    const int fmt = static_cast<int>(static_cast<uint32_t>(entry) >> 30);
#pragma unroll
    for (int i = 0; i < 4; ++i) ks[i] = 1.0f, rt[i] = 1.0f;
    vscale = 1.0f;
    if (fmt == VK_FMT_FP8E4M3) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 x = r.k[c];
        const uint32_t lo[2] = {x.x, x.y}, hi[2] = {x.z, x.w};
        uint32_t t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t bl = (lo[i >> 2] >> (8 * (i & 3))) & 0xFFu;
          const uint32_t bh = (hi[i >> 2] >> (8 * (i & 3))) & 0xFFu;
          t[i] = h2u(fp8x2(bl | (bh << 16)));
        }
        ka[2 * c] = __builtin_bit_cast(h8_t, u4_t{t[0], t[1], t[2], t[3]});
        ka[2 * c + 1] = __builtin_bit_cast(h8_t, u4_t{t[4], t[5], t[6], t[7]});
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint32_t x = r.v[j].x;
        va[j] = __builtin_bit_cast(h4_t, u2_t{h2u(fp8x2((x & 0xFFu) | ((x & 0xFF00u) << 8))),
                                              h2u(fp8x2(((x >> 16) & 0xFFu) | ((x >> 8) & 0x00FF0000u)))});
      }
      if constexpr (!DYN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ks[i] = P.fp8_scale;
        vscale = P.fp8_scale;
      } else {
        const int t0 = unit_of(lu) * 16;
        ks[0] = r.ks4.x; ks[1] = r.ks4.y; ks[2] = r.ks4.z; ks[3] = r.ks4.w;
        float vv[4] = {r.vs4.x, r.vs4.y, r.vs4.z, r.vs4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = attended_tok(t0 + 4 * grp + i) ? vv[i] : 0.0f;
        const float vmax = max_rows(fmaxf(fmaxf(vv[0], vv[1]), fmaxf(vv[2], vv[3])));
        const float inv = vmax > 0.0f ? 1.0f / vmax : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) rt[i] = vv[i] * inv;
        vscale = vmax;
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 x0 = r.k[2 * c], x1 = r.k[2 * c + 1];
        const uint32_t lo[4] = {x0.x, x0.y, x0.z, x0.w}, hi[4] = {x1.x, x1.y, x1.z, x1.w};
        uint32_t t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          t[i] = ((lo[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) | (((hi[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16);
        ka[2 * c] = __builtin_bit_cast(h8_t, u4_t{t[0], t[1], t[2], t[3]});
        ka[2 * c + 1] = __builtin_bit_cast(h8_t, u4_t{t[4], t[5], t[6], t[7]});
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) va[j] = __builtin_bit_cast(h4_t, u2_t{r.v[j].x, r.v[j].y});
    }
  };

  // A operands and scales of a non-ternary unit, loaded here: fp8 / fp16 through the two steps
  // above; lossless pages (LL instances) rebuilt from their streams.
  auto operands_other = [&](int lu, int32_t entry, h8_t (&ka)[NS], h4_t (&va)[NB], float (&ks)[4], float (&rt)[4],
                            float& vscale) {
    const int fmt = static_cast<int>(static_cast<uint32_t>(entry) >> 30);
    if (!(LL && fmt == VK_FMT_LOSSLESS)) {
      OtherRaw r;
      load_other(lu, entry, r);
      convert_other(lu, entry, r, ka, va, ks, rt, vscale);
      return;
    }
    const int64_t idx = entry & 0x3FFFFFFF;
    const int upi = ((unit_of(lu) * 16) & (P.bs - 1)) >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) ks[r] = 1.0f, rt[r] = 1.0f;
    vscale = 1.0f;
    {

      // bfloat16 values of the unit's K and V groups, rebuilt from the exponent codes (escapes
      // from the exception list, this lane's run of it) and the sign+mantissa bytes, or read
      // raw; each group scaled by one power of two into f16 (largest magnitude below 2^15,
      // exact for every value within 2^-28 of it) and the scale taken back out of the scores
      // (ks) and of the P*V sum (vscale).  This lane's D/4 values of a group, in position order
      // p: keys dims dbase + p; values dim 16 (p / 4) + c16, token 4 grp + p % 4 -- the very
      // positions of its A operands, so each value goes straight into its operand word (as
      // bfloat16 first, converted once the group's largest exponent is known).
      const uint8_t* pg = P.pool[3] + (layer * P.cap[3] + idx) * P.page_bytes[3];
      const int64_t slot_b = 32 * D + 16;
      constexpr int NW = D / 32;     // 8-value chunks per lane (one code word each)
      // out: the operand words as bfloat16 pairs.  Keys: row 2 (w/2) + q/4, word q % 4, half
      // w % 2 (the pair (d, d + 8) of a 16-dim block); values: row j / 2, words 2 (j % 2) and
      // 2 (j % 2) + 1 hold tokens (0, 1) and (2, 3) of dim 16 j + c16
      auto lossless_group = [&](const uint8_t* slot, bool keys, uint32_t (&out)[NW][4]) -> float {
        const uint4 hd = *reinterpret_cast<const uint4*>(slot);
        const int cen = static_cast<int>(hd.x & 0xFFu);
        const bool raw = (hd.x >> 8) & 1u;
        const uint8_t* body = slot + 16;
        const uint8_t* codes = body + 16 * D;
        // element index (stored order) of the first value of chunk w; values: the chunk is
        // dims 16 (2w) + c16 and 16 (2w + 1) + c16, four tokens each
        auto e0 = [&](int w) { return keys ? c16 * D + dbase + 8 * w : (32 * w + c16) * 16 + 4 * grp; };
        auto put = [&](int w, int q, uint32_t h) {   // q = position within the chunk
          if (keys) out[2 * (w >> 1) + (q >> 2)][q & 3] |= h << (16 * (w & 1));
          else out[w][2 * (q >> 2) + ((q >> 1) & 1)] |= h << (16 * (q & 1));
        };
#pragma unroll
        for (int x = 0; x < NW; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) out[x][y] = 0u;
        int emax = 0;
        if (raw) {
          const uint16_t* b16 = reinterpret_cast<const uint16_t*>(body);
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            uint32_t v[4];
            if (keys) {
              const uint4 x = *reinterpret_cast<const uint4*>(b16 + e0(w));
              v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
            } else {
              const uint2 x = *reinterpret_cast<const uint2*>(b16 + e0(w));
              const uint2 y = *reinterpret_cast<const uint2*>(b16 + e0(w) + 256);
              v[0] = x.x; v[1] = x.y; v[2] = y.x; v[3] = y.y;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const uint32_t h = (v[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
              emax = max(emax, static_cast<int>((h >> 7) & 0xFFu));
              put(w, q, h);
            }
          }
        } else {
          uint32_t cw[NW];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            if (keys) {
              cw[w] = *reinterpret_cast<const uint32_t*>(codes + (e0(w) >> 1));
            } else {
              cw[w] = static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(codes + (e0(w) >> 1))) |
                      (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(codes + ((e0(w) + 256) >> 1))) << 16);
            }
          }
          int cnt = 0;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t x = cw[w];
            cnt += __builtin_popcount(x & (x >> 1) & (x >> 2) & (x >> 3) & 0x11111111u);
          }
          int incl = cnt;  // exclusive prefix over the lanes: this lane's first exception
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
          }
          const uint8_t* exc = codes + 8 * D + (incl - cnt);
          int k = 0;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            uint32_t sm[2];
            if (keys) {
              const uint2 x = *reinterpret_cast<const uint2*>(body + e0(w));
              sm[0] = x.x; sm[1] = x.y;
            } else {
              sm[0] = *reinterpret_cast<const uint32_t*>(body + e0(w));
              sm[1] = *reinterpret_cast<const uint32_t*>(body + e0(w) + 256);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const uint32_t cd = (cw[w] >> (4 * q)) & 0xFu;
              const uint32_t e = cd == 15u ? exc[k++] : static_cast<uint32_t>(cen - 11) + cd;
              const uint32_t b = (sm[q >> 2] >> (8 * (q & 3))) & 0xFFu;
              emax = max(emax, static_cast<int>(e & 0xFFu));
              put(w, q, ((b & 0x80u) << 8) | ((e & 0xFFu) << 7) | (b & 0x7Fu));
            }
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) emax = max(emax, __shfl_xor(emax, off, 64));
        const int sh = emax == 0 ? 0 : min(141 - emax, 126);
        const float mul = pow2i(sh);
#pragma unroll
        for (int x = 0; x < NW; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            const uint32_t u = out[x][y];
            out[x][y] = f16_bits(__uint_as_float(u << 16) * mul) | (f16_bits(__uint_as_float(u & 0xFFFF0000u) * mul) << 16);
          }
        return pow2i(-sh);
      };
      uint32_t ow[NW][4];
      const float kinv = lossless_group(pg + kvh * P.tile_bytes[3] + upi * slot_b, true, ow);
#pragma unroll
      for (int c = 0; c < 2 * NC; ++c) ka[c] = __builtin_bit_cast(h8_t, u4_t{ow[c][0], ow[c][1], ow[c][2], ow[c][3]});
#pragma unroll
      for (int r = 0; r < 4; ++r) ks[r] = kinv;
      vscale = lossless_group(pg + (P.hkv + kvh) * P.tile_bytes[3] + upi * slot_b, false, ow);
#pragma unroll
      for (int j = 0; j < NB; ++j) va[j] = __builtin_bit_cast(h4_t, u2_t{ow[j >> 1][2 * (j & 1)], ow[j >> 1][2 * (j & 1) + 1]});
    }
  };


  // Block x = n_splits: the fp8 / fp16 units of every attended range.  Every wave scans the
  // range 64 units at a time (a ballot over one block-table entry per lane) and takes every
  // fourth such unit.  Their values enter the product as themselves (fp8 scaled by
  // fp8_scale): no offsets, no gamma bookkeeping (vcur stays 1, tsum 0).
  if (mixed_part) {
    make_qb();
    vcur = 1.0f;
    // only the two ranges the host found to hold every fp8 / fp16 unit are scanned
    const int m_lo[2] = {a.mix[b][0], a.mix[b][2]}, m_hi[2] = {min(a.mix[b][1], U), min(a.mix[b][3], U)};
    // the extra blocks' waves take the units in turn
    const int n_take = LL ? NW : NW * a.n_mix_parts;
    const int my_turn = LL ? wave : (split - a.n_splits) * NW + wave;
    // one fp8 / fp16 (LL: lossless) unit: scores, online softmax, P*V
    auto mix_unit = [&](const int lu, const h8_t (&ka)[NS], const h4_t (&va)[NB], const float (&ksc)[4],
                        const float (&prt)[4], const float vscale) {
          f4_t s4 = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int s = 0; s < NS; ++s) s4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[s], qb[s], s4, 0, 0, 0);
          const int u = unit_of(lu);
          float sc[4];
          float mx = -INFINITY;
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = u * 16 + 4 * grp + r;
            const bool att = R.single ? t < L : (t < R.sinks || (t >= R.w0 && t < L));
            sc[r] = att ? s4[r] * (ksc[r] * qsl) : -INFINITY;
            mx = fmaxf(mx, sc[r]);
          }
          mx = max_rows(mx);
          if (__builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mx)) == __builtin_bit_cast(int, -INFINITY)) return;
          if (__ballot(mx > m) != 0) {
            const float mn = fmaxf(m, mx);
            const float corr = __builtin_amdgcn_exp2f(m - mn);
  #pragma unroll
            for (int j = 0; j < NB; ++j) oacc[j] *= corr;
            lsum *= corr;
            m = mn;
          }
          const float ms = m - 14.0f;
          const h2_t p01 = {static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[0] - ms)),
                            static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[1] - ms))};
          const h2_t p23 = {static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[2] - ms)),
                            static_cast<_Float16>(__builtin_amdgcn_exp2f(sc[3] - ms))};
          h2_t q01 = as_h2(slot0(h2u(p01))), q23 = as_h2(slot0(h2u(p23)));
          if constexpr (!DYN) {
            lsum = __builtin_amdgcn_fdot2(q01, ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2(q23, ones, lsum, false);
          } else {
            // each token's value scale relative to the unit's largest; the sum takes each weight
            // as P*V sees it (the f16 product divided back by the ratio) so both round alike
            const float pf[4] = {__builtin_amdgcn_exp2f(sc[0] - ms), __builtin_amdgcn_exp2f(sc[1] - ms),
                                 __builtin_amdgcn_exp2f(sc[2] - ms), __builtin_amdgcn_exp2f(sc[3] - ms)};
            _Float16 qh[4];
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              qh[r] = static_cast<_Float16>(pf[r] * prt[r]);
              const float qr = static_cast<float>(qh[r]);  // below the f16 normal range: unrounded
              if (NSL == 1 || cslot == 0) lsum += qr >= 0x1p-14f ? qr / prt[r] : pf[r];
            }
            q01 = as_h2(slot0(h2u(h2_t{qh[0], qh[1]})));
            q23 = as_h2(slot0(h2u(h2_t{qh[2], qh[3]})));
          }
          const h4_t pb = __builtin_bit_cast(h4_t, u2_t{h2u(q01), h2u(q23)});
          const float vs14 = vscale * (1.0f / 16384.0f);
  #pragma unroll
          for (int j = 0; j < NB; ++j) {
            const f4_t t4 = __builtin_amdgcn_mfma_f32_16x16x16f16(va[j], pb, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            oacc[j] += t4 * vs14;
          }
    };
    if constexpr (LL || D > 128) {
      int rank = 0;  // non-ternary units seen so far (uniform)
      for (int rg = 0; rg < 2; ++rg) {
        for (int c0 = m_lo[rg]; c0 < m_hi[rg]; c0 += 64) {
          const int lu_l = c0 + lane;
          const bool in_rg = lu_l < m_hi[rg];
          const int32_t ent_l = in_rg ? bt[(unit_of(lu_l) * 16) >> P.bs_shift] : 0;
          const uint32_t fmt_l = static_cast<uint32_t>(ent_l) >> 30;
          uint64_t todo = __ballot(in_rg && (LL ? fmt_l == VK_FMT_LOSSLESS
                                                : fmt_l != VK_FMT_TERNARY2 && fmt_l != VK_FMT_LOSSLESS));
          while (todo) {
            const int k = __builtin_ctzll(todo);
            todo &= todo - 1;
            if (rank++ % n_take != my_turn) continue;
            const int lu = c0 + k;
            const int32_t entry = __builtin_amdgcn_readlane(ent_l, k);
            h8_t ka[NS];
            h4_t va[NB];
            float ksc[4], prt[4], vscale;
            operands_other(lu, entry, ka, va, ksc, prt, vscale);
            mix_unit(lu, ka, va, ksc, prt, vscale);
          }
        }
      }
    } else {
      // The wave first lists its units, up to 64 at a time (lane j holds the j-th), then runs
      // them with the next unit's loads in flight while it computes one.  These blocks run
      // while the ternary blocks keep the memory system full, where every load waits a long
      // queue: one load round trip per unit, one after another, would set their time.
      for (int first = 0;; first += 64) {
        int rank = 0, mine = 0, n = 0;  // (uniform)
        int my_lu = 0;
        int32_t my_ent = 0;
        for (int rg = 0; rg < 2; ++rg) {
          for (int c0 = m_lo[rg]; c0 < m_hi[rg]; c0 += 64) {
            const int lu_l = c0 + lane;
            const bool in_rg = lu_l < m_hi[rg];
            const int32_t ent_l = in_rg ? bt[(unit_of(lu_l) * 16) >> P.bs_shift] : 0;
            const uint32_t fmt_l = static_cast<uint32_t>(ent_l) >> 30;
            uint64_t todo = __ballot(in_rg && fmt_l != VK_FMT_TERNARY2 && fmt_l != VK_FMT_LOSSLESS);
            while (todo) {
              const int k = __builtin_ctzll(todo);
              todo &= todo - 1;
              if (rank++ % n_take != my_turn) continue;
              const int j = mine++ - first;
              if (j < 0 || j >= 64) continue;
              const int32_t e = __builtin_amdgcn_readlane(ent_l, k);
              my_lu = lane == j ? c0 + k : my_lu;
              my_ent = lane == j ? e : my_ent;
              ++n;
            }
          }
        }
        if (n == 0) break;
        // Unit i's words are converted to operands, the next fp8 unit's loads go out into the
        // same registers (a clamped index repeats the last unit), and unit i is computed while
        // they land.  fp16 units (the sinks: rare, and twice the registers) load when their turn
        // comes.
        auto fetch8 = [&](int i, OtherRaw& r) {
          const int ii = min(i, n - 1);
          const int32_t e = __builtin_amdgcn_readlane(my_ent, ii);
          if ((static_cast<uint32_t>(e) >> 30) == VK_FMT_FP8E4M3) load_other(__builtin_amdgcn_readlane(my_lu, ii), e, r);
        };
        OtherRaw raw;
        fetch8(0, raw);
        for (int i = 0; i < n; ++i) {
          const int lu = __builtin_amdgcn_readlane(my_lu, i);
          const int32_t entry = __builtin_amdgcn_readlane(my_ent, i);
          h8_t ka[NS];
          h4_t va[NB];
          float ksc[4], prt[4], vscale;
          if ((static_cast<uint32_t>(entry) >> 30) == VK_FMT_FP8E4M3) convert_other(lu, entry, raw, ka, va, ksc, prt, vscale);
          else operands_other(lu, entry, ka, va, ksc, prt, vscale);
          fetch8(i + 1, raw);
          mix_unit(lu, ka, va, ksc, prt, vscale);
        }
        if (n < 64) break;
      }
    }
  }

  // One step of the ring loop: units k + S gi .. k + S gi + S - 1 of a range [c0, c_end) whose
  // metadata is cc; refill(lu, row) starts the copy of unit lu into a ring row.  Slots are
  // taken two at a time: wait until their copies have landed (at most NR - 2 units' ring copies,
  // NCP each, were issued after them; vector memory returns in issue order and any other load in between only
  // makes the wait stricter; the compiler's own wait counting does not follow buffer-to-LDS
  // copies into every ring array), read them into registers, and refill them with the units
  // NR ahead before any compute.
  constexpr int S = SU;  // units per step
  auto step = [&](auto GI, int k, int c0, int c_end, const Chunk& cc, auto&& refill) {
    using std::integral_constant;
    constexpr int gi = decltype(GI)::value;
    UnitRaw<NC, NV> r[S];
    auto take2 = [&](auto H) {
      constexpr int i = 2 * decltype(H)::value;  // first unit of the pair in this step
      if constexpr (i < S) {
        __builtin_amdgcn_s_waitcnt(wait_vm(NCP * (NR - 2)));
        read_unit(ring_row(integral_constant<int, S * gi + i>{}), r[i]);
        read_unit(ring_row(integral_constant<int, S * gi + i + 1>{}), r[i + 1]);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the slot reads have returned
        refill(k + NR + S * gi + i, ring_row(integral_constant<int, S * gi + i>{}));
        refill(k + NR + S * gi + i + 1, ring_row(integral_constant<int, S * gi + i + 1>{}));
      }
    };
    take2(integral_constant<int, 0>{});
    take2(integral_constant<int, 1>{});
    const int lu0 = k + S * gi;
    if (lu0 >= c_end) return;
    // a step whose units in the range are ternary with the chunk's gamma pair runs the clean
    // path (masked when a unit is partly attended or the range ends inside the step); any
    // other takes the general path
    const int n_in = min(S, c_end - lu0);
    const uint64_t in = (uint64_t{1} << n_in) - 1;
    const bool partial = n_in < S || ((cc.fmask >> (lu0 - c0)) & in) != in;
    if (((cc.cmask >> (lu0 - c0)) & in) == in && (PCLEAN || !partial)) {
      process_clean(cc, r, partial, lu0, c_end, ProdF4{});
    } else {
      process_group(lu0, cc, c0, r[0], r[1], ProdF4{});
      if constexpr (S == 4) process_group(lu0 + 2, cc, c0, r[2], r[3], ProdF4{});
    }
  };
  auto ring_round = [&](int k, int c0, int c_end, const Chunk& cc, auto&& refill) {
    using std::integral_constant;
    step(integral_constant<int, 0>{}, k, c0, c_end, cc, refill);
    if constexpr (NR / S >= 2) step(integral_constant<int, 1>{}, k, c0, c_end, cc, refill);
    if constexpr (NR / S >= 4) {
      step(integral_constant<int, 2>{}, k, c0, c_end, cc, refill);
      step(integral_constant<int, 3>{}, k, c0, c_end, cc, refill);
    }
  };
  auto prologue_copies = [&](int u0, auto&& refill) {
    using std::integral_constant;
    auto one = [&](auto I) { refill(u0 + decltype(I)::value, ring_row(I)); };
    one(integral_constant<int, 0>{});
    one(integral_constant<int, 1>{});
    one(integral_constant<int, 2>{});
    one(integral_constant<int, 3>{});
    if constexpr (NR == 8) {
      one(integral_constant<int, 4>{});
      one(integral_constant<int, 5>{});
      one(integral_constant<int, 6>{});
      one(integral_constant<int, 7>{});
    }
  };

  // Short ranges (at most NR units per wave: launches too small to fill the GPU) send every
  // copy at once and walk the slots in a run-time loop: one copy of the step's code instead
  // of one per slot group, so a wave fetches far fewer instruction bytes (a launch this small
  // is bound by latencies, cold instruction fetches among them).
  const bool short_range = u_end - u_begin <= NR;
  if (!STEAL && !mixed_part && u_begin < u_end && short_range) {
    using std::integral_constant;
    Chunk ch = load_chunk(u_begin);
    auto prologue = [&](auto I) { dma_unit(u_begin + decltype(I)::value, ch, ch, u_begin, ring_row(I)); };
    prologue(integral_constant<int, 0>{});
    prologue(integral_constant<int, 1>{});
    prologue(integral_constant<int, 2>{});
    prologue(integral_constant<int, 3>{});
    if constexpr (NR == 8) {
      prologue(integral_constant<int, 4>{});
      prologue(integral_constant<int, 5>{});
      prologue(integral_constant<int, 6>{});
      prologue(integral_constant<int, 7>{});
    }
    make_qb();  // (the f16 product: see ProdF16)
    chunk_flags(ch, u_begin);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // every copy has landed
    auto slot_row = [&](int i) -> const uint8_t* {  // ring row of slot i (wave-uniform)
      const uint8_t* p = ring0[wave];
      p = i == 1 ? ring1[wave] : p;
      p = i == 2 ? ring2[wave] : p;
      p = i == 3 ? ring3[wave] : p;
      if constexpr (NR == 8) {
        p = i == 4 ? ring4[wave] : p;
        p = i == 5 ? ring5[wave] : p;
        p = i == 6 ? ring6[wave] : p;
        p = i == 7 ? ring7[wave] : p;
      }
      return p;
    };
    constexpr int S = SU;  // units per step; NR is a multiple of S, so every slot read is < NR
#pragma unroll 1
    for (int lu0 = u_begin; lu0 < u_end; lu0 += S) {
      UnitRaw<NC, NV> r[S];
#pragma unroll
      for (int i = 0; i < S; ++i) read_unit(slot_row(lu0 - u_begin + i), r[i]);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      const int n_in = min(S, u_end - lu0);
      const uint64_t in = (uint64_t{1} << n_in) - 1;
      const bool partial = n_in < S || ((ch.fmask >> (lu0 - u_begin)) & in) != in;
      if (((ch.cmask >> (lu0 - u_begin)) & in) == in && (PCLEAN || !partial)) {
        process_clean(ch, r, partial, lu0, u_end, ProdF16{});
      } else {
        process_group(lu0, ch, u_begin, r[0], r[1], ProdF16{});
        if constexpr (S == 4) process_group(lu0 + 2, ch, u_begin, r[2], r[3], ProdF16{});
      }
    }
  }

  if (!STEAL && !mixed_part && u_begin < u_end && !short_range) {
    // ring slot s holds unit k + s while the group of slots (2i, 2i + 1) is processed; a
    // processed slot is refilled with the unit NR ahead.  The first copies go out as soon as
    // the first chunk's block-table entries are in (they lie in that chunk); the next chunk's
    // metadata and the query set-up follow while they are in flight.
    using std::integral_constant;
    Chunk ch_cur = load_chunk(u_begin);
    auto prologue = [&](auto I) { dma_unit(u_begin + decltype(I)::value, ch_cur, ch_cur, u_begin, ring_row(I)); };
    prologue(integral_constant<int, 0>{});
    prologue(integral_constant<int, 1>{});
    prologue(integral_constant<int, 2>{});
    prologue(integral_constant<int, 3>{});
    if constexpr (NR == 8) {
      prologue(integral_constant<int, 4>{});
      prologue(integral_constant<int, 5>{});
      prologue(integral_constant<int, 6>{});
      prologue(integral_constant<int, 7>{});
    }
    // (no next chunk: the copies never select it, and it stays a copy of the current one)
    Chunk ch_nxt = u_begin + CH < u_end ? load_chunk(u_begin + CH) : ch_cur;
    make_qt();
    for (int c0 = u_begin; c0 < u_end; c0 += CH) {
      const int c_end = min(c0 + CH, u_end);
      chunk_flags(ch_cur, c0);
      constexpr int S = SU;  // units per step
#pragma unroll 1
      for (int k = c0; k < c_end; k += NR) {
        auto step = [&](auto GI) {
          constexpr int gi = decltype(GI)::value;
          UnitRaw<NC, NV> r[S];
          // Slots are taken two at a time: wait until their copies have landed (at most
          // NR - 2 units' ring copies (NCP each) were issued after them; vector memory returns in issue order
          // and any other load in between only makes the wait stricter; the compiler's own
          // wait counting does not follow buffer-to-LDS copies into every ring array), read
          // them into registers, and refill them with the units NR ahead before any compute.
          auto take2 = [&](auto H) {
            constexpr int i = 2 * decltype(H)::value;  // first unit of the pair in this step
            if constexpr (i < S) {
              __builtin_amdgcn_s_waitcnt(wait_vm(NCP * (NR - 2)));
              read_unit(ring_row(integral_constant<int, S * gi + i>{}), r[i]);
              read_unit(ring_row(integral_constant<int, S * gi + i + 1>{}), r[i + 1]);
              __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the slot reads have returned
              dma_unit(k + NR + S * gi + i, ch_cur, ch_nxt, c0, ring_row(integral_constant<int, S * gi + i>{}));
              dma_unit(k + NR + S * gi + i + 1, ch_cur, ch_nxt, c0,
                       ring_row(integral_constant<int, S * gi + i + 1>{}));
            }
          };
          take2(integral_constant<int, 0>{});
          take2(integral_constant<int, 1>{});
          const int lu0 = k + S * gi;
          if (lu0 >= c_end) return;
          // a step whose units in the range are ternary with the chunk's gamma pair runs the
          // clean path (masked when a unit is partly attended or the range ends inside the
          // step); any other takes the general path
          const int n_in = min(S, c_end - lu0);
          const uint64_t in = (uint64_t{1} << n_in) - 1;
          const bool partial = n_in < S || ((ch_cur.fmask >> (lu0 - c0)) & in) != in;
          if (((ch_cur.cmask >> (lu0 - c0)) & in) == in && (PCLEAN || !partial)) {
            process_clean(ch_cur, r, partial, lu0, c_end, ProdF4{});
          } else {
            process_group(lu0, ch_cur, c0, r[0], r[1], ProdF4{});
            if constexpr (S == 4) process_group(lu0 + 2, ch_cur, c0, r[2], r[3], ProdF4{});
          }
        };
        step(integral_constant<int, 0>{});
        if constexpr (NR / S >= 2) step(integral_constant<int, 1>{});
        if constexpr (NR / S >= 4) {
          step(integral_constant<int, 2>{});
          step(integral_constant<int, 3>{});
        }
      }
      ch_cur = ch_nxt;  // the next chunk's metadata was fetched one chunk ahead
      if (c0 + 2 * CH < u_end) ch_nxt = load_chunk(c0 + 2 * CH);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no copy into the ring is left in flight
  }

  if constexpr (STEAL) {
    // Work stealing inside the block: its units go in pieces of kPiece to whichever wave asks
    // next (an LDS counter), so every wave stays busy until the block's units run out.  A wave
    // asks for its next piece when it starts one, so its ring copies run on into that piece; a
    // piece holds two ring rounds, which gives the next piece's metadata a round to arrive.
    // The counter only grows, so every wave leaves the loop.
    static_assert(kPiece % NR == 0 && kPiece <= CH, "whole ring rounds per piece");
    const int n_pieces = (s_end - s_begin + kPiece - 1) / kPiece;
    auto grab = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(&lds_next, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    int p_cur = mixed_part ? n_pieces : grab();
    if (p_cur < n_pieces) {
      int p_nxt = grab();
      int cs = s_begin + p_cur * kPiece, ce = min(cs + kPiece, s_end);
      int ns = cs, ne = cs;  // next piece [ns, ne); empty when there is none
      if (p_nxt < n_pieces) ns = s_begin + p_nxt * kPiece, ne = min(ns + kPiece, s_end);
      Chunk ch_cur = load_chunk(cs);
      Chunk ch_nxt = ch_cur;
      // copy of unit lu: in the current piece, or position lu - cs - kPiece of the next one;
      // a unit past either piece gets an empty record range (it reads no memory)
      auto refill = [&](int lu, uint8_t* row) {
        const bool in_cur = lu - cs < kPiece;
        const int li = in_cur ? lu - cs : lu - cs - kPiece;
        const int un = in_cur ? lu : ns + li;
        const bool valid = in_cur ? un < ce : un < ne;
        const uint32_t lo = __builtin_amdgcn_readlane(in_cur ? ch_cur.plo : ch_nxt.plo, li);
        const uint32_t hi = __builtin_amdgcn_readlane(in_cur ? ch_cur.phi : ch_nxt.phi, li);
        const uint8_t* pg = reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
        const int upi = valid ? ((unit_of(un) * 16) & (P.bs - 1)) >> 4 : 0;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pg), 0, valid ? page_bytes0 : 0, kBufferWord3);
        const int soff = kvh * tile0 + upi * 4 * D;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)row, 16, dma_off, soff, 0, 0);
      };
      prologue_copies(cs, refill);
      if (p_nxt < n_pieces) ch_nxt = load_chunk(ns);
      make_qt();
      while (true) {
        chunk_flags(ch_cur, cs);
#pragma unroll 1
        for (int k = cs; k < cs + kPiece; k += NR) ring_round(k, cs, ce, ch_cur, refill);
        if (p_nxt >= n_pieces) break;
        p_cur = p_nxt;
        cs = ns;
        ce = ne;
        ch_cur = ch_nxt;
        p_nxt = grab();
        ns = ne = cs;
        if (p_nxt < n_pieces) {
          ns = s_begin + p_nxt * kPiece;
          ne = min(ns + kPiece, s_end);
          ch_nxt = load_chunk(ns);
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no copy into the ring is left in flight
    }
  }

  // ---------------- this wave's partial state -> LDS ----------------
  // (dimension d of head h of wave w sits at h D + swz(h, d) of the wave's staging rows: the
  // XOR spreads the heads' rows, written by lanes of one column each, over the LDS banks)
  // 4-wave blocks stage in LDS of their own (8-16 KB), so a wave that has finished stages its
  // outputs while slower waves still compute; 12-wave blocks reuse the ring, once every wave
  // has left its loop.
  constexpr bool OWN_STAGE = !STEAL;
  __shared__ __attribute__((aligned(16))) float stage[OWN_STAGE ? NW * G * D : 4];
  constexpr int PER = (NW * RB) / (G * D * 4) < NW ? (NW * RB) / (G * D * 4) : NW;  // waves per ring array
  static_assert(OWN_STAGE || (PER >= 1 && (NW + PER - 1) / PER <= 4), "the waves' outputs fit ring arrays 0-3");
  auto out_row = [&](int w) -> float* {
    if constexpr (OWN_STAGE) return stage + w * (G * D);
    const int q = w / PER;
    uint8_t* r = q == 0 ? &ring0[0][0] : q == 1 ? &ring1[0][0] : q == 2 ? &ring2[0][0] : &ring3[0][0];
    return reinterpret_cast<float*>(r) + (w % PER) * (G * D);
  };
  auto swz = [](int h, int d) { return d ^ ((h & 7) << 2); };  // stays in d's 32-float block
  if constexpr (!OWN_STAGE) __syncthreads();
  lsum = sum_rows(lsum);
  tsum = sum_rows(tsum);
  // sum the slots (each head's columns hold the units of its own clean steps) with row
  // rotations: after rotating by 8 a lane holds the sum over columns c16 and c16 ^ 8, and a
  // rotation by 4 of that sum then covers all four slots
  auto slot_sum = [](float x) {
    if constexpr (NSL >= 2)
      x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
    if constexpr (NSL == 4)
      x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
    return x;
  };
  lsum = slot_sum(lsum);
  tsum = slot_sum(tsum);
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[j][r] = slot_sum(oacc[j][r]);
  if (c16 < G) {
    constexpr float kInv = 1.0f / 16384.0f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // ternary tokens added p' (off_j + u 2^-14); their values are gamma (u - 1)
      const float sub = tsum * (va_off<NV>(j) + kInv);
      *reinterpret_cast<float4*>(out_row(wave) + c16 * D + swz(c16, 16 * j + 4 * grp)) =
          float4{(oacc[j][0] - sub) * vcur, (oacc[j][1] - sub) * vcur, (oacc[j][2] - sub) * vcur,
                 (oacc[j][3] - sub) * vcur};
    }
    if (grp == 0) {
      lds_m[wave][c16] = m;
      lds_l[wave][c16] = lsum * kInv;
    }
  }
  __syncthreads();

  // ---------------- merge the four waves ----------------
  // four consecutive outputs of one head per thread: the waves' weights once, then one
  // 16-byte LDS read per wave and one store (partials: (D + 2)-float records, 8-byte aligned)
  static_assert(D % 4 == 0, "whole float4 groups per head");
  for (int e = threadIdx.x; e < G * D / 4; e += 64 * NW) {
    const int hh = (4 * e) / D, dd = (4 * e) % D;
    float mw[NW], lw[NW];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = lds_m[w][hh];
      lw[w] = lds_l[w][hh];
      M = fmaxf(M, mw[w]);
    }
    float4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float4 o = *reinterpret_cast<const float4*>(out_row(w) + hh * D + swz(hh, dd));
      if (lw[w] > 0.0f) {  // a wave with nothing attended adds nothing (its outputs are not set)
        const float wt = __builtin_amdgcn_exp2f(mw[w] - M);
        num.x = fmaf(wt, o.x, num.x);
        num.y = fmaf(wt, o.y, num.y);
        num.z = fmaf(wt, o.z, num.z);
        num.w = fmaf(wt, o.w, num.w);
        den = fmaf(wt, lw[w], den);
      }
    }
    const int64_t qh = qh0 + hh;
    if (a.n_parts == 1) {
      const float inv = 1.0f / den;
      *reinterpret_cast<float4*>(a.out + (qo0 + hh) * D + dd) = float4{num.x * inv, num.y * inv, num.z * inv, num.w * inv};
    } else if (!a.fused_merge) {
      float* part = a.partials + (qh * a.n_parts + split) * (D + 2);
      *reinterpret_cast<float2*>(part + dd) = float2{num.x, num.y};
      *reinterpret_cast<float2*>(part + dd + 2) = float2{num.z, num.w};
      if (dd == 0) *reinterpret_cast<float2*>(part + D) = float2{M, den};
    } else {
      // device-coherent stores (they reach the memory every XCD reads, not only this XCD's L2),
      // so the block that merges, on any XCD, reads them with device-coherent loads
      // (8-byte stores: the (D + 2)-float records are 8-byte aligned)
      float* part = a.partials + (qh * a.n_parts + split) * (D + 2);
      auto st2 = [](float* p, float x, float y) {
        const uint64_t v = (static_cast<uint64_t>(__float_as_uint(y)) << 32) | __float_as_uint(x);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };
      st2(part + dd, num.x, num.y);
      st2(part + dd + 2, num.z, num.w);
      if (dd == 0) st2(part + D, M, den);
    }
  }
  if (a.n_parts > 1 && a.fused_merge) merge_parts_last_block<D, G, NW>(a, b, kvh, qh0, qo0);
}

// Combines split partials: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One block per (sequence, query head); weights computed once into LDS, then
// every dimension sums its column with eight independent loads in flight.
template <int D>
__global__ __launch_bounds__(D) void k_merge(DecodeArgs a) {
  __shared__ float wts[64];
  __shared__ float den_s;
  const int64_t qh = static_cast<int64_t>(blockIdx.y) * a.hq + blockIdx.x;
  const int dd = threadIdx.x;
  const int ns = a.n_parts;  // <= 64
  const float* base = a.partials + qh * ns * (D + 2);
  if (dd < 64) {
    const float ms = dd < ns ? base[dd * (D + 2) + D] : -INFINITY;
    const float ls = dd < ns ? base[dd * (D + 2) + D + 1] : 0.0f;
    float M = ms;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float wgt = ls > 0.0f ? exp2f(ms - M) : 0.0f;
    float den = wgt * ls;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
    wts[dd] = wgt;
    if (dd == 0) den_s = den;
  }
  __syncthreads();
  float num = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float o8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o8[k] = s0 + k < ns ? base[(s0 + k) * (D + 2) + dd] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) num = s0 + k < ns ? fmaf(wts[s0 + k], o8[k], num) : num;
  }
  a.out[(static_cast<int64_t>(a.rows[blockIdx.y]) * a.hq + blockIdx.x) * D + dd] = num / den_s;
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t s, LaunchTimer* t) {
  // matrix-core path: grid (hkv, n_seqs, n_parts), parts n_splits .. take the fp8 / fp16 pages;
  // vector-ALU path: grid (n_splits, hkv, n_seqs)
  const dim3 grid = a.kernel == VK_DECODE_VALU ? dim3(a.n_splits, a.P.hkv, a.n_seqs)
                   : a.n_order > 0               ? dim3(a.P.hkv, a.n_order, 1)
                                                 : dim3(a.P.hkv, a.n_seqs, a.n_splits + a.n_mix_parts);
  if (a.n_order > 0 && (a.kernel == VK_DECODE_VALU || a.steal ||
                        a.n_order != a.n_seqs * (a.n_splits + a.n_mix_parts)))
    return hipErrorInvalidValue;
  if (t) t->begin(VK_KERNEL_DECODE, s);
  if (a.kernel == VK_DECODE_VALU) {
    if (a.q_dtype == VK_DTYPE_BF16) k_decode<D, G, 1><<<grid, 64, 0, s>>>(a);
    else k_decode<D, G, 0><<<grid, 64, 0, s>>>(a);
  } else if (a.steal) {  // all-ternary launch with a block per CU: 12 waves share each block's units
    if (a.q_dtype == VK_DTYPE_BF16) k_decode_mfma<D, G, 1, 8, false, true><<<grid, 64 * kStealWaves, 0, s>>>(a);
    else k_decode_mfma<D, G, 0, 8, false, true><<<grid, 64 * kStealWaves, 0, s>>>(a);
  } else if (a.P.fp8_dynamic) {  // dynamic FP8 pages: their scale handling in its own instance
    if (a.q_dtype == VK_DTYPE_BF16) k_decode_mfma<D, G, 1, 8, true, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
    else k_decode_mfma<D, G, 0, 8, true, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
  } else if (a.units_per_iter == 8) {
    if (a.q_dtype == VK_DTYPE_BF16) k_decode_mfma<D, G, 1, 8, false, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
    else k_decode_mfma<D, G, 0, 8, false, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
  } else {
    if (a.q_dtype == VK_DTYPE_BF16) k_decode_mfma<D, G, 1, 4, false, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
    else k_decode_mfma<D, G, 0, 4, false, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
  }
  if (a.lossless) {  // the lossless pages: one block per (KV head, sequence), part n_splits + n_mix_parts
    DecodeArgs b = a;
    b.part_base = a.n_splits + a.n_mix_parts;
    b.n_order = 0;
    const dim3 g1(a.P.hkv, a.n_seqs, 1);
    if (a.q_dtype == VK_DTYPE_BF16) k_decode_mfma<D, G, 1, 8, false, false, true><<<g1, 64 * kMfmaWaves, 0, s>>>(b);
    else k_decode_mfma<D, G, 0, 8, false, false, true><<<g1, 64 * kMfmaWaves, 0, s>>>(b);
  }
  if (t) t->end(VK_KERNEL_DECODE, s);
  if (a.n_parts > 1 && !a.fused_merge) {
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

// Head dim 256: the vector-ALU kernel, or the matrix-core kernel with a 4-slot ring of 2 KB
// rows (no stealing blocks, no lossless pages: the host sends neither), then the merge when
// there are several parts.
template <int G>
hipError_t launch_d256(const DecodeArgs& a, hipStream_t s, LaunchTimer* t) {
  if (a.lossless || a.steal) return hipErrorInvalidValue;
  if (a.n_order > 0 && (a.kernel == VK_DECODE_VALU || a.n_order != a.n_seqs * (a.n_splits + a.n_mix_parts)))
    return hipErrorInvalidValue;
  if (t) t->begin(VK_KERNEL_DECODE, s);
  if (a.kernel == VK_DECODE_VALU) {
    if (a.n_mix_parts) return hipErrorInvalidValue;
    const dim3 grid(a.n_splits, a.P.hkv, a.n_seqs);
    if (a.q_dtype == VK_DTYPE_BF16) k_decode<256, G, 1><<<grid, 64, 0, s>>>(a);
    else k_decode<256, G, 0><<<grid, 64, 0, s>>>(a);
  } else {
    const dim3 grid = a.n_order > 0 ? dim3(a.P.hkv, a.n_order, 1) : dim3(a.P.hkv, a.n_seqs, a.n_splits + a.n_mix_parts);
    if (a.P.fp8_dynamic) {
      if (a.q_dtype == VK_DTYPE_BF16) k_decode_mfma<256, G, 1, 4, true, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
      else k_decode_mfma<256, G, 0, 4, true, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
    } else {
      if (a.q_dtype == VK_DTYPE_BF16) k_decode_mfma<256, G, 1, 4, false, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
      else k_decode_mfma<256, G, 0, 4, false, false><<<grid, 64 * kMfmaWaves, 0, s>>>(a);
    }
  }
  if (t) t->end(VK_KERNEL_DECODE, s);
  if (a.n_parts > 1 && !a.fused_merge) {
    if (t) t->begin(VK_KERNEL_MERGE, s);
    k_merge<256><<<dim3(a.hq, a.n_seqs), 256, 0, s>>>(a);
    if (t) t->end(VK_KERNEL_MERGE, s);
  }
  return hipGetLastError();
}

}  // namespace

// This file is compiled twice (VK_DECODE_DIM = 64 or 128), so that the kernel instances build
// in two halves in parallel; the head-dim-64 half also holds the head-dim-256 instances.
#if VK_DECODE_DIM == 64
hipError_t launch_decode_d64(const DecodeArgs& a, int32_t group, hipStream_t s, LaunchTimer* t) {
  if (a.P.dim == 256) {
    switch (group) {
      case 1: return launch_d256<1>(a, s, t);
      case 2: return launch_d256<2>(a, s, t);
      case 4: return launch_d256<4>(a, s, t);
      case 8: return launch_d256<8>(a, s, t);
    }
    return hipErrorInvalidValue;
  }
  return launch_d<64>(a, group, s, t);
}
#elif VK_DECODE_DIM == 128
hipError_t launch_decode_d64(const DecodeArgs& a, int32_t group, hipStream_t s, LaunchTimer* t);

hipError_t launch_decode(const DecodeArgs& a, int32_t group, hipStream_t s, LaunchTimer* t) {
  if (a.P.dim == 128) return launch_d<128>(a, group, s, t);
  if (a.P.dim == 64 || a.P.dim == 256) return launch_decode_d64(a, group, s, t);
  return hipErrorInvalidValue;
}
#else
#error "compile with -DVK_DECODE_DIM=64 or -DVK_DECODE_DIM=128"
#endif

}  // namespace vk
