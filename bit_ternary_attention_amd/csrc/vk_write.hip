// Write side: per-tensor absmean scale, ternary quantisation, 2-bit packing
// and page scatter, for gfx950.
//
// Follows "Show HN: Vantage-V-AI" (newshot.cc), section "core architecture":
// gamma = mean(|X|) per tensor, states {-1, 0, +1}, four elements per uint8.
// FP8 recent pages and FP16 anchor (sink) pages follow "Minima-KV"
// (twodots.gr), section "Recent, Anchor and Stale".
//
// Three kernels per append call:
//   k_absmean_partial  pass 1: fixed-partition float64 sums of |x|, one per
//                      (segment, 32 KiB block), no atomics -> deterministic
//   k_gamma_finalize   one wave per segment: fixed-order sum, gamma = fp32(S/N),
//                      and the exact 16-bit magnitude threshold of a nonzero code
//   k_pack             pass 2: one wave per (16-token unit, K|V, head) tile;
//                      codes from an integer compare against the threshold,
//                      keys stored token-major, values rearranged through LDS
//                      into per-unit chunks (one chunk per decode lane)
//
// Exactness of the threshold: with d = gamma + eps > 0 and RNE float32
// division, round(x/d) is nonzero exactly when the float32 quotient exceeds
// 1/2, i.e. when |x|/d > 1/2 + 2^-25 (the midpoint to the next float32 above
// 1/2; a tie rounds to 1/2, whose significand is even).  d * (1/2 + 2^-25)
// is exact in float64 (24 + 25 significand bits), so no division is needed
// and the compare is exact.  The magnitude order of 16-bit patterns equals
// their value order, so the compare runs on the raw bits.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "host_state.h"
#include "vk_params.h"

namespace vk {
namespace {

template <int DT>
__device__ __forceinline__ float to_f32(uint32_t h) {  // low 16 bits
  if (DT == 1) return __uint_as_float(h << 16);
  return __half2float(__ushort_as_half(static_cast<unsigned short>(h)));
}

// Sum of |x| over the eight 16-bit values of a 16-byte load, in float64.
template <int DT>
__device__ __forceinline__ double abs_sum8(uint4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s += static_cast<double>(fabsf(to_f32<DT>(ws[k] & 0xFFFFu)));
    s += static_cast<double>(fabsf(to_f32<DT>(ws[k] >> 16)));
  }
  return s;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Fixed-order block reduction (256 threads = 4 waves).
__device__ __forceinline__ double block_sum256(double x) {
  __shared__ double part[4];
  x = wave_sum(x);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[wave] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) t = ((part[0] + part[1]) + part[2]) + part[3];
  return t;
}

// Exact value of a non-negative 16-bit magnitude pattern.
template <int DT>
__device__ double value16(uint32_t m) {
  if (DT == 1) return static_cast<double>(__uint_as_float(m << 16));
  const uint32_t e = m >> 10, f = m & 0x3FFu;
  if (e == 0) return ldexp(static_cast<double>(f), -24);
  if (e == 31) return __longlong_as_double(0x7FF0000000000000ll);
  return ldexp(static_cast<double>(f + 1024u), static_cast<int>(e) - 25);
}

// Smallest magnitude pattern m with value(m) > d * (1/2 + 2^-25): codes are
// nonzero exactly for |x| >= value(m).  The predicate is monotone in m and holds
// from the infinity pattern on; one wave finds its first m in three rounds of 64
// candidates (steps 512, 8, 1).  Every lane of the wave calls it; the result is uniform.
template <int DT>
__device__ uint32_t threshold16_wave(float d) {
  const double tau = static_cast<double>(d) * (0.5 + 0x1p-25);
  const uint32_t top = DT == 1 ? 0x7F80u : 0x7C00u;  // +infinity
  const uint32_t lane = threadIdx.x & 63;
  auto above = [&](uint32_t m) { return m >= top || value16<DT>(m) > tau; };
  const uint64_t b1 = __ballot(above(lane * 512u));
  if (b1 & 1u) return 0u;
  // first holding candidate; none below 32256 puts it in the last step (above(32768) holds)
  const uint32_t j1 = b1 ? static_cast<uint32_t>(__builtin_ctzll(b1)) : 64u;
  const uint32_t lo1 = (j1 - 1u) * 512u;  // above(lo1) fails
  const uint64_t b2 = __ballot(above(lo1 + lane * 8u));  // lo1 + 512 holds
  const uint32_t j2 = b2 ? static_cast<uint32_t>(__builtin_ctzll(b2)) : 64u;
  const uint32_t lo2 = lo1 + (j2 - 1u) * 8u;  // above(lo2) fails, above(lo2 + 8) holds
  const uint64_t b3 = __ballot(lane >= 1u && lane <= 8u && above(lo2 + lane));
  return lo2 + static_cast<uint32_t>(__builtin_ctzll(b3));
}

// Sum of n float64 partials by one wave: lane j adds partials j, j + 64, ... in
// that order (eight loads in flight), then a fixed butterfly.  Uniform result.
__device__ double sum_partials_wave(const double* p, int n) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (int j0 = lane; j0 < n; j0 += 8 * 64) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j0 + u * 64 < n ? p[j0 + u * 64] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  return wave_sum(s);
}

template <int DT>
__device__ __forceinline__ SegInfo finalize_wave(double s, int64_t n, float eps) {
  SegInfo info;
  if (n == 0) {
    info.gamma = 0.0f;
    info.thresh = 0x8000u;  // no magnitude reaches it: every code 0 (never read)
    return info;
  }
  info.gamma = static_cast<float>(s / static_cast<double>(n));
  const float d = info.gamma + eps;  // float32, as the encoding defines it
  info.thresh = threshold16_wave<DT>(d);
  return info;
}

// 2-bit fields (code + 1) of eight 16-bit inputs, element e at bits 2e.
// u = 1 + nz - 2*nz*neg per 16-bit half: nz = (|x| >= T), neg = sign bit.
__device__ __forceinline__ uint32_t code_word8(uint4 w, uint32_t thresh) {
  const uint32_t add = (0x8000u - thresh) * 0x00010001u;  // halves never carry: <= 0x7FFF + 0x7FFF
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t y = (ws[k] & 0x7FFF7FFFu) + add;
    const uint32_t nz = (y >> 15) & 0x00010001u;
    const uint32_t ng = (ws[k] >> 15) & 0x00010001u;
    const uint32_t u = 0x00010001u + nz - ((nz & ng) << 1);
    out |= ((u | (u >> 14)) & 0xFu) << (4 * k);
  }
  return out;
}

// OCP e4m3fn of a float32, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3fn_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = static_cast<uint32_t>(rintf(a * 512.0f));  // subnormal steps of 2^-9 (8 -> min normal)
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t m3 = (b >> 20) & 7u, rest = b & 0xFFFFFu;
    code = ((((b >> 23) - 120u) << 3) | m3);
    if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) code += 1;  // carry into exponent is right
  }
  return sign | code;
}

template <int DT>
__device__ __forceinline__ uint32_t to_f16_bits(uint32_t h) {
  if (DT == 0) return h;
  return static_cast<uint32_t>(__half_as_ushort(__float2half_rn(to_f32<1>(h))));
}

// ------------------------------------------------------------- pass 1 ---

template <int DT>
__global__ __launch_bounds__(kAbsThreads) void k_absmean_partial(AppendArgs a) {
  const int seg = blockIdx.y, blk = blockIdx.x;
  const int kv = seg & 1, li = seg >> 1;
  const int i = li % a.n_seqs, l_rel = li / a.n_seqs;
  const AppendSeqDesc d = a.descs[i];
  const int64_t row = static_cast<int64_t>(a.P.hkv) * a.P.dim;
  const int64_t n = static_cast<int64_t>(d.tern_hi - d.tern_lo) * row;
  const uint16_t* base =
      (kv ? a.v : a.k) + ((static_cast<int64_t>(l_rel) * a.n_seqs + i) * a.n_tokens + d.tern_lo) * row;
  const int64_t start = static_cast<int64_t>(blk) * kAbsElemsPerBlock;
  uint4 w[kAbsIters];
#pragma unroll
  for (int it = 0; it < kAbsIters; ++it) {
    const int64_t e = start + (static_cast<int64_t>(it) * kAbsThreads + threadIdx.x) * kAbsElemsPerThreadIter;
    w[it] = e < n ? *reinterpret_cast<const uint4*>(base + e) : make_uint4(0, 0, 0, 0);
  }
  double acc = 0.0;
#pragma unroll
  for (int it = 0; it < kAbsIters; ++it) acc += abs_sum8<DT>(w[it]);
  const double total = block_sum256(acc);
  if (threadIdx.x == 0) a.partials[static_cast<int64_t>(seg) * a.n_blk + blk] = total;
}

template <int DT>
__global__ __launch_bounds__(64) void k_gamma_finalize(AppendArgs a) {
  const int seg = blockIdx.x;
  const int i = (seg >> 1) % a.n_seqs;
  const AppendSeqDesc d = a.descs[i];
  const int64_t n = static_cast<int64_t>(d.tern_hi - d.tern_lo) * a.P.hkv * a.P.dim;
  const double s = sum_partials_wave(a.partials + static_cast<int64_t>(seg) * a.n_blk, a.n_blk);
  const SegInfo info = finalize_wave<DT>(s, n, a.eps);
  if (threadIdx.x == 0) a.seg[seg] = info;
}

// ------------------------------------------------------------- pass 2 ---

// MIXED = false: every page of the call is ternary (the fp8 / fp16 routes are left out, which
// keeps the register count, and so the resident waves per SIMD, where the ternary route needs it)
template <int DT, int D, bool MIXED>
__global__ __launch_bounds__(64) void k_pack(AppendArgs a) {
  constexpr int CPR = D / 8;     // 16-byte chunks per token row
  constexpr int RPI = 64 / CPR;  // rows per wave-wide load
  constexpr int NI = 16 / RPI;   // loads per lane per unit
  constexpr int DPL = D / 64;    // head dims per lane in the transposed fp8 / fp16 value stores
  __shared__ uint32_t lds[D * 16 * 2 / 4 + 4];
  uint16_t* lds16 = reinterpret_cast<uint16_t*>(lds);
  uint8_t* lds8 = reinterpret_cast<uint8_t*>(lds);

  const int lane = threadIdx.x;
  const int li = blockIdx.y;
  const int i = li % a.n_seqs, l_rel = li / a.n_seqs;
  const int layer = a.layer_begin + l_rel;
  const AppendSeqDesc d = a.descs[i];
  const int hkv = a.P.hkv;
  const int64_t row = static_cast<int64_t>(hkv) * D;
  const int t1 = d.t0 + a.n_tokens;
  const int n_tasks = a.max_units * 2 * hkv;
  const int c = lane % CPR, rg = lane / CPR;

  // each block takes a contiguous run of tasks: its consecutive tasks are the heads (then K or
  // V) of the same 16 tokens, so a block walks whole input rows instead of one head's slice
  const int per_blk = (n_tasks + gridDim.x - 1) / gridDim.x;
  const int task_end = min(n_tasks, (static_cast<int>(blockIdx.x) + 1) * per_blk);
  for (int task = blockIdx.x * per_blk; task < task_end; ++task) {
    const int h = task % hkv;
    const int kv = (task / hkv) & 1;
    const int uk = task / (2 * hkv);
    const int unit = d.unit_first + uk;
    if (unit * 16 >= t1) continue;  // uniform over the block
    const int pos0 = unit * 16;
    const int page = pos0 >> a.P.bs_shift;
    const int upi = (pos0 & (a.P.bs - 1)) >> 4;
    const int32_t entry = a.entries[d.page_off + page - d.page_first];
    const int fmt = static_cast<int>(static_cast<uint32_t>(entry) >> 30);
    const int64_t idx = entry & 0x3FFFFFFF;
    uint8_t* tile = a.P.pool[fmt] + (static_cast<int64_t>(layer) * a.P.cap[fmt] + idx) * a.P.page_bytes[fmt] +
                    static_cast<int64_t>(kv * hkv + h) * a.P.tile_bytes[fmt];
    const uint16_t* src =
        (kv ? a.v : a.k) + (static_cast<int64_t>(l_rel) * a.n_seqs + i) * a.n_tokens * row + h * D + c * 8;

    if (l_rel == 0 && kv == 0 && h == 0 && lane == 0 && (uk == 0 || upi == 0))
      a.P.block_table[static_cast<int64_t>(d.slot) * a.P.max_pages + page] = entry;

    uint4 w[NI];
    bool ok[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r = rg * NI + k;
      const int j = pos0 + r - d.t0;  // call-relative token
      ok[k] = j >= 0 && j < a.n_tokens;
      w[k] = ok[k] ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * row) : make_uint4(0, 0, 0, 0);
    }

    if (fmt == VK_FMT_TERNARY2) {
      const SegInfo si = a.seg[(l_rel * a.n_seqs + i) * 2 + kv];
      if (upi == 0 && h == 0 && lane == 0)
        a.P.gamma[(static_cast<int64_t>(layer) * a.P.cap[0] + idx) * 2 + kv] = si.gamma;
      if (kv == 0) {
#pragma unroll
        for (int k = 0; k < NI; ++k) {
          const int r = rg * NI + k;
          const uint32_t cw = code_word8(w[k], si.thresh);
          *reinterpret_cast<uint16_t*>(tile + (upi * 16 + r) * (D / 4) + 2 * c) = static_cast<uint16_t>(cw);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NI; ++k) {
          const int r = rg * NI + k;
          lds16[c * 16 + r] = static_cast<uint16_t>(code_word8(w[k], si.thresh));
        }
        __syncthreads();
        // value tile, chunked per 16-token unit: lane = chunk 4*cq + g = tokens 4g..4g+3 of
        // dimensions 16j + cq; LDS rows (4g, 4g+1) and (4g+2, 4g+3) arrive as one dword each
        const int cq = lane >> 2, g = lane & 3;
        const uint32_t* l32 = reinterpret_cast<const uint32_t*>(lds16);
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const int dd = 16 * j + cq;
          const int cc = dd >> 3, e = dd & 7;
          const uint32_t f01 = (l32[cc * 8 + 2 * g] >> (2 * e)) & 0x00030003u;
          const uint32_t f23 = (l32[cc * 8 + 2 * g + 1] >> (2 * e)) & 0x00030003u;
          if (D == 128) {
            w0 |= f01 << (2 * j);
            w1 |= f23 << (2 * j);
          } else {
            w0 |= (f01 << (2 * j)) | (f23 << (8 + 2 * j));
          }
        }
        uint8_t* vdst = tile + upi * 4 * D + lane * (D / 16);
        if (D == 128) *reinterpret_cast<uint2*>(vdst) = make_uint2(w0, w1);
        else *reinterpret_cast<uint32_t*>(vdst) = w0;
        __syncthreads();
      }
    } else if (!MIXED) {
      // (not reached: the host launches this instance only when every page is ternary)
    } else if (fmt == VK_FMT_FP8E4M3) {
      const bool dyn = a.P.fp8_dynamic != 0;
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int r = rg * NI + k;
        const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        float s = a.P.fp8_scale;
        if (dyn) {
          // dynamic FP8: s = float32(max |x| / 448) over the row (the CPR lanes of rg)
          float amax = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(to_f32<DT>((ws[e >> 1] >> (16 * (e & 1))) & 0xFFFFu)));
#pragma unroll
          for (int off = 1; off < CPR; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
          s = amax / 448.0f;
          if (c == 0 && ok[k])
            *reinterpret_cast<float*>(tile + static_cast<int64_t>(a.P.bs) * D + 4 * (upi * 16 + r)) = s;
        }
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = to_f32<DT>((ws[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
          b[e] = dyn ? (s > 0.0f ? e4m3fn_rne(x / s) : 0u) : e4m3fn_rne(s == 1.0f ? x : x / s);
        }
        if (kv == 0) {
          if (ok[k]) {
            uint2 o;
            o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
            o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
            *reinterpret_cast<uint2*>(tile + (upi * 16 + r) * D + 8 * c) = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) lds8[(8 * c + e) * 16 + r] = static_cast<uint8_t>(b[e]);
        }
      }
      if (kv == 1) {
        __syncthreads();
        const bool full = pos0 >= d.t0 && pos0 + 16 <= t1;
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int dd = lane * DPL + j;
          uint8_t* dst = tile + static_cast<int64_t>(dd) * a.P.bs + upi * 16;
          if (full) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(lds8 + dd * 16);
          } else {
            for (int t = 0; t < 16; ++t)
              if (pos0 + t >= d.t0 && pos0 + t < t1) dst[t] = lds8[dd * 16 + t];
          }
        }
        __syncthreads();
      }
    } else {  // VK_FMT_F16
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int r = rg * NI + k;
        const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        uint32_t hb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hb[e] = to_f16_bits<DT>((ws[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        if (kv == 0) {
          if (ok[k]) {
            uint4 o;
            o.x = hb[0] | (hb[1] << 16);
            o.y = hb[2] | (hb[3] << 16);
            o.z = hb[4] | (hb[5] << 16);
            o.w = hb[6] | (hb[7] << 16);
            *reinterpret_cast<uint4*>(tile + ((upi * 16 + r) * D + 8 * c) * 2) = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) lds16[(8 * c + e) * 16 + r] = static_cast<uint16_t>(hb[e]);
        }
      }
      if (kv == 1) {
        __syncthreads();
        const bool full = pos0 >= d.t0 && pos0 + 16 <= t1;
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int dd = lane * DPL + j;
          uint16_t* dst = reinterpret_cast<uint16_t*>(tile) + static_cast<int64_t>(dd) * a.P.bs + upi * 16;
          if (full) {
            const uint4* s4 = reinterpret_cast<const uint4*>(lds16 + dd * 16);
            reinterpret_cast<uint4*>(dst)[0] = s4[0];
            reinterpret_cast<uint4*>(dst)[1] = s4[1];
          } else {
            for (int t = 0; t < 16; ++t)
              if (pos0 + t >= d.t0 && pos0 + t < t1) dst[t] = lds16[dd * 16 + t];
          }
        }
        __syncthreads();
      }
    }
  }
}

// ------------------------------------------------------- flat tensor ---

template <int DT>
__global__ __launch_bounds__(kAbsThreads) void k_flat_absmean(QuantArgs a) {
  const int blk = blockIdx.x;
  const int64_t start = static_cast<int64_t>(blk) * kAbsElemsPerBlock;
  uint4 w[kAbsIters];
#pragma unroll
  for (int it = 0; it < kAbsIters; ++it) {
    const int64_t e = start + (static_cast<int64_t>(it) * kAbsThreads + threadIdx.x) * kAbsElemsPerThreadIter;
    w[it] = e < a.n ? *reinterpret_cast<const uint4*>(a.x + e) : make_uint4(0, 0, 0, 0);
  }
  double acc = 0.0;
#pragma unroll
  for (int it = 0; it < kAbsIters; ++it) acc += abs_sum8<DT>(w[it]);
  const double total = block_sum256(acc);
  if (threadIdx.x == 0) a.partials[blk] = total;
}

template <int DT>
__global__ __launch_bounds__(64) void k_flat_finalize(QuantArgs a) {
  if (a.gamma_in) {
    SegInfo info;
    info.gamma = *a.gamma_in;
    info.thresh = threshold16_wave<DT>(info.gamma + a.eps);
    if (threadIdx.x == 0) {
      a.seg[0] = info;
      *a.gamma_out = info.gamma;
    }
    return;
  }
  const SegInfo info = finalize_wave<DT>(sum_partials_wave(a.partials, a.n_blk), a.n, a.eps);
  if (threadIdx.x == 0) {
    a.seg[0] = info;
    *a.gamma_out = info.gamma;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_flat_pack(QuantArgs a) {
  const uint32_t thresh = a.seg[0].thresh;
  const int64_t n8 = a.n / 8;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < n8;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const uint4 w = reinterpret_cast<const uint4*>(a.x)[g];
    reinterpret_cast<uint16_t*>(a.packed)[g] = static_cast<uint16_t>(code_word8(w, thresh));
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int32_t n_seg, hipStream_t s, LaunchTimer* t) {
  const bool bf = a.dtype == VK_DTYPE_BF16;
  if (a.n_blk > 0) {
    const dim3 g1(a.n_blk, n_seg);
    if (t) t->begin(VK_KERNEL_ABSMEAN, s);
    if (bf) k_absmean_partial<1><<<g1, kAbsThreads, 0, s>>>(a);
    else k_absmean_partial<0><<<g1, kAbsThreads, 0, s>>>(a);
    if (t) t->end(VK_KERNEL_ABSMEAN, s);
    if (t) t->begin(VK_KERNEL_FINALIZE, s);
    if (bf) k_gamma_finalize<1><<<n_seg, 64, 0, s>>>(a);
    else k_gamma_finalize<0><<<n_seg, 64, 0, s>>>(a);
    if (t) t->end(VK_KERNEL_FINALIZE, s);
  }
  // enough one-wave blocks to keep every SIMD busy (about 16 per CU), at most one per task
  const int n_tasks = a.max_units * 2 * a.P.hkv;
  const int gy = a.n_layers * a.n_seqs;
  const int gx_max = gy < 16 ? 16384 / gy : 1024;
  const dim3 g2(n_tasks < gx_max ? n_tasks : gx_max, gy);
  if (t) t->begin(VK_KERNEL_PACK, s);
  if (a.P.dim == 128 && a.all_ternary) {
    if (bf) k_pack<1, 128, false><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 128, false><<<g2, 64, 0, s>>>(a);
  } else if (a.P.dim == 128) {
    if (bf) k_pack<1, 128, true><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 128, true><<<g2, 64, 0, s>>>(a);
  } else if (a.all_ternary) {
    if (bf) k_pack<1, 64, false><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 64, false><<<g2, 64, 0, s>>>(a);
  } else {
    if (bf) k_pack<1, 64, true><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 64, true><<<g2, 64, 0, s>>>(a);
  }
  if (t) t->end(VK_KERNEL_PACK, s);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const bool bf = a.dtype == VK_DTYPE_BF16;
  if (!a.gamma_in) {
    if (bf) k_flat_absmean<1><<<a.n_blk, kAbsThreads, 0, s>>>(a);
    else k_flat_absmean<0><<<a.n_blk, kAbsThreads, 0, s>>>(a);
  }
  if (bf) k_flat_finalize<1><<<1, 64, 0, s>>>(a);
  else k_flat_finalize<0><<<1, 64, 0, s>>>(a);
  int64_t blocks = (a.n / 8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (bf) k_flat_pack<1><<<static_cast<unsigned>(blocks), 256, 0, s>>>(a);
  else k_flat_pack<0><<<static_cast<unsigned>(blocks), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace vk
