// Write side: per-tensor absmean scale, ternary quantisation, 2-bit packing
// and page scatter, for gfx950.
//
// Follows "Show HN: Vantage-V-AI" (newshot.cc), section "core architecture":
// gamma = mean(|X|) per tensor, states {-1, 0, +1}, four elements per uint8.
// FP8 recent pages and FP16 anchor (sink) pages follow "Minima-KV"
// (twodots.gr), section "Recent, Anchor and Stale".
//
// Two kernels per append call:
//   k_absmean_partial  pass 1: fixed-partition float64 sums of |x|, one per
//                      (segment, 32 KiB block), no atomics -> deterministic
//   k_pack             pass 2: one wave per (16-token unit, K|V, head) tile;
//                      the segment's gamma = fp32(S/N) from a fixed-order sum of
//                      its partials and the exact 16-bit magnitude threshold of a
//                      nonzero code, derived by every wave that needs them;
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

#include <mutex>

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

// Index of the sequence whose range [off_i, off_{i+1}) holds x, for per-sequence offsets that
// do not decrease with i (FIELD: a member of AppendSeqDesc): one load per lane and a ballot per
// 64 sequences.  Every lane of the wave calls it; the result is uniform.
template <int32_t AppendSeqDesc::*FIELD>
__device__ __forceinline__ int find_seq(const AppendSeqDesc* descs, int n_seqs, int x) {
  const int lane = threadIdx.x & 63;
  int i = 0;
  for (int j0 = 0; j0 < n_seqs; j0 += 64) {
    const int j = j0 + lane;
    const uint64_t le = __ballot(j < n_seqs && descs[j].*FIELD <= x);
    i += __builtin_popcountll(le);
    if (le != ~uint64_t{0}) break;
  }
  return i - 1;
}

// ------------------------------------------------------------- pass 1 ---

// grid (absmean blocks of every sequence, layer x K|V): the sequences' blocks one after another,
// so a ragged call (sequences of different token counts) launches no idle blocks
template <int DT>
__global__ __launch_bounds__(kAbsThreads) void k_absmean_partial(AppendArgs a) {
  static_assert(kAbsElemsPerBlock == kAbsBlockElems, "block size shared with the host planner");
  const int x = blockIdx.x;
  const int kv = blockIdx.y & 1, l_rel = blockIdx.y >> 1;
  // (a call whose sequences all have the same block count finds its sequence without a load)
  const int i = a.seq_blk ? x / a.seq_blk : find_seq<&AppendSeqDesc::blk_off>(a.descs, a.n_seqs, x);
  const AppendSeqDesc d = a.descs[i];
  const int blk = x - d.blk_off;
  const int64_t row = static_cast<int64_t>(a.P.hkv) * a.P.dim;
  const int64_t n = static_cast<int64_t>(d.tern_hi - d.tern_lo) * row;
  const uint16_t* base =
      (kv ? a.v : a.k) + (static_cast<int64_t>(l_rel) * a.total_tokens + d.tok_off + d.tern_lo) * row;
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
  if (threadIdx.x == 0) a.partials[static_cast<int64_t>(blockIdx.y) * a.total_blk + x] = total;
}

// gamma and threshold of a segment (layer, sequence, K|V), by one wave: its partials are blocks
// [blk_off, blk_off + n) of its (layer, K|V) row.  Every pack wave that codes a tile of the
// segment derives them itself, with the same fixed-order sum, so all agree bit for bit (the
// partials of a call are a few KB, read from L2): no finalize launch between the two passes.
template <int DT>
__device__ __forceinline__ SegInfo segment_info_n(const AppendArgs& a, int64_t n, int blk_off, int l_rel, int kv) {
  const int n_blk = static_cast<int>((n + kAbsElemsPerBlock - 1) / kAbsElemsPerBlock);
  const double s = sum_partials_wave(a.partials + static_cast<int64_t>(l_rel * 2 + kv) * a.total_blk + blk_off, n_blk);
  return finalize_wave<DT>(s, n, a.eps);
}

template <int DT>
__device__ __forceinline__ SegInfo segment_info(const AppendArgs& a, const AppendSeqDesc& d, int l_rel, int kv) {
  const int64_t n = static_cast<int64_t>(d.tern_hi - d.tern_lo) * a.P.hkv * a.P.dim;
  const int n_blk = static_cast<int>((n + kAbsElemsPerBlock - 1) / kAbsElemsPerBlock);
  const double s = sum_partials_wave(a.partials + static_cast<int64_t>(l_rel * 2 + kv) * a.total_blk + d.blk_off, n_blk);
  return finalize_wave<DT>(s, n, a.eps);
}

// Codes of one (16-token unit, K|V, head) tile from this lane's input words w (rows rg * NI + k,
// 16-byte chunk c of the row), stored in the page layout: keys token-major (16-bit stores of
// eight codes), values through an LDS transpose into the decode's chunks (lane = chunk
// 4 cq + g = tokens 4g..4g+3 of dimensions 16j + cq; LDS rows (4g, 4g+1) and (4g+2, 4g+3)
// arrive as one dword each; head dim 256 keeps two head-dim-128 chunks side by side).  One
// wave; the value path holds two barriers, so every lane of the block calls it.
template <int D>
__device__ __forceinline__ void store_ternary_tile(const uint4 (&w)[16 / (64 / (D / 8))], uint32_t thresh, uint8_t* tile,
                                                   int upi, int kv, uint16_t* lds16) {
  constexpr int CPR = D / 8, NI = 16 / (64 / CPR);
  const int lane = threadIdx.x, c = lane % CPR, rg = lane / CPR;
  if (kv == 0) {
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r = rg * NI + k;
      const uint32_t cw = code_word8(w[k], thresh);
      *reinterpret_cast<uint16_t*>(tile + (upi * 16 + r) * (D / 4) + 2 * c) = static_cast<uint16_t>(cw);
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int r = rg * NI + k;
    lds16[c * 16 + r] = static_cast<uint16_t>(code_word8(w[k], thresh));
  }
  __syncthreads();
  const int cq = lane >> 2, g = lane & 3;
  const uint32_t* l32 = reinterpret_cast<const uint32_t*>(lds16);
  uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const int dd = 16 * j + cq;
    const int cc = dd >> 3, e = dd & 7;
    const uint32_t f01 = (l32[cc * 8 + 2 * g] >> (2 * e)) & 0x00030003u;
    const uint32_t f23 = (l32[cc * 8 + 2 * g + 1] >> (2 * e)) & 0x00030003u;
    if (D == 64) {
      w0 |= (f01 << (2 * j)) | (f23 << (8 + 2 * j));
    } else if (j < 8) {
      w0 |= f01 << (2 * j);
      w1 |= f23 << (2 * j);
    } else {
      w2 |= f01 << (2 * (j - 8));
      w3 |= f23 << (2 * (j - 8));
    }
  }
  uint8_t* vdst = tile + upi * 4 * D + lane * (D / 16);
  if (D == 256) *reinterpret_cast<uint4*>(vdst) = make_uint4(w0, w1, w2, w3);
  else if (D == 128) *reinterpret_cast<uint2*>(vdst) = make_uint2(w0, w1);
  else *reinterpret_cast<uint32_t*>(vdst) = w0;
  __syncthreads();
}

// ------------------------------------------------------------- pass 2 ---

// Tasks are (16-token unit, K|V, KV head) of every sequence of the call, the sequences' tasks
// one after another within a layer, layer after layer; each block takes a contiguous run of
// tasks_per_blk of them, so its consecutive tasks are the heads (then K or V) of the same 16
// tokens and it walks whole input rows.
// MODE 0: every page of the call is ternary (the other routes are left out, which keeps the
// register count, and so the resident waves per SIMD, where the ternary route needs it);
// MODE 1: ternary, fp8 and fp16 pages; MODE 2: a list of lossless units; MODE 3: a list of fp8 /
// fp16 units (a call that holds some runs MODE 0 over every task, which skips them and keeps the
// ternary route's register count, then MODE 3 over them).
template <int DT, int D, int MODE>
__global__ __launch_bounds__(64) void k_pack(AppendArgs a) {
  constexpr int CPR = D / 8;     // 16-byte chunks per token row
  constexpr int RPI = 64 / CPR;  // rows per wave-wide load
  constexpr int NI = 16 / RPI;   // loads per lane per unit
  constexpr int DPL = D / 64;    // head dims per lane in the transposed fp8 / fp16 value stores
  __shared__ uint32_t lds[D * 16 * 2 / 4 + 4];
  __shared__ uint32_t lds_bm[MODE == 2 ? 64 : 1], lds_off[MODE == 2 ? 64 : 1];  // lossless exceptions
  uint16_t* lds16 = reinterpret_cast<uint16_t*>(lds);
  uint8_t* lds8 = reinterpret_cast<uint8_t*>(lds);

  const int lane = threadIdx.x;
  const int hkv = a.P.hkv;
  const int64_t row = static_cast<int64_t>(hkv) * D;
  const int c = lane % CPR, rg = lane / CPR;

  // MODES 2 and 3 run over a list of (sequence index, unit) pairs, one task per block
  constexpr bool LIST = MODE >= 2;
  const int32_t* list = MODE == 2 ? a.ll_units : a.ot_units;
  const int n_list = MODE == 2 ? a.n_ll_units : a.n_ot_units;
  const int64_t g_end = static_cast<int64_t>(a.n_layers) * (LIST ? 2LL * hkv * n_list : a.total_tasks);
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * (LIST ? 1 : a.tasks_per_blk);
  const int64_t g1 = LIST ? g0 + 1 : (g0 + a.tasks_per_blk < g_end ? g0 + a.tasks_per_blk : g_end);
  int i = -1, l_rel = -1, task_end = 0;
  AppendSeqDesc d{};
  SegInfo seg_k{}, seg_v{};  // the current (layer, sequence)'s records, derived when first needed
  bool have_k = false, have_v = false;
  for (int64_t g = g0; g < g1; ++g) {
    int h, kv, uk;
    if constexpr (LIST) {
      const int64_t per_layer = 2LL * hkv * n_list;
      l_rel = static_cast<int>(g / per_layer);
      const int r = static_cast<int>(g - static_cast<int64_t>(l_rel) * per_layer);
      const int lu = r / (2 * hkv);
      h = r % hkv;
      kv = (r / hkv) & 1;
      i = list[2 * lu];
      d = a.descs[i];
      uk = list[2 * lu + 1] - d.unit_first;
    } else {
      const int lr = static_cast<int>(g / a.total_tasks);
      const int t = static_cast<int>(g - static_cast<int64_t>(lr) * a.total_tasks);
      if (lr != l_rel || t >= task_end) {  // uniform: the block moves on to another sequence
        l_rel = lr;
        i = a.seq_tasks ? t / a.seq_tasks : find_seq<&AppendSeqDesc::task_off>(a.descs, a.n_seqs, t);
        d = a.descs[i];
        task_end = d.task_off + ((d.t0 + d.n_tokens + 15) / 16 - d.unit_first) * 2 * hkv;
        have_k = have_v = false;
      }
      const int task = t - d.task_off;
      h = task % hkv;
      kv = (task / hkv) & 1;
      uk = task / (2 * hkv);
    }
    const int layer = a.layer_begin + l_rel;
    const int t1 = d.t0 + d.n_tokens;
    const int unit = d.unit_first + uk;
    if (unit * 16 >= t1) continue;  // uniform over the block
    const int pos0 = unit * 16;
    const int page = pos0 >> a.P.bs_shift;
    const int upi = (pos0 & (a.P.bs - 1)) >> 4;
    // The block-table entry, the input tile and (MODE 0: every page ternary or lossless) the
    // segment's absmean partials are loaded before anything waits for one of them: each needs
    // only the sequence's descriptor.
    const int32_t entry = a.entries[d.page_off + page - d.page_first];
    const uint16_t* src =
        (kv ? a.v : a.k) + (static_cast<int64_t>(l_rel) * a.total_tokens + d.tok_off) * row + h * D + c * 8;
    uint4 w[NI];
    bool ok[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r = rg * NI + k;
      const int j = pos0 + r - d.t0;  // call-relative token
      ok[k] = j >= 0 && j < d.n_tokens;
      w[k] = ok[k] ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * row) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (MODE == 0) {  // (a lossless unit derives the record too; it is not used)
      if (kv == 0 && !have_k) {
        seg_k = segment_info<DT>(a, d, l_rel, 0);
        have_k = true;
      }
      if (kv == 1 && !have_v) {
        seg_v = segment_info<DT>(a, d, l_rel, 1);
        have_v = true;
      }
    }
    const int fmt = static_cast<int>(static_cast<uint32_t>(entry) >> 30);
    const int64_t idx = entry & 0x3FFFFFFF;
    uint8_t* tile = a.P.pool[fmt] + (static_cast<int64_t>(layer) * a.P.cap[fmt] + idx) * a.P.page_bytes[fmt] +
                    static_cast<int64_t>(kv * hkv + h) * a.P.tile_bytes[fmt];

    if (!LIST && l_rel == 0 && kv == 0 && h == 0 && lane == 0 && (uk == 0 || upi == 0))
      a.P.block_table[static_cast<int64_t>(d.slot) * a.P.max_pages + page] = entry;
    if (!LIST && fmt == VK_FMT_LOSSLESS) continue;  // written by the launch over the lossless units

    if (!LIST && fmt == VK_FMT_TERNARY2) {
      if (kv == 0 && !have_k) {
        seg_k = segment_info<DT>(a, d, l_rel, 0);
        have_k = true;
      }
      if (kv == 1 && !have_v) {
        seg_v = segment_info<DT>(a, d, l_rel, 1);
        have_v = true;
      }
      const SegInfo si = kv == 0 ? seg_k : seg_v;
      if (upi == 0 && h == 0 && lane == 0)
        a.P.gamma[(static_cast<int64_t>(layer) * a.P.cap[0] + idx) * 2 + kv] = si.gamma;
      store_ternary_tile<D>(w, si.thresh, tile, upi, kv, lds16);
    } else if (MODE == 0) {
      // fp8 / fp16 units: written by the MODE 3 launch over their list
    } else if ((MODE == 1 || MODE == 3) && fmt == VK_FMT_FP8E4M3) {
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
        // dimension j * 64 + lane: each store instruction writes 64 consecutive 16-byte rows
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int dd = j * 64 + lane;
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
    } else if (MODE == 2) {  // the list holds lossless units only
      // One group: the 16 tokens of this unit, head h, K or V (bfloat16 input).  Exponent
      // fields around the group's centre c = floor(mean of the nonzero fields) as 4-bit codes
      // (15 = escape), a sign+mantissa byte per value, and the escaped fields in decode-lane
      // order; raw values when more than 8 D fields escape.  Slot: [16-byte header][...].
      // Fields are taken from the input words w[] whenever they are needed (no copies held).
      uint8_t* slot = tile + static_cast<int64_t>(upi) * (32 * D + 16);
      auto half = [&](int q) -> uint32_t {  // value q of this lane: row rg * NI + q / 8, dim 8 c + q % 8
        const uint4 x = w[q >> 3];
        const int e = q & 7;
        const uint32_t wd = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
        return (wd >> (16 * (e & 1))) & 0xFFFFu;
      };
      auto field = [&](int q) { return (half(q) >> 7) & 0xFFu; };
      // the fields are recomputed from w[] in every phase below: an empty asm that "changes" w[]
      // keeps the compiler from holding each phase's per-value results (3 x 8 NI registers)
      auto launder = [&]() {
#pragma unroll
        for (int k = 0; k < NI; ++k) asm volatile("" : "+v"(w[k].x), "+v"(w[k].y), "+v"(w[k].z), "+v"(w[k].w));
      };
      uint32_t esum = 0, ecnt = 0;
#pragma unroll
      for (int q = 0; q < 8 * NI; ++q) {
        const uint32_t f = field(q);
        esum += f;
        ecnt += f != 0u;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        esum += __shfl_xor(esum, off, 64);
        ecnt += __shfl_xor(ecnt, off, 64);
      }
      const int cen = __builtin_amdgcn_readfirstlane(ecnt ? static_cast<int>(esum / ecnt) : 0);
      auto code = [&](int q) -> uint32_t {
        const int ee = static_cast<int>(field(q));
        return (ee >= cen - 11 && ee <= cen + 3) ? static_cast<uint32_t>(ee - cen + 11) : 15u;
      };
      auto smb = [&](int q) { const uint32_t hx = half(q); return ((hx >> 8) & 0x80u) | (hx & 0x7Fu); };
      launder();
      int n_exc = 0;
#pragma unroll
      for (int q = 0; q < 8 * NI; ++q) n_exc += code(q) == 15u;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) n_exc += __shfl_xor(n_exc, off, 64);
      n_exc = __builtin_amdgcn_readfirstlane(n_exc);
      const bool raw = n_exc > 8 * D;
      if (lane == 0) {
        *reinterpret_cast<uint4*>(slot) = make_uint4(static_cast<uint32_t>(cen) | (raw ? 0x100u : 0u),
                                                     raw ? 0u : static_cast<uint32_t>(n_exc), 0u, 0u);
      }
      uint8_t* body = slot + 16;
      launder();
      if (raw) {
        if (kv == 0) {
#pragma unroll
          for (int k = 0; k < NI; ++k)
            *reinterpret_cast<uint4*>(body + ((rg * NI + k) * D + 8 * c) * 2) = w[k];
        } else {
#pragma unroll
          for (int q = 0; q < 8 * NI; ++q) lds16[(8 * c + q % 8) * 16 + rg * NI + q / 8] = static_cast<uint16_t>(half(q));
          __syncthreads();
#pragma unroll
          for (int j = 0; j < DPL; ++j) {
            const int dd = lane * DPL + j;
            const uint4* s4 = reinterpret_cast<const uint4*>(lds16 + dd * 16);
            reinterpret_cast<uint4*>(body + dd * 32)[0] = s4[0];
            reinterpret_cast<uint4*>(body + dd * 32)[1] = s4[1];
          }
          __syncthreads();
        }
      } else {
        // sign+mantissa bytes and codes in the stored order (keys token-major, values
        // dimension-major, codes two per byte, element 2i in the low nibble of byte i)
        uint8_t* codes = body + 16 * D;
        if (kv == 0) {
#pragma unroll
          for (int k = 0; k < NI; ++k) {
            const int r = rg * NI + k;
            uint32_t lo = 0, hi = 0, nib = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lo |= smb(8 * k + e) << (8 * e);
              hi |= smb(8 * k + 4 + e) << (8 * e);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) nib |= code(8 * k + e) << (4 * e);
            *reinterpret_cast<uint2*>(body + r * D + 8 * c) = make_uint2(lo, hi);
            *reinterpret_cast<uint32_t*>(codes + (r * D + 8 * c) / 2) = nib;
          }
        } else {
          uint8_t* lsm = lds8;            // [D][16] sign+mantissa bytes
          uint8_t* lcd = lds8 + 16 * D;   // [D][16] codes, one per byte
#pragma unroll
          for (int q = 0; q < 8 * NI; ++q) {
            const int at = (8 * c + q % 8) * 16 + rg * NI + q / 8;
            lsm[at] = static_cast<uint8_t>(smb(q));
            lcd[at] = static_cast<uint8_t>(code(q));
          }
          __syncthreads();
#pragma unroll
          for (int j = 0; j < DPL; ++j) {
            const int dd = lane * DPL + j;
            *reinterpret_cast<uint4*>(body + dd * 16) = *reinterpret_cast<const uint4*>(lsm + dd * 16);
            const uint4 q4 = *reinterpret_cast<const uint4*>(lcd + dd * 16);   // codes of tokens 0..15
            const uint32_t qs[4] = {q4.x, q4.y, q4.z, q4.w};
            uint32_t pk[2] = {0u, 0u};
#pragma unroll
            for (int t = 0; t < 16; ++t) pk[t >> 3] |= ((qs[t >> 2] >> (8 * (t & 3))) & 0xFu) << (4 * (t & 7));
            *reinterpret_cast<uint2*>(codes + dd * 8) = make_uint2(pk[0], pk[1]);
          }
          __syncthreads();
        }
        if (n_exc > 0) {
          // exceptions in decode-lane order: keys lane = (d / (D/4)) * 16 + t, position d % (D/4);
          // values lane = (t / 4) * 16 + d % 16, position (d / 16) * 4 + t % 4
          auto lane_pos = [&](int q, int& L, int& pos) {
            const int t = rg * NI + q / 8, d = 8 * c + q % 8;
            L = kv == 0 ? (d / (D / 4)) * 16 + t : (t / 4) * 16 + (d % 16);
            pos = kv == 0 ? d % (D / 4) : (d / 16) * 4 + (t % 4);
          };
          lds_bm[lane] = 0u;
          __syncthreads();
          launder();
#pragma unroll
          for (int q = 0; q < 8 * NI; ++q) {
            if (code(q) != 15u) continue;
            int L, pos;
            lane_pos(q, L, pos);
            atomicOr(&lds_bm[L], 1u << pos);
          }
          __syncthreads();
          // exclusive prefix of the lanes' escape counts
          const int cnt = __builtin_popcount(lds_bm[lane]);
          int incl = cnt;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
          }
          lds_off[lane] = static_cast<uint32_t>(incl - cnt);
          __syncthreads();
          launder();
          uint8_t* exc = codes + 8 * D;
#pragma unroll
          for (int q = 0; q < 8 * NI; ++q) {
            if (code(q) != 15u) continue;
            int L, pos;
            lane_pos(q, L, pos);
            const uint32_t rank = lds_off[L] + __builtin_popcount(lds_bm[L] & ((1u << pos) - 1u));
            exc[rank] = static_cast<uint8_t>(field(q));
          }
          __syncthreads();
        }
      }
    } else if (MODE == 1 || MODE == 3) {  // VK_FMT_F16
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
        // 16-byte piece k * 64 + lane (dimension p / 2, tokens 8 (p % 2) .. + 7): each store
        // instruction writes 64 consecutive pieces
#pragma unroll
        for (int k = 0; k < 2 * DPL; ++k) {
          const int p = k * 64 + lane;
          const int dd = p >> 1, th = (p & 1) * 8;
          uint16_t* dst = reinterpret_cast<uint16_t*>(tile) + static_cast<int64_t>(dd) * a.P.bs + upi * 16 + th;
          if (full) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(lds16 + dd * 16 + th);
          } else {
            for (int t = 0; t < 8; ++t)
              if (pos0 + th + t >= d.t0 && pos0 + th + t < t1) dst[t] = lds16[dd * 16 + th + t];
          }
        }
        __syncthreads();
      }
    }
  }
}

// ------------------------------------------------------- flat tensor ---

// All-ternary appends at head dims 64 and 128 (every touched page ternary): the tasks of
// k_pack, but a block's run of tasks is pipelined: the next task's block-table entry and input
// tile are loaded before the current one is coded and stored, so a block streams its run
// instead of paying a loaded-memory round trip per task.  Launched with about as many blocks
// as fit the GPU at once (short appends then run in one round).  Appends into partly filled
// ternary pages are refused on the host, so a task's unit starts at or after the call's first
// token.
template <int DT, int D>
__global__ __launch_bounds__(64) void k_pack_tern(AppendArgs a) {
  constexpr int CPR = D / 8;     // 16-byte chunks per token row
  constexpr int RPI = 64 / CPR;  // rows per wave-wide load
  constexpr int NI = 16 / RPI;   // loads per lane per unit
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
  __shared__ uint32_t lds[D * 16 * 2 / 4 + 4];
  uint16_t* lds16 = reinterpret_cast<uint16_t*>(lds);
  const int lane = threadIdx.x;
  const int hkv = a.P.hkv;
  const int64_t row = static_cast<int64_t>(hkv) * D;
  const int c = lane % CPR, rg = lane / CPR;
  const int64_t g_end = static_cast<int64_t>(a.n_layers) * a.total_tasks;
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * a.tasks_per_blk;
  const int64_t g1 = g0 + a.tasks_per_blk < g_end ? g0 + a.tasks_per_blk : g_end;
  if (g0 >= g1) return;  // (uniform)

  // What one task needs once its loads are out (uniform except src).
  struct Task {
    int l_rel, seq, h, kv, uk, upi, page, slot, rows, blk_off;
    int64_t seg_n;          // elements of the task's segment (its sequence's ternary tokens x heads x D)
    const int32_t* ent_p;   // its block-table entry in the call's entry list
    const uint16_t* src;    // this lane's chunk of the unit's first row
  };
  // the sequence the block's decoding has reached (tasks are decoded in increasing order)
  int cur_l = -1, cur_i = 0, task_end = 0;
  AppendSeqDesc d{};
  auto decode_task = [&](int64_t g) -> Task {
    const int lr = static_cast<int>(g / a.total_tasks);
    const int tt = static_cast<int>(g - static_cast<int64_t>(lr) * a.total_tasks);
    if (lr != cur_l || tt >= task_end) {
      cur_l = lr;
      cur_i = a.seq_tasks ? tt / a.seq_tasks : find_seq<&AppendSeqDesc::task_off>(a.descs, a.n_seqs, tt);
      d = a.descs[cur_i];
      task_end = d.task_off + ((d.t0 + d.n_tokens + 15) / 16 - d.unit_first) * 2 * hkv;
    }
    Task t;
    const int task = tt - d.task_off;
    t.l_rel = lr;
    t.seq = cur_i;
    t.h = task % hkv;
    t.kv = (task / hkv) & 1;
    t.uk = task / (2 * hkv);
    const int pos0 = (d.unit_first + t.uk) * 16;
    t.page = pos0 >> a.P.bs_shift;
    t.upi = (pos0 & (a.P.bs - 1)) >> 4;
    t.slot = d.slot;
    t.rows = d.t0 + d.n_tokens - pos0;  // (>= 1: every task's unit holds tokens of the call)
    t.blk_off = d.blk_off;
    t.seg_n = static_cast<int64_t>(d.tern_hi - d.tern_lo) * hkv * D;
    t.ent_p = a.entries + (d.page_off + t.page - d.page_first);
    t.src = (t.kv ? a.v : a.k) + (static_cast<int64_t>(lr) * a.total_tokens + d.tok_off + (pos0 - d.t0)) * row +
            t.h * D + c * 8;
    return t;
  };
  auto load = [&](const Task& t, uint4 (&w)[NI], int32_t& ent) {
    ent = *t.ent_p;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r = rg * NI + k;
      w[k] = r < t.rows ? *reinterpret_cast<const uint4*>(t.src + static_cast<int64_t>(r) * row) : make_uint4(0, 0, 0, 0);
    }
  };
  // the segment records (gamma, code threshold) of the (layer, sequence) last coded
  int seg_l = -1, seg_i = -1;
  SegInfo seg_k{}, seg_v{};
  bool have_k = false, have_v = false;
  auto process = [&](const Task& t, const uint4 (&w)[NI], int32_t ent) {
    const int64_t layer = a.layer_begin + t.l_rel;
    const int64_t idx = ent & 0x3FFFFFFF;
    uint8_t* tile = a.P.pool[0] + (layer * a.P.cap[0] + idx) * a.P.page_bytes[0] +
                    static_cast<int64_t>(t.kv * hkv + t.h) * a.P.tile_bytes[0];
    if (t.l_rel == 0 && t.kv == 0 && t.h == 0 && lane == 0 && (t.uk == 0 || t.upi == 0))
      a.P.block_table[static_cast<int64_t>(t.slot) * a.P.max_pages + t.page] = ent;
    if (t.l_rel != seg_l || t.seq != seg_i) {
      seg_l = t.l_rel;
      seg_i = t.seq;
      have_k = have_v = false;
    }
    if (t.kv == 0 && !have_k) {
      seg_k = segment_info_n<DT>(a, t.seg_n, t.blk_off, t.l_rel, 0);
      have_k = true;
    }
    if (t.kv == 1 && !have_v) {
      seg_v = segment_info_n<DT>(a, t.seg_n, t.blk_off, t.l_rel, 1);
      have_v = true;
    }
    const SegInfo si = t.kv == 0 ? seg_k : seg_v;
    if (t.upi == 0 && t.h == 0 && lane == 0) a.P.gamma[(layer * a.P.cap[0] + idx) * 2 + t.kv] = si.gamma;
    store_ternary_tile<D>(w, si.thresh, tile, t.upi, t.kv, lds16);
  };

  // Two tasks in flight: while one buffer's task is coded, the other buffer's loads land.  An
  // index past the run repeats its last task (loaded, never processed), so every iteration
  // issues the same loads.
  Task ta = decode_task(g0);
  uint4 wa[NI], wb[NI];
  int32_t ea, eb;
  load(ta, wa, ea);
  for (int64_t g = g0; g < g1; g += 2) {
    const Task tb = decode_task(g + 1 < g1 ? g + 1 : g1 - 1);
    load(tb, wb, eb);
    process(ta, wa, ea);
    ta = decode_task(g + 2 < g1 ? g + 2 : g1 - 1);
    load(ta, wa, ea);
    if (g + 1 < g1) process(tb, wb, eb);
  }
}

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

hipError_t launch_append(const AppendArgs& a, hipStream_t s, LaunchTimer* t) {
  const bool bf = a.dtype == VK_DTYPE_BF16;
  if (a.total_blk > 0) {
    const dim3 g1(a.total_blk, 2 * a.n_layers);
    if (t) t->begin(VK_KERNEL_ABSMEAN, s);
    if (bf) k_absmean_partial<1><<<g1, kAbsThreads, 0, s>>>(a);
    else k_absmean_partial<0><<<g1, kAbsThreads, 0, s>>>(a);
    if (t) t->end(VK_KERNEL_ABSMEAN, s);
  }
  const dim3 g2(a.pack_blocks);
  if (t) t->begin(VK_KERNEL_PACK, s);
  // the lean instance (MODE 0) when every page is ternary or lossless, or when the fp8 / fp16
  // units go to a launch of their own over their list
  const bool lean = a.all_ternary || a.n_ot_units > 0;
  if (a.pack_pipelined && (a.P.dim == 128 || a.P.dim == 64)) {  // every page ternary (set on the host)
    if (a.P.dim == 128) {
      if (bf) k_pack_tern<1, 128><<<g2, 64, 0, s>>>(a);
      else k_pack_tern<0, 128><<<g2, 64, 0, s>>>(a);
    } else {
      if (bf) k_pack_tern<1, 64><<<g2, 64, 0, s>>>(a);
      else k_pack_tern<0, 64><<<g2, 64, 0, s>>>(a);
    }
  } else if (a.P.dim == 256) {  // (no lossless pages at head dim 256: refused on the host)
    if (lean) {
      if (bf) k_pack<1, 256, 0><<<g2, 64, 0, s>>>(a);
      else k_pack<0, 256, 0><<<g2, 64, 0, s>>>(a);
    } else {
      if (bf) k_pack<1, 256, 1><<<g2, 64, 0, s>>>(a);
      else k_pack<0, 256, 1><<<g2, 64, 0, s>>>(a);
    }
  } else if (a.P.dim == 128 && lean) {
    if (bf) k_pack<1, 128, 0><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 128, 0><<<g2, 64, 0, s>>>(a);
  } else if (a.P.dim == 128) {
    if (bf) k_pack<1, 128, 1><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 128, 1><<<g2, 64, 0, s>>>(a);
  } else if (lean) {
    if (bf) k_pack<1, 64, 0><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 64, 0><<<g2, 64, 0, s>>>(a);
  } else {
    if (bf) k_pack<1, 64, 1><<<g2, 64, 0, s>>>(a);
    else k_pack<0, 64, 1><<<g2, 64, 0, s>>>(a);
  }
  // the fp8 / fp16 units: one block per (layer, unit, K|V, head), after the main launch, which
  // writes their block-table entries
  if (a.n_ot_units > 0) {
    const dim3 g4(static_cast<unsigned>(2LL * a.P.hkv * a.n_ot_units * a.n_layers));
    if (a.P.dim == 256) {
      if (bf) k_pack<1, 256, 3><<<g4, 64, 0, s>>>(a);
      else k_pack<0, 256, 3><<<g4, 64, 0, s>>>(a);
    } else if (a.P.dim == 128) {
      if (bf) k_pack<1, 128, 3><<<g4, 64, 0, s>>>(a);
      else k_pack<0, 128, 3><<<g4, 64, 0, s>>>(a);
    } else {
      if (bf) k_pack<1, 64, 3><<<g4, 64, 0, s>>>(a);
      else k_pack<0, 64, 3><<<g4, 64, 0, s>>>(a);
    }
  }
  // the lossless units: one block per (layer, unit, K|V, head); bfloat16 input only (checked on
  // the host)
  if (a.n_ll_units > 0 && a.P.dim != 256) {
    const dim3 g3(static_cast<unsigned>(2LL * a.P.hkv * a.n_ll_units * a.n_layers));
    if (a.P.dim == 128) k_pack<1, 128, 2><<<g3, 64, 0, s>>>(a);
    else k_pack<1, 64, 2><<<g3, 64, 0, s>>>(a);
  }
  if (t) t->end(VK_KERNEL_PACK, s);
  return hipGetLastError();
}

// Scratch of the allocation-free flat entry point: the finalize record (256 bytes) and the
// absmean partials (8 bytes per 16384-element block) of one tensor of at most
// kQuantNoAllocMaxElems elements.  Every device the library runs on holds one copy, and every
// call on that device shares it.
static __device__ __align__(256) uint8_t scratch[kQuantNoAllocScratchBytes];

hipError_t quantize_noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the array's name is a host-side stand-in: its device address is looked up once per
    // device, with that device current, and only that address is handed to kernels
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
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
