// Fused bitmask-apply + sampler for gfx950: one token per row.
//
// What it computes (logits-processor page, "Ops: sample" and "How it
// works"): per-row temperature; top-k, top-p and min-p each keep the
// largest-probability tokens above a cutoff, so their intersection is one
// threshold; temperature <= 0 is greedy; the draw is a Gumbel-max over the
// kept set with variates from a counter-based generator keyed by (seed, row,
// offset).  The packed allow-mask folds into the reads: a token is a
// candidate only when its bit is set (bit v % 32 of word v / 32, Modular MAX
// "apply_packed_bitmask"), it lies below the vocab size and its logit is
// finite -- so a masked token is never drawn.  The logits are only read.
//
// One block of 1024 threads (16 wave64s) per row.  Each pass walks the row
// in groups of 4 consecutive tokens per thread (one generator call serves a
// group); trip counts are uniform across the block so wave-wide shuffles and
// ballots always see every lane.
//
//   pass 1   max logit and its (lowest) index, count of candidate tokens
//            -> greedy rows and rows with no candidate end here;
//   top-k    4 radix passes over an order-preserving 32-bit key of the logit
//            (temperature > 0 keeps the order), counting tokens: the key of
//            the k-th largest logit, ties kept -- exact integer work;
//   top-p    one pass for the softmax mass Z, then 4 radix passes summing
//            mass instead of counts: the largest key whose tokens at or above
//            it hold at least p * Z.  Masses are fixed-point integers
//            (2^31 * exp(z - z_max)), so the sums do not depend on the order
//            of the atomic adds and the cut is deterministic;
//   min-p    z - z_max >= ln(min_p), no pass of its own;
//   draw     Gumbel-max over the kept tokens: key = z - ln(-ln u), u from
//            Philox4x32-10 (counter (i / 4, row, offset lo, offset hi), key
//            (seed lo, seed hi), word i % 4; u = (floor(x / 2^9) + 1/2) / 2^23),
//            ties to the lowest index.
//
// Histogram updates go through wave-level aggregation: lanes that hit the
// same bin are combined with a ballot and one lane adds the group's total,
// so the clustered high digits of float keys do not serialise on LDS
// atomics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;

struct SampleArgs {
  const float* temperature;   // per row, or nullptr: temperature_all
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
  float temperature_all;
  int32_t top_k_all;
  float top_p_all;
  float min_p_all;
  uint32_t seed_lo, seed_hi, offset_lo, offset_hi;
};

struct F32Bits {
  using Bits = uint32_t;
  static __device__ __forceinline__ float value(uint32_t b) { return __uint_as_float(b); }
};
struct BF16Bits {
  using Bits = uint16_t;
  static __device__ __forceinline__ float value(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
};
struct F16Bits {
  using Bits = uint16_t;
  static __device__ __forceinline__ float value(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }
};

// Monotone map from float order to unsigned order (for non-NaN values).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0;
    const uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

__device__ __forceinline__ float unit_uniform(uint32_t x) {
  return (static_cast<float>(x >> 9) + 0.5f) * (1.0f / 8388608.0f);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & 63; }

template <typename V>
__device__ __forceinline__ V wave_sum(V v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Add w (for every lane with `active`) into hist[bin], one LDS atomic per
// distinct bin in the wave.  Every lane of the wave must call it.
template <typename V>
__device__ __forceinline__ void wave_hist_add(V* hist, bool active, uint32_t bin, V w) {
  uint64_t pending = __ballot(active);
  while (pending) {
    const int leader = __ffsll(static_cast<long long>(pending)) - 1;
    const uint32_t lb = __shfl(bin, leader);
    const bool same = active && bin == lb;
    const uint64_t group = __ballot(same);
    const V total = wave_sum(same ? w : V(0));
    if (lane_id() == leader) atomicAdd(&hist[lb], total);
    active = active && !same;
    pending &= ~group;
  }
}

template <typename D>
struct RowView {
  const typename D::Bits* row;
  const uint32_t* mrow;   // nullptr: no mask
  int32_t V;

  // value and candidacy of token i (< V)
  __device__ __forceinline__ float value(int32_t i, uint32_t word, bool* ok) const {
    const float x = D::value(row[i]);
    const bool bit = mrow ? ((word >> (static_cast<uint32_t>(i) & 31u)) & 1u) : true;
    *ok = bit && __builtin_isfinite(x);
    return x;
  }
};

// Radix select from the top: the largest key K such that the weight (count
// or mass) of candidate tokens with key >= K reaches `need`.  `keep_ok`
// filters the tokens that take part.
template <typename D, typename W>
__device__ uint32_t radix_select(const RowView<D>& rv, int32_t ngroups, W need, float inv_t, float zmax,
                                 bool by_mass, W* hist, uint32_t* s_digit, W* s_need) {
  const int t = static_cast<int>(threadIdx.x);
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = t; b < 256; b += kSampleThreads) hist[b] = W(0);
    __syncthreads();
    for (int32_t base = 0; base < ngroups; base += kSampleThreads) {
      const int32_t g = base + t;
      const int32_t i0 = 4 * g;
      const uint32_t word = (rv.mrow && i0 < rv.V) ? rv.mrow[i0 >> 5] : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int32_t i = i0 + q;
        bool ok = false;
        float x = 0.f;
        if (g < ngroups && i < rv.V) x = rv.value(i, word, &ok);
        const uint32_t key = order_key(x);
        ok = ok && (key & pmask) == prefix;
        W w = W(1);
        if (by_mass) w = ok ? static_cast<W>(expf(x * inv_t - zmax) * 2147483648.0f) : W(0);
        wave_hist_add<W>(hist, ok, (key >> shift) & 255u, w);
      }
    }
    __syncthreads();
    if (t == 0) {
      W cum = W(0);
      int d = 255;
      for (; d > 0; --d) {
        if (cum + hist[d] >= need) break;
        cum += hist[d];
      }
      *s_digit = static_cast<uint32_t>(d);
      *s_need = need - cum;
    }
    __syncthreads();
    prefix |= *s_digit << shift;
    pmask |= 255u << shift;
    need = *s_need;
    __syncthreads();
  }
  return prefix;
}

template <typename D>
__global__ __launch_bounds__(kSampleThreads) void sample_rows(const typename D::Bits* __restrict__ logits, int64_t ls,
                                                              const uint32_t* __restrict__ mask, int64_t ms,
                                                              int32_t V, SampleArgs a, int64_t row_base,
                                                              int64_t* __restrict__ out) {
  __shared__ float s_best[kSampleWaves];
  __shared__ int32_t s_besti[kSampleWaves];
  __shared__ uint32_t s_count[kSampleWaves];
  __shared__ unsigned long long s_mass[kSampleWaves];
  __shared__ uint32_t hist_n[256];
  __shared__ unsigned long long hist_m[256];
  __shared__ uint32_t s_digit;
  __shared__ uint32_t s_need_n;
  __shared__ unsigned long long s_need_m;

  const int64_t r = blockIdx.x;
  const int t = static_cast<int>(threadIdx.x);
  const int wave = t >> 6;
  const RowView<D> rv{logits + r * ls, mask ? mask + r * ms : nullptr, V};
  const int32_t ngroups = (V + 3) / 4;

  const float temp = a.temperature ? a.temperature[r] : a.temperature_all;
  const int32_t top_k = a.top_k ? a.top_k[r] : a.top_k_all;
  const float top_p = a.top_p ? a.top_p[r] : a.top_p_all;
  const float min_p = a.min_p ? a.min_p[r] : a.min_p_all;

  // ---- pass 1: max, argmax (lowest index), candidate count
  float best = -__builtin_inff();
  int32_t besti = 0x7FFFFFFF;
  uint32_t count = 0;
  for (int32_t base = 0; base < ngroups; base += kSampleThreads) {
    const int32_t g = base + t;
    const int32_t i0 = 4 * g;
    if (g < ngroups) {
      const uint32_t word = rv.mrow ? rv.mrow[i0 >> 5] : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int32_t i = i0 + q;
        if (i < V) {
          bool ok;
          const float x = rv.value(i, word, &ok);
          if (ok) {
            ++count;
            if (x > best) {  // strictly greater: the first (lowest) index wins ties within a thread
              best = x;
              besti = i;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int32_t oi = __shfl_xor(besti, o);
    if (ob > best || (ob == best && oi < besti)) {
      best = ob;
      besti = oi;
    }
    count += __shfl_xor(count, o);
  }
  if (lane_id() == 0) {
    s_best[wave] = best;
    s_besti[wave] = besti;
    s_count[wave] = count;
  }
  __syncthreads();
  best = s_best[0];
  besti = s_besti[0];
  count = s_count[0];
  for (int w = 1; w < kSampleWaves; ++w) {
    if (s_best[w] > best || (s_best[w] == best && s_besti[w] < besti)) {
      best = s_best[w];
      besti = s_besti[w];
    }
    count += s_count[w];
  }
  if (count == 0 || !(temp > 0.f)) {  // no candidate, or greedy
    if (t == 0) out[r] = count == 0 ? -1 : besti;
    return;
  }

  const float inv_t = 1.0f / temp;
  const float zmax = best * inv_t;
  uint32_t cut = 0;   // keep tokens with order_key(x) >= cut

  if (top_k > 0 && static_cast<uint32_t>(top_k) < count) {
    const uint32_t k = radix_select<D, uint32_t>(rv, ngroups, static_cast<uint32_t>(top_k), inv_t, zmax, false,
                                                 hist_n, &s_digit, &s_need_n);
    cut = max(cut, k);
  }
  if (top_p < 1.0f) {
    unsigned long long mass = 0;
    for (int32_t base = 0; base < ngroups; base += kSampleThreads) {
      const int32_t g = base + t;
      const int32_t i0 = 4 * g;
      if (g < ngroups) {
        const uint32_t word = rv.mrow ? rv.mrow[i0 >> 5] : 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t i = i0 + q;
          if (i < V) {
            bool ok;
            const float x = rv.value(i, word, &ok);
            if (ok) mass += static_cast<unsigned long long>(expf(x * inv_t - zmax) * 2147483648.0f);
          }
        }
      }
    }
    mass = wave_sum(mass);
    if (lane_id() == 0) s_mass[wave] = mass;
    __syncthreads();
    unsigned long long total = 0;
    for (int w = 0; w < kSampleWaves; ++w) total += s_mass[w];
    __syncthreads();
    unsigned long long target = static_cast<unsigned long long>(ceil(static_cast<double>(top_p) *
                                                                     static_cast<double>(total)));
    if (target == 0) target = 1;
    const uint32_t k = radix_select<D, unsigned long long>(rv, ngroups, target, inv_t, zmax, true, hist_m,
                                                           &s_digit, &s_need_m);
    cut = max(cut, k);
  }
  const bool use_min_p = min_p > 0.f;
  const float ln_min_p = use_min_p ? logf(min_p) : 0.f;

  // ---- draw: Gumbel-max over the kept tokens
  float bk = -__builtin_inff();
  int32_t bi = 0x7FFFFFFF;
  for (int32_t base = 0; base < ngroups; base += kSampleThreads) {
    const int32_t g = base + t;
    const int32_t i0 = 4 * g;
    if (g < ngroups) {
      const uint32_t word = rv.mrow ? rv.mrow[i0 >> 5] : 0u;
      uint32_t c[4] = {static_cast<uint32_t>(g), static_cast<uint32_t>(row_base + r), a.offset_lo, a.offset_hi};
      philox4x32_10(c, a.seed_lo, a.seed_hi);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int32_t i = i0 + q;
        if (i < V) {
          bool ok;
          const float x = rv.value(i, word, &ok);
          const float z = x * inv_t;
          ok = ok && order_key(x) >= cut && (!use_min_p || z - zmax >= ln_min_p);
          if (ok) {
            const float u = unit_uniform(c[q]);
            const float key = z - logf(-logf(u));
            if (key > bk) {
              bk = key;
              bi = i;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(bk, o);
    const int32_t oi = __shfl_xor(bi, o);
    if (ob > bk || (ob == bk && oi < bi)) {
      bk = ob;
      bi = oi;
    }
  }
  __syncthreads();
  if (lane_id() == 0) {
    s_best[wave] = bk;
    s_besti[wave] = bi;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < kSampleWaves; ++w)
      if (s_best[w] > bk || (s_best[w] == bk && s_besti[w] < bi)) {
        bk = s_best[w];
        bi = s_besti[w];
      }
    // bk == -inf only if no token survived the cut, which cannot happen (the max token always does)
    out[r] = bi == 0x7FFFFFFF ? besti : bi;
  }
}

}  // namespace mi
