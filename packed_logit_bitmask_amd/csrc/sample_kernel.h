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
// One block per row (1024 threads when each compute unit holds one row;
// 256 when many rows share a unit, or 512 for filtered 16-bit rows, two to a
// unit), or, for a few rows without top-k, top-p or min-p, one 256-thread
// block per segment of a row, the segments merging by an atomic maximum.  A
// few filtered 16-bit rows split the same way when the caller gives a
// workspace: their cuts come first from merged per-segment histograms
// (split_hist, split_search below).  Given a workspace, a large batch of
// filtered 16-bit rows hands out its dense rows first (row_classes,
// heavy_first_row below), so that they spread over the compute units.
// Each pass walks the row in groups of 8 consecutive tokens per thread
// through raw buffer loads (16-byte vectors when the row start is aligned),
// several groups in flight per thread; trip counts are uniform across the
// block.
//
//   pass 1   max logit over the candidates and its (lowest) index -> greedy
//            rows and rows with no candidate end here; skipped when the row
//            uses neither top-p nor min-p (nothing else needs it), and for
//            16-bit rows with top-k or top-p (their key histogram gives it);
//   16-bit   bf16 and fp16 rows with top-k or top-p, in 1024- or 512-thread
//            blocks: one pass counts the tokens the mask allows under each
//            of the 65536 16-bit keys (LDS, 16- or 8-bit counters); the
//            maximum and both cuts follow from the counts (fine_search).
//            A row whose mask allows at most 4096 tokens (and that is not
//            held in registers) lists its candidates instead and selects
//            both cuts on the list (sparse_search).  The radix passes below remain for a
//            row where one key holds more tokens than its counter can
//            (65536 or 256);
//   fp32     fp32 rows with top-k or top-p in 1024-thread blocks: one pass
//            counts and sums mass under the top 12 bits of each order key
//            (coarse_hist32), a search picks the cut's bucket, and the draw
//            pass lists the candidates of that bucket in LDS, where a radix
//            select over the low 20 bits gives the exact cut; a bucket too
//            crowded for the list, and fp32 rows in smaller blocks, take
//            the radix passes below;
//   top-k    radix search over an order-preserving 32-bit key of the logit
//            (temperature > 0 keeps the order), counting tokens: the key of
//            the k-th largest logit, ties kept -- exact integer work;
//   top-p    the same radix search summing softmax mass instead of counts:
//            the largest key whose tokens at or above it hold at least p * Z
//            (Z is the total of the first pass's mass histogram).  Masses
//            are fixed-point integers (2^31 * exp(z - z_max), the
//            exponential by the hardware base-2 instruction), so the sums do
//            not depend on the order of the atomic adds: the cut is
//            deterministic.  Both searches share the passes, one per 8-bit
//            digit: 4 for fp32, 3 for fp16, 2 for bf16 (the low digits of a
//            16-bit type's key are the same for every token of a prefix);
//            each digit is picked by a wave-parallel suffix scan;
//   min-p    z - z_max >= ln(min_p), no pass of its own;
//   draw     Gumbel-max over the kept tokens: the largest z - ln(-ln u),
//            compared as z log2(e) - log2(-log2 u) (the same order; two
//            hardware log2 instructions), u from
//            Philox4x32-10 (counter (i / 4, row, offset lo, offset hi), key
//            (seed lo, seed hi), word i % 4; u = (floor(x / 2^9) + 1/2) / 2^23),
//            ties to the lowest index.  A pass of its own, except where the
//            last radix pass (fp32) draws as it counts.  After the
//            16-bit search the kept test runs on packed 16-bit keys, and a
//            sparse kept set is first listed in LDS so the generator runs
//            on the list alone.
//
// The radix histograms are private to each wave (LDS), folded after every
// pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apply_kernels.h"  // raw buffer resources (Rsrc, make_rsrc, load_word, load16, kSkip)

namespace mi {

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

// kZeroLowBits: low bits of the binary32 pattern that are zero for every
// value of the type (bf16 keeps 7 fraction bits, fp16 10, subnormals fewer),
// so radix digits that lie wholly inside them never need a pass.
struct F32Bits {
  using Bits = uint32_t;
  static constexpr int kZeroLowBits = 0;
  static __device__ __forceinline__ float value(uint32_t b) { return __uint_as_float(b); }
};
struct BF16Bits {
  using Bits = uint16_t;
  static constexpr int kZeroLowBits = 16;
  static constexpr uint32_t kKey16Lo = 0x0080u, kKey16Hi = 0xFF7Fu;  // 16-bit order keys of -max, +max
  static constexpr uint32_t kExp16 = 0x7F80u;                           // exponent field
  static __device__ __forceinline__ float value(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
};
struct F16Bits {
  using Bits = uint16_t;
  static constexpr int kZeroLowBits = 13;
  static constexpr uint32_t kKey16Lo = 0x0400u, kKey16Hi = 0xFBFFu;  // 16-bit order keys of -max, +max
  static constexpr uint32_t kExp16 = 0x7C00u;                           // exponent field
  static __device__ __forceinline__ float value(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }
};

// Monotone map from float order to unsigned order (for non-NaN values).
// -0 takes the key of +0: the two compare equal, so a cut at zero keeps both.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  b = b == 0x80000000u ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The raw 16-bit float (bf16, fp16) whose 16-bit order key is k: the
// inverse of order_key16x2 below (a key with the top bit set is a value of
// sign 0; otherwise the bits were inverted).
__device__ __forceinline__ uint32_t bits_of_key16(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7FFFu) : (k ^ 0xFFFFu);
}

// Softmax mass of a token in fixed point, 2^31 exp(z - z_max) with z = x / T,
// about 2^31 at the maximum and less below it: the hardware base-2
// exponential of x log2(e) / T - z_max log2(e) (one fma per token: the two
// products are the same for the whole row), converted through u32.  Every
// top-p search sums these, so equal inputs always give equal sums.
__device__ __forceinline__ uint32_t fixed_mass(float x, float inv_t, float zmax) {
  const float a = inv_t * 1.4426950408889634f, b = -(zmax * 1.4426950408889634f);
  return static_cast<uint32_t>(__builtin_amdgcn_exp2f(fmaf(x, a, b)) * 2147483648.0f);
}

// Whether an order key belongs to a finite value: keys of finite floats run
// from that of -FLT_MAX (0x00800000) to that of +FLT_MAX (0xFF7FFFFF); the
// infinities and NaNs lie outside.
__device__ __forceinline__ bool finite_key(uint32_t key) { return key - 0x00800000u < 0xFF000000u; }

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // each product as one 64-bit multiply: one v_mad_u64_u32 instead of a
    // v_mul_hi_u32 / v_mul_lo_u32 pair (a third faster on gfx950)
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c[0];
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c[2];
    // each three-way xor as one v_bitop3_b32 (truth table 0x96: a ^ b ^ c),
    // which the compiler does not form by itself here
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c[1], k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c[3], k1, 0x96);
    c[0] = n0;
    c[1] = static_cast<uint32_t>(p1);
    c[2] = n2;
    c[3] = static_cast<uint32_t>(p0);
  }
}

// (k + 1/2) 2^-23 for the top 23 bits k of x: exact in binary32, so one fma
__device__ __forceinline__ float unit_uniform(uint32_t x) {
  return fmaf(static_cast<float>(x >> 9), 1.0f / 8388608.0f, 0.5f / 8388608.0f);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & 63; }

// ---- Wave scans by DPP.  A wave64 is four rows of 16 lanes: row shifts
// (row_shr:n) combine lanes inside a row, then row broadcasts (lane 15 of a
// row into the next row, lane 31 into rows 2 and 3) combine the rows.  Every
// step is one VALU move, with none of the LDS round trips that __shfl makes.
// Lanes a move has no source for (or whose row it leaves out) read 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_read(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, true));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_read(unsigned long long v) {
  const uint32_t lo = dpp_read<CTRL, ROWS>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_read<CTRL, ROWS>(static_cast<uint32_t>(v >> 32));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Inclusive sums inside each 16-lane row, then lane 15 of rows 0 and 2 added
// into rows 1 and 3: lane 31 then holds the total of lanes 0..31 and lane 63
// that of lanes 32..63 (each half-wave's sum).
template <typename T>
__device__ __forceinline__ T half_wave_scan(T x) {
  x += dpp_read<kDppShr1, 0xF>(x);
  x += dpp_read<kDppShr2, 0xF>(x);
  x += dpp_read<kDppShr4, 0xF>(x);
  x += dpp_read<kDppShr8, 0xF>(x);
  x += dpp_read<kDppBcast15, 0xA>(x);
  return x;
}

// Inclusive prefix sum over the wave's 64 lanes (lane 63 holds the total).
template <typename T>
__device__ __forceinline__ T wave_prefix_sum(T x) {
  x = half_wave_scan(x);
  x += dpp_read<kDppBcast31, 0xC>(x);
  return x;
}

// Maximum over the wave's 64 lanes, in every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp_read<kDppShr1, 0xF>(x));
  x = max(x, dpp_read<kDppShr2, 0xF>(x));
  x = max(x, dpp_read<kDppShr4, 0xF>(x));
  x = max(x, dpp_read<kDppShr8, 0xF>(x));
  x = max(x, dpp_read<kDppBcast15, 0xA>(x));
  x = max(x, dpp_read<kDppBcast31, 0xC>(x));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// Lane 63's value, in every lane.
__device__ __forceinline__ uint32_t lane63(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
__device__ __forceinline__ unsigned long long lane63(unsigned long long x) {
  return (static_cast<unsigned long long>(lane63(static_cast<uint32_t>(x >> 32))) << 32) | lane63(static_cast<uint32_t>(x));
}


// One row's logits and mask, read 8 consecutive tokens (a group) at a time.
// The loads go through raw buffer resources that end at the row's vocab
// size (logits) and its last mask word, so a load for a group past the end
// gets an out-of-range offset and returns 0 instead of branching: the
// compiler then issues every load of a batch before the first wait.  A row
// without a mask has a resource of size 0 and all tokens below V count.
template <typename D>
struct RowView {
  using Bits = typename D::Bits;
  const Bits* row;
  bool has_mask;
  int32_t V;
  bool aligned;   // row start 16-byte aligned: whole groups load as vectors
  Rsrc rl, rm;

  __device__ __forceinline__ RowView(const Bits* row_, const uint32_t* mrow, int32_t V_)
      : row(row_), has_mask(mrow != nullptr), V(V_), aligned((reinterpret_cast<uintptr_t>(row_) & 15u) == 0),
        rl(make_rsrc(row_, static_cast<uint32_t>(V_) * sizeof(Bits))),
        rm(make_rsrc(mrow, mrow ? static_cast<uint32_t>((V_ + 31) / 32) * 4u : 0u)) {}

  // A group as loaded: its mask word and its logits as raw 32-bit words
  // (2 tokens per word for 16-bit types), so a batch in flight costs 5 or 9
  // registers per group rather than 8 decoded floats.
  struct Raw {
    uint32_t w;
    uint32_t v[sizeof(Bits) == 2 ? 4 : 8];
  };

  // Issue group g's loads; `full` says the whole group lies below V (else
  // every load takes the out-of-range offset and returns 0).
  template <bool VEC>
  __device__ __forceinline__ Raw load_raw(int32_t g, bool full) const {
    Raw r;
    r.w = load_word(rm, full ? (g >> 2) * 4 : kSkip);
    if constexpr (sizeof(Bits) == 2) {
      if constexpr (VEC) {
        const uint4 v = load16(rl, full ? g * 16 : kSkip);
        r.v[0] = v.x;
        r.v[1] = v.y;
        r.v[2] = v.z;
        r.v[3] = v.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rl, full ? (8 * g + 2 * q) * 2 : kSkip, 0, 0);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rl, full ? (8 * g + 2 * q + 1) * 2 : kSkip, 0, 0);
          r.v[q] = lo | (hi << 16);
        }
      }
    } else {
      if constexpr (VEC) {
        const uint4 a = load16(rl, full ? g * 32 : kSkip);
        const uint4 b = load16(rl, full ? g * 32 + 16 : kSkip);
        r.v[0] = a.x;
        r.v[1] = a.y;
        r.v[2] = a.z;
        r.v[3] = a.w;
        r.v[4] = b.x;
        r.v[5] = b.y;
        r.v[6] = b.z;
        r.v[7] = b.w;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) r.v[q] = load_word(rl, full ? (8 * g + q) * 4 : kSkip);
      }
    }
    return r;
  }

  // Group g's mask bits (token q in bit q); 0 for a group past the full ones.
  __device__ __forceinline__ uint32_t mask_bits(const Raw& r, int32_t g, bool full) const {
    return full ? (has_mask ? (r.w >> ((g & 3) * 8)) & 0xFFu : 0xFFu) : 0u;
  }

  // Group values only.
  __device__ __forceinline__ void values(const Raw& r, float x[8]) const {
    if constexpr (sizeof(Bits) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[2 * q] = D::value(static_cast<Bits>(r.v[q] & 0xFFFFu));
        x[2 * q + 1] = D::value(static_cast<Bits>(r.v[q] >> 16));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = D::value(r.v[q]);
    }
  }

  // Group g's values and a bit per token that is a candidate (mask bit set,
  // finite logit); 0 for a group past the full ones.
  __device__ __forceinline__ uint32_t decode(const Raw& r, int32_t g, bool full, float x[8]) const {
    const uint32_t bits = has_mask ? (r.w >> ((g & 3) * 8)) & 0xFFu : 0xFFu;
    if constexpr (sizeof(Bits) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[2 * q] = D::value(static_cast<Bits>(r.v[q] & 0xFFFFu));
        x[2 * q + 1] = D::value(static_cast<Bits>(r.v[q] >> 16));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = D::value(r.v[q]);
    }
    uint32_t ok = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (((bits >> q) & 1u) && __builtin_isfinite(x[q])) ok |= 1u << q;
    return full ? ok : 0u;
  }

  // Group g's values with every position that is not a candidate by the
  // mask (bit clear, or past the full groups) set to -inf.  Non-finite
  // logits pass through: a caller taking maxima sees them in the result.
  __device__ __forceinline__ void gated(const Raw& r, int32_t g, bool full, float xv[8]) const {
    const uint32_t bits = full ? (has_mask ? (r.w >> ((g & 3) * 8)) & 0xFFu : 0xFFu) : 0u;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t u;
      if constexpr (sizeof(Bits) == 2)
        u = __float_as_uint(D::value(static_cast<Bits>(q & 1 ? r.v[q >> 1] >> 16 : r.v[q >> 1] & 0xFFFFu)));
      else
        u = r.v[q];
      const uint32_t m = 0u - ((bits >> q) & 1u);  // all ones for a candidate
      xv[q] = __uint_as_float((u & m) | (0xFF800000u & ~m));
    }
  }

  // The last, partial group (tokens 8 * (V / 8) .. V - 1), by plain loads.
  __device__ __forceinline__ uint32_t load_tail(float x[8]) const {
    const int32_t i0 = V & ~7;
    uint32_t ok = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      x[q] = 0.f;
      if (i0 + q < V) {
        x[q] = D::value(row[i0 + q]);
        const bool bit = has_mask ? ((load_word(rm, ((i0 + q) >> 5) * 4) >> ((i0 + q) & 31)) & 1u) : true;
        if (bit && __builtin_isfinite(x[q])) ok |= 1u << q;
      }
    }
    return ok;
  }
};

template <int BYTES, int THREADS, bool VEC, typename D, typename F>
__device__ __forceinline__ void walk_groups_raw(const RowView<D>& rv, F& f) {
  // groups in flight per thread: BYTES of logits (the misaligned path, with
  // one load per token, keeps at most 4).  All of a batch's loads are
  // issued before its first group is used.  (Double-buffering half batches,
  // so the next batch's loads overlap this batch's arithmetic, measured a
  // few percent slower in every mode.)
  constexpr int kFull = BYTES / (8 * static_cast<int>(sizeof(typename D::Bits)));
  constexpr int kInFlight = VEC ? kFull : (kFull < 4 ? kFull : 4);
  const int32_t nfull = rv.V >> 3;
  const int t = static_cast<int>(threadIdx.x);
  for (int32_t base = 0; base < nfull; base += kInFlight * THREADS) {
    typename RowView<D>::Raw raw[kInFlight];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const int32_t g = base + j * THREADS + t;
      raw[j] = rv.template load_raw<VEC>(g, g < nfull);
    }
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const int32_t g = base + j * THREADS + t;
      f(g, raw[j], g < nfull);
    }
  }
}

// Walk the full 8-token groups of the row as loaded: f(g, raw, full) for
// group g (full: the whole group lies below V; groups past the row come
// with full == false).  The partial last group, if any, is the caller's.
template <int BYTES, int THREADS, typename D, typename F>
__device__ __forceinline__ void walk_row_raw(const RowView<D>& rv, F&& f) {
  if (rv.aligned)
    walk_groups_raw<BYTES, THREADS, true>(rv, f);
  else
    walk_groups_raw<BYTES, THREADS, false>(rv, f);
}

// Walk the row: f(i0, x[8], ok) for every 8-token group, BYTES of logits
// per thread loaded before any is used (128 when a compute unit holds one
// row; 64 when several rows share it, for fewer registers).  Every thread of
// the block calls f the same number of times (groups it does not own come
// with ok == 0), so f may hold block-uniform control flow.
template <int BYTES, int THREADS, typename D, typename F>
__device__ __forceinline__ void walk_row(const RowView<D>& rv, F&& f) {
  walk_row_raw<BYTES, THREADS>(rv, [&](int32_t g, const typename RowView<D>::Raw& raw, bool full) {
    float x[8];
    const uint32_t ok = rv.decode(raw, g, full, x);
    f(8 * g, x, ok);
  });
  if (rv.V & 7) {
    float x[8] = {};
    const uint32_t ok = threadIdx.x == 0 ? rv.load_tail(x) : 0u;
    f(rv.V & ~7, x, ok);
  }
}

// Per-wave private histograms for the threshold search: counts for top-k,
// fixed-point softmax mass for top-p.
struct SelectState {
  uint32_t prefix_k, need_k;            // top-k: key prefix so far, count still needed below it
  unsigned long long need_p;            // top-p: mass still needed below the prefix
  uint32_t prefix_p;
};

// One wave's view of a 256-bin histogram for the radix search: lane l
// holds bins 4l .. 4l+3, and a shuffle scan gives every lane the suffix
// total S(4l) = hist[4l] + ... + hist[255].
template <typename T>
struct WaveSuffix {
  T h[4];
  T incl;  // S(4l)

  __device__ __forceinline__ explicit WaveSuffix(const T* hist) {
    const int l = lane_id();
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = hist[4 * l + j];
    incl = h[0] + h[1] + h[2] + h[3];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const T v = __shfl_down(incl, o);
      if (l + o < 64) incl += v;
    }
  }

  __device__ __forceinline__ T total() const { return __shfl(incl, 0); }

  // The digit d the search takes: the largest d >= 1 with S(d) >= need,
  // else 0; and S(d + 1), the total of the bins above it.
  __device__ __forceinline__ void pick(T need, int* d, T* above) const {
    const int l = lane_id();
    const uint64_t m = __ballot(incl >= need);   // lanes 0 .. L, as S falls with l
    const int L = m ? 63 - __clzll(static_cast<long long>(m)) : 0;
    T s = incl - (h[0] + h[1] + h[2] + h[3]);  // S(4l + 4), the bins above this lane
    int j = 0;
    T ab = 0;
    bool found = false;
#pragma unroll
    for (int q = 3; q >= 1; --q) {
      const T next = s + h[q];
      if (!found && next >= need) {
        j = q;
        ab = s;
        found = true;
      }
      s = next;
    }
    if (!found) ab = s;  // j = 0: the bins above bin 4l
    *d = __shfl(4 * l + j, L);
    *above = __shfl(ab, L);
  }
};

// Dynamic LDS the kernel needs when a row may use top-k or top-p (the
// per-wave histograms); 0 otherwise.
constexpr size_t sample_hist_bytes(int threads) {
  return static_cast<size_t>(threads / 64) * 256 * (sizeof(uint32_t) + sizeof(unsigned long long));
}

// The full-resolution histogram of a 16-bit type's keys: 65536 counters,
// several to a word, plus one spare word per lane that non-candidates add to
// (so the add needs no branch and spreads over the banks).  1024-thread
// blocks (one per compute unit) count in 16 bits, two per word (128 KB);
// 512-thread blocks, for batches with more rows than compute units, count
// in 8 bits, four per word (64 KB), so two blocks share a unit and one's
// passes overlap the other's searches.  Either way a thread owns 32 words.
template <int THREADS>
constexpr int kFineBits = THREADS == 1024 ? 16 : 8;
constexpr int fine_words(int threads) { return 65536 / (32 / (threads == 1024 ? 16 : 8)); }
constexpr size_t sample_fine_bytes(int threads) {
  return static_cast<size_t>(fine_words(threads) + 64) * sizeof(uint32_t);
}

// Whether a block shape searches 16-bit keys through the full histogram.
template <typename D, int THREADS>
constexpr bool kFineSearch = sizeof(typename D::Bits) == 2 && (THREADS == 1024 || THREADS == 512);

// Two 16-bit order keys at once, from a word holding two raw 16-bit floats
// (low token in the low half): a negative value's bits are inverted, a
// positive one's sign bit set, so unsigned key order is value order.  -0
// keeps a key of its own, one below +0's (callers that need the two equal
// handle it).
__device__ __forceinline__ uint32_t order_key16x2(uint32_t two) {
  typedef short short2_t __attribute__((ext_vector_type(2)));
  const short2_t sign = __builtin_bit_cast(short2_t, two) >> static_cast<short>(15);  // per half: 0 or all ones
  return two ^ (__builtin_bit_cast(uint32_t, sign) | 0x80008000u);
}

// Count the tokens the mask allows under their 16-bit keys into `fine`
// (LDS, CB-bit counters, KW = 32 / CB to a word: key k in word k / KW), from
// a cleared start; returns this thread's number of allowed tokens below V.
// A token the mask rules out adds to its lane's spare word (after the 65536
// keys) instead, so the add needs no branch and spreads over the banks.
// Ends with a barrier.  A row of at most 4 groups per thread may come
// already loaded in pre[4] (group j * THREADS + t in pre[j], with
// `preloaded` set); otherwise the pass reads the row.
template <typename D, int BYTES, int THREADS, int CB>
__device__ __forceinline__ uint32_t count_keys(const RowView<D>& rv, uint32_t* fine,
                                               const typename RowView<D>::Raw (&pre)[4], bool preloaded) {
  constexpr uint32_t KW = 32 / CB;
  constexpr uint32_t kWords = 65536 / KW;
  const int t = static_cast<int>(threadIdx.x);
  uint4* f4 = reinterpret_cast<uint4*>(fine);
  for (int i = t; i < static_cast<int>(kWords + 64) / 4; i += THREADS) f4[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  uint32_t allowed = 0;
  const uint32_t spare = KW * (kWords + static_cast<uint32_t>(lane_id()));
  const auto add = [&](uint32_t k, uint32_t bit) {
    const uint32_t kk = bit ? k : spare;
    atomicAdd(&fine[kk / KW], 1u << ((kk % KW) * CB));
  };
  const auto group = [&](int32_t g, const typename RowView<D>::Raw& raw, bool full) {
    const uint32_t bits = rv.mask_bits(raw, g, full);
    allowed += __builtin_popcount(bits);
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      const uint32_t k2 = order_key16x2(raw.v[p2]);
      add(k2 & 0xFFFFu, (bits >> (2 * p2)) & 1u);
      add(k2 >> 16, (bits >> (2 * p2 + 1)) & 1u);
    }
  };
  if (preloaded) {
    const int32_t nfull = rv.V >> 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t g = j * THREADS + t;
      group(g, pre[j], g < nfull);
    }
  } else {
    walk_row_raw<BYTES, THREADS>(rv, group);
  }
  if ((rv.V & 7) && t == 0) {  // the partial last group, by plain loads
    for (int32_t i = rv.V & ~7; i < rv.V; ++i) {
      const uint32_t bit = rv.has_mask ? (load_word(rv.rm, (i >> 5) * 4) >> (i & 31)) & 1u : 1u;
      allowed += bit;
      add(order_key16x2(rv.row[i]) & 0xFFFFu, bit);
    }
  }
  __syncthreads();
  return allowed;
}

// Top-k and top-p cuts of a 16-bit row from one pass over it.  Each finite
// bf16 or fp16 value has a 16-bit key of its own, and the tokens under one
// key share their value, so a count per key answers both searches exactly:
// top-k counts down from the largest key; top-p sums count x mass per key,
// the mass being the fixed-point one the radix search sums token by token,
// so the cut is the same.  The pass counts every token the mask allows,
// finite or not, under its key; the keys of the finite values form
// [D::kKey16Lo, D::kKey16Hi], and only those count as candidates.  -0 and +0
// have adjacent keys: a cut on either is the value zero, which keeps both.
// The largest candidate (*best; -inf when the row has none) is the highest
// finite key with a count.  A counter is 16 or 8 bits wide (kFineBits), so a
// key holding 65536 (or 256) tokens or more would wrap into its neighbour:
// the counts then fall short of the tokens counted, and the function returns
// false for the radix search to take over (no thread reads `fine` after the
// barrier that decides it).  On success *cut is the order key (of the
// widened value) at and above which tokens are kept, 0 to keep every
// candidate; *cut16 the same cut as a 16-bit key (0 to keep all), and *kept
// the number of candidates it keeps.  A row of at most 4 groups per thread
// comes already loaded in pre[4] (group j * THREADS + t in pre[j], with
// `preloaded` set); otherwise the pass reads the row.
template <typename D, int BYTES, int THREADS>
__device__ __forceinline__ bool fine_search(const RowView<D>& rv, uint32_t* fine, float inv_t, bool use_k,
                                            int32_t top_k, bool use_p, float top_p, float* best, uint32_t* cut,
                                            uint32_t* cut16, uint32_t* kept,
                                            const typename RowView<D>::Raw (&pre)[4], bool preloaded) {
  using Bits = typename D::Bits;
  constexpr int kWaves = THREADS / 64;
  constexpr int CB = kFineBits<THREADS>;        // bits per counter
  constexpr uint32_t KW = 32 / CB;              // keys per word
  constexpr uint32_t KPT = 65536 / THREADS;     // keys per thread: 64 or 128
  static_assert(KPT / KW == 32, "a thread owns 32 words of the histogram");
  constexpr uint32_t KPL = KPT / 64;            // keys per lane in the final search
  constexpr uint32_t kCount = (1u << CB) - 1u;  // one counter's bits
  constexpr uint32_t kSpan = D::kKey16Hi - D::kKey16Lo;
  // The keys of non-finite values fill whole words at both ends of the key
  // space, so a word holds finite keys only or none: words [kW0, kW1).
  static_assert(D::kKey16Lo % KW == 0 && (D::kKey16Hi + 1) % KW == 0, "finite keys start and end on a word");
  constexpr uint32_t kW0 = D::kKey16Lo / KW, kW1 = (D::kKey16Hi + 1) / KW;
  __shared__ uint32_t s_d[kWaves], s_kmax[kWaves], s_c[kWaves], s_cut[2], s_cross[2];
  __shared__ uint32_t s_above_n[2], s_kept[2];
  __shared__ unsigned long long s_m[kWaves], s_above[2];
  const int t = static_cast<int>(threadIdx.x);
  const int lane = lane_id(), wave = t >> 6;
  // the count of key k, from the word that holds it
  const auto count_in = [](uint32_t w, uint32_t k) { return (w >> ((k % KW) * CB)) & kCount; };
  // every count of a word, summed: one dot product with ones
  const auto word_sum = [](uint32_t w) {
    if constexpr (CB == 16) {
      typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
      const u16x2 ones = {1, 1};
      return __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, w), ones, 0u, false);
    } else {
      return __builtin_amdgcn_udot4(w, 0x01010101u, 0u, false);
    }
  };

  if (t < 2) {
    s_cut[t] = 0u;
    s_cross[t] = ~0u;  // no crossing: keep every candidate
  }
  const uint32_t allowed = count_keys<D, BYTES, THREADS, CB>(rv, fine, pre, preloaded);  // tokens the mask allows below V

  // ---- sums: thread t holds keys [KPT t, KPT t + KPT), words [32t, 32t + 32),
  // read eight at a time in a rotated order so a wave's lanes hit different
  // banks.  Only the threads at the two ends of the key space hold words of
  // non-finite keys.
  const uint32_t k0 = KPT * static_cast<uint32_t>(t);
  const auto in_range = [](uint32_t k) { return k - D::kKey16Lo <= kSpan; };
  const uint32_t wt = 32u * static_cast<uint32_t>(t);
  const bool inside = wt >= kW0 && wt + 32u <= kW1;
  uint32_t c = 0, all = 0, ktop = 0;  // candidates, every count, highest candidate key + 1
  uint32_t nz = 0;                    // bit j: word 32t + j counts a candidate
  for (int j0 = 0; j0 < 32; j0 += 8) {
    uint32_t wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) wv[u] = fine[wt + ((j0 + u + t) & 31)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t jj = static_cast<uint32_t>((j0 + u + t) & 31);
      const uint32_t ws = word_sum(wv[u]);
      all += ws;
      if (inside || wt + jj - kW0 < kW1 - kW0) {
        c += ws;
        nz |= (wv[u] ? 1u : 0u) << jj;
      }
    }
  }
  if (nz) {
    const int jt = 31 - __builtin_clz(nz);
    const uint32_t w = fine[wt + jt];
    ktop = k0 + KW * jt + static_cast<uint32_t>(31 - __builtin_clz(w)) / CB + 1u;
  }
  // block totals (the shortfall of every count against the tokens counted,
  // the highest key) and suffix totals of c, high keys first
  const uint32_t pc = wave_prefix_sum(c);
  const uint32_t wc = lane63(pc);
  uint32_t sc = wc - pc + c;
  const uint32_t wd = lane63(wave_prefix_sum(allowed - all));  // 0 unless a count wrapped
  const uint32_t wk = wave_max(ktop);
  if (lane == 0) {
    s_c[wave] = wc;
    s_kmax[wave] = wk;
    s_d[wave] = wd;
  }
  __syncthreads();
  uint32_t tot_c = 0, tot_d = 0;
  ktop = 0;
  for (int w = 0; w < kWaves; ++w) {
    tot_c += s_c[w];
    tot_d += s_d[w];
    ktop = max(ktop, s_kmax[w]);
    if (w > wave) sc += s_c[w];
  }
  if (tot_d != 0) return false;  // a count wrapped
  if (tot_c == 0) {
    *best = -__builtin_inff();
    return true;
  }
  *best = D::value(static_cast<Bits>(bits_of_key16(ktop - 1)));
  const float zmax = *best * inv_t;
  const auto mass = [&](uint32_t k) { return fixed_mass(D::value(static_cast<Bits>(bits_of_key16(k))), inv_t, zmax); };
  const auto cut_of = [](uint32_t k) { return order_key(D::value(static_cast<Bits>(bits_of_key16(k)))); };

  // ---- top-p masses per thread, then their suffix totals.  The keys that
  // hold tokens crowd a narrow band, so a thread walking its own 32 words
  // would leave most waves idle while the others step through every slot of
  // theirs.  Instead, at step s each half-wave takes the 32 words of one
  // thread (word s * THREADS + t to lane t, so thread (s * THREADS + t) / 32
  // owns the half-wave's words), adds up the masses of its word's counters,
  // sums them over the half-wave and stores that thread's total; a wave whose
  // 64 words are all zero skips the step.  Every thread's total is written
  // exactly once.
  unsigned long long m = 0, sm = 0, tot_m = 0;
  if (use_p) {
    __shared__ unsigned long long s_own[THREADS];
    constexpr int kBatch = 4;  // steps per batch: their words, masses and half-wave sums side by side
    for (int s0 = 0; s0 < 32; s0 += kBatch) {
      uint32_t wb[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) wb[j] = fine[(s0 + j) * THREADS + t];
      unsigned long long mw[kBatch] = {};
      if (__ballot((wb[0] | wb[1] | wb[2] | wb[3]) != 0u)) {  // else every total of the batch is 0
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const uint32_t ka = KW * static_cast<uint32_t>((s0 + j) * THREADS + t);  // the word's first key
          if (wb[j] && in_range(ka)) {  // a word holds finite keys only or none
            // its keys have one sign, so their raw bits run from ka's up (a
            // positive value) or down (a negative one)
            const uint32_t b0 = bits_of_key16(ka), step = (ka & 0x8000u) ? 1u : ~0u;
#pragma unroll
            for (uint32_t e = 0; e < KW; ++e) {
              const uint32_t n = count_in(wb[j], e);
              if (n)
                mw[j] += static_cast<unsigned long long>(n) *
                         fixed_mass(D::value(static_cast<Bits>(b0 + e * step)), inv_t, zmax);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) mw[j] = half_wave_scan(mw[j]);  // lanes 31 and 63: each half-wave's total
      }
      if ((lane & 31) == 31) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) s_own[static_cast<uint32_t>((s0 + j) * THREADS + t) / 32u] = mw[j];
      }
    }
    __syncthreads();
    m = s_own[t];
    const unsigned long long pm = wave_prefix_sum(m);
    const unsigned long long wm = lane63(pm);
    sm = wm - pm + m;
    if (lane == 0) s_m[wave] = wm;
    __syncthreads();
    for (int w = 0; w < kWaves; ++w) {
      tot_m += s_m[w];
      if (w > wave) sm += s_m[w];
    }
  }

  // ---- each search: the thread whose keys hold the crossing posts its
  // number and the total above them; then one wave per search takes those
  // keys, KPL consecutive ones per lane, and a suffix scan finds the largest
  // key whose suffix reaches the need (top-k on wave 0, top-p on wave 1)
  const uint32_t need_k = static_cast<uint32_t>(top_k);  // more than the candidates: keep all
  const double pz = fmax(static_cast<double>(top_p), 0.0) * static_cast<double>(tot_m);
  const unsigned long long target = static_cast<unsigned long long>(ceil(pz));
  const unsigned long long need_p = target ? target : 1ull;  // p <= 0 keeps just the largest value
  if (t == 0) s_kept[0] = s_kept[1] = tot_c;  // a search without a crossing keeps every candidate
  if (use_k && need_k <= tot_c && sc >= need_k && sc - c < need_k) {
    s_cross[0] = static_cast<uint32_t>(t);
    s_above[0] = sc - c;
    s_above_n[0] = sc - c;
  }
  if (use_p && need_p <= tot_m && sm >= need_p && sm - m < need_p) {
    s_cross[1] = static_cast<uint32_t>(t);
    s_above[1] = sm - m;
    s_above_n[1] = sc - c;
  }
  __syncthreads();
  const int which = wave;  // 0: top-k, 1: top-p
  if (which < 2 && (which == 0 ? use_k : use_p) && s_cross[which] != ~0u) {
    const unsigned long long need = which == 0 ? static_cast<unsigned long long>(need_k) : need_p;
    const uint32_t kb = KPT * s_cross[which] + KPL * static_cast<uint32_t>(lane);  // this lane's first key
    uint32_t n[KPL];
    unsigned long long vv[KPL];
    unsigned long long v = 0;
    uint32_t vn = 0;  // and the candidates at and above kb
#pragma unroll
    for (uint32_t j = 0; j < KPL; ++j) {
      const uint32_t kx = kb + j;
      n[j] = in_range(kx) ? count_in(fine[kx / KW], kx) : 0u;
      vv[j] = which == 0 ? n[j] : (n[j] ? static_cast<unsigned long long>(n[j]) * mass(kx) : 0ull);
      v += vv[j];
      vn += n[j];
    }
    // suffix totals over the lanes, from prefix sums
    const unsigned long long pv = wave_prefix_sum(v);
    const uint32_t pn = wave_prefix_sum(vn);
    const unsigned long long total = lane63(pv) - pv + v + s_above[which];  // the searched total at and above kb
    vn = lane63(pn) - pn + vn;
    const uint64_t hit = __ballot(total >= need);
    const int L = 63 - __clzll(static_cast<long long>(hit));
    // within lane L: the largest of its keys whose suffix still reaches the need
    uint32_t jsel = 0, nsel = vn;
    unsigned long long acc = total;
    uint32_t accn = vn;
#pragma unroll
    for (uint32_t j = 1; j < KPL; ++j) {
      acc -= vv[j - 1];
      accn -= n[j - 1];
      if (acc >= need) {
        jsel = j;
        nsel = accn;
      }
    }
    const uint32_t key = KPT * s_cross[which] + KPL * static_cast<uint32_t>(L) +
                         static_cast<uint32_t>(__shfl(static_cast<int>(jsel), L));
    const uint32_t at_cut = static_cast<uint32_t>(__shfl(static_cast<int>(nsel), L)) + s_above_n[which];
    if (lane == 0) {
      s_cut[which] = key;  // a key: 0 (non-finite) keeps all
      s_kept[which] = at_cut;
    }
  }
  __syncthreads();
  *cut16 = max(s_cut[0], s_cut[1]);
  *cut = *cut16 ? cut_of(*cut16) : 0u;
  *kept = min(use_k ? s_kept[0] : tot_c, use_p ? s_kept[1] : tot_c);  // the tighter cut keeps fewer
  return true;
}

// ---- sparse 16-bit rows with top-k or top-p (512- and 1024-thread blocks,
// rows longer than those held in registers): when the mask allows at most
// kSparseMax tokens below V, the candidates are listed in LDS (token and
// 16-bit key) from the groups the mask allows -- the logits of other groups
// are not read -- and both cuts come from a radix select over the list
// (two 8-bit digits of the key), counting for top-k and summing the same
// fixed-point masses for top-p: the same cuts as fine_search's histogram
// over all 65536 keys, whose clearing, filling and scanning cost as much
// for a few hundred candidates as for a full row.  The draw then runs on
// the list.  A dense row pays one read of its mask words to find out.
constexpr uint32_t kSparseMax = 4096;
constexpr uint32_t kSparseSlots = 2 * kSparseMax;  // list slots, an equal region per wave
constexpr size_t sparse_lds_bytes() { return kSparseSlots * (4 + 2) + 2 * 256 * (4 + 8); }

// The row's candidates, as sparse_search left them: wave w's entries in
// slots [w * per_wave, w * per_wave + nw).
template <int THREADS>
struct SparseList {
  static constexpr uint32_t kPerWave = kSparseSlots / (THREADS / 64);
  const uint32_t* idx;   // token
  const uint16_t* key;   // 16-bit order key
  __device__ __forceinline__ explicit SparseList(const uint32_t* lds)
      : idx(lds), key(reinterpret_cast<const uint16_t*>(lds + kSparseSlots)) {}
};

// Whether the row is sparse (the mask allows at most kSparseMax tokens); if
// so, lists its candidates, sets *best (-inf without a candidate) and
// *cut16 (the lower of the two cuts as a 16-bit key, 0 to keep every
// candidate), leaves this wave's entry count in *nw and returns true.
// Otherwise returns false and only LDS has changed.  Block-uniform; ends
// with a barrier.
template <typename D, int THREADS>
__device__ __forceinline__ bool sparse_search(const RowView<D>& rv, uint32_t* lds, float inv_t, bool use_k,
                                              int32_t top_k, bool use_p, float top_p, float* best, uint32_t* cut16,
                                              uint32_t* nw_out) {
  constexpr int kWaves = THREADS / 64;
  constexpr uint32_t kPerWave = SparseList<THREADS>::kPerWave;
  static_assert(sparse_lds_bytes() <= sample_fine_bytes(THREADS), "the list fits the histogram's LDS");
  uint32_t* lidx = lds;
  uint16_t* lkey = reinterpret_cast<uint16_t*>(lds + kSparseSlots);
  uint32_t* hn = lds + kSparseSlots + kSparseSlots / 2;                  // two digits' counts
  unsigned long long* hm = reinterpret_cast<unsigned long long*>(hn + 512);  // and masses
  __shared__ uint32_t s_red[kWaves], s_cnt[kWaves];
  __shared__ SelectState s_ss;
  const int t = static_cast<int>(threadIdx.x);
  const int lane = lane_id(), wave = t >> 6;
  const int32_t nfull = rv.V >> 3;
  const int32_t ngroups = (rv.V + 7) >> 3;  // the last one partial when V % 8 != 0
  // group g's mask bits below V (a group past the row loads nothing and has none)
  const auto gbits = [&](int32_t g) {
    uint32_t b = (load_word(rv.rm, g < ngroups ? (g >> 2) * 4 : kSkip) >> ((g & 3) * 8)) & 0xFFu;
    if (g == nfull) b &= (1u << (rv.V & 7)) - 1u;
    return b;
  };
  const auto block_sum = [&](uint32_t x) {
    x = lane63(wave_prefix_sum(x));
    __syncthreads();
    if (lane == 0) s_red[wave] = x;
    __syncthreads();
    uint32_t sum = 0;
    for (int w = 0; w < kWaves; ++w) sum += s_red[w];
    return sum;
  };

  // ---- the allowed tokens' logits (only groups the mask allows are read),
  // and the candidates listed in this wave's region: allowed tokens with
  // finite values
  uint32_t nw = 0;  // this wave's entries (the same in every lane)
  uint32_t km = 0;  // the largest key this lane listed
  const uint32_t region = static_cast<uint32_t>(wave) * kPerWave;
  const auto load_values = [&](int32_t base, const uint32_t (&b)[8], uint32_t (&v)[8][4]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int32_t g = base + j * THREADS + t;
      if (rv.aligned && g < nfull) {
        const uint4 q4 = load16(rv.rl, b[j] ? g * 16 : kSkip);
        v[j][0] = q4.x;
        v[j][1] = q4.y;
        v[j][2] = q4.z;
        v[j][3] = q4.w;
      } else {  // a misaligned row, or the partial last group: the allowed tokens one by one
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
              rv.rl, ((b[j] >> (2 * q2)) & 1u) ? (8 * g + 2 * q2) * 2 : kSkip, 0, 0);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
              rv.rl, ((b[j] >> (2 * q2 + 1)) & 1u) ? (8 * g + 2 * q2 + 1) * 2 : kSkip, 0, 0);
          v[j][q2] = lo | (hi << 16);
        }
      }
    }
  };
  // Per group, the candidates as 8 bits: allowed, and finite (exponent
  // field not all ones, tested on both halves of a word at once: adding the
  // field's lowest bit to the field carries into the half's top bit only
  // when the field is full).  One prefix sum over the batch places each
  // lane's entries; then each lane walks its own candidates, so a group
  // costs its wave one step per candidate of its busiest lane rather than
  // one per token.
  const auto list_values = [&](int32_t base, const uint32_t (&b)[8], const uint32_t (&v)[8][4]) {
    constexpr uint32_t kE = D::kExp16 * 0x00010001u;                     // both halves' exponent fields
    constexpr uint32_t kL = (D::kExp16 & (~D::kExp16 + 1u)) * 0x00010001u;  // and their lowest bits
    uint32_t cand[8];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t nf = 0;  // word q2's low token non-finite: bit 2 q2; its high token: bit 16 + 2 q2
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) nf |= (((v[j][q2] & kE) + kL) & 0x80008000u) >> (15 - 2 * q2);
      cand[j] = b[j] & ~(nf | (nf >> 15));
      cnt += static_cast<uint32_t>(__builtin_popcount(cand[j]));
    }
    if (!__ballot(cnt != 0u)) return;
    const uint32_t incl = wave_prefix_sum(cnt);  // this lane's entries go after those of the lanes below it
    uint32_t pos = nw + incl - cnt;
    nw += lane63(incl);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t g = static_cast<uint32_t>(base + j * THREADS + t);
      for (uint32_t c = cand[j]; c != 0u; c &= c - 1u) {
        const uint32_t q = static_cast<uint32_t>(__builtin_ctz(c));
        const uint32_t lo = (q & 2u) ? v[j][1] : v[j][0];  // token q sits in word q / 2, half q % 2
        const uint32_t hi = (q & 2u) ? v[j][3] : v[j][2];
        const uint32_t key = order_key16x2((((q & 4u) ? hi : lo) >> ((q & 1u) * 16u)) & 0xFFFFu) & 0xFFFFu;
        if (pos < kPerWave) {
          lidx[region + pos] = 8u * g + q;
          lkey[region + pos] = static_cast<uint16_t>(key);
        }
        km = max(km, key);
        ++pos;
      }
    }
  };
  // the count first, from the mask alone: a dense row reads no logits here;
  // meanwhile both digits' histograms of the select are cleared
  for (int i = t; i < 512; i += THREADS) {
    hn[i] = 0u;
    hm[i] = 0ull;
  }
  uint32_t allowed = 0;
  *cut16 = 0u;
  *nw_out = 0u;
  if (ngroups <= 16 * THREADS) {
    // at most two batches of groups: their mask bytes, all requested at
    // once, stay in registers from the count to the listing
    const int nb = ngroups <= 8 * THREADS ? 1 : 2;
    uint32_t b[2][8] = {};
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (h < nb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[h][j] = gbits((8 * h + j) * THREADS + t);
      }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) allowed += __builtin_popcount(b[h][j]);
    allowed = block_sum(allowed);
    if (allowed > kSparseMax) return false;
    if (allowed == 0u) {  // nothing allowed: no candidate
      *best = -__builtin_inff();
      return true;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (h < nb) {
        uint32_t v[8][4];
        load_values(8 * h * THREADS, b[h], v);
        list_values(8 * h * THREADS, b[h], v);
      }
  } else {
    for (int32_t base = 0; base < ngroups; base += 8 * THREADS) {
      uint32_t b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = gbits(base + j * THREADS + t);
#pragma unroll
      for (int j = 0; j < 8; ++j) allowed += __builtin_popcount(b[j]);
    }
    allowed = block_sum(allowed);
    if (allowed > kSparseMax) return false;
    if (allowed == 0u) {
      *best = -__builtin_inff();
      return true;
    }
    for (int32_t base = 0; base < ngroups; base += 8 * THREADS) {
      uint32_t b[8], v[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = gbits(base + j * THREADS + t);
      load_values(base, b, v);
      list_values(base, b, v);
    }
  }

  // ---- the largest candidate and the candidate count (a wave whose region
  // overflowed sends the row to the histogram search)
  km = wave_max(km);
  __syncthreads();
  if (lane == 0) {
    s_red[wave] = km;
    s_cnt[wave] = nw;
  }
  __syncthreads();
  km = 0;
  uint32_t ntot = 0;
  bool over = false;
  for (int w = 0; w < kWaves; ++w) {
    km = max(km, s_red[w]);
    ntot += s_cnt[w];
    over |= s_cnt[w] > kPerWave;
  }
  if (over) return false;
  *nw_out = nw;
  if (km == 0u) {  // every allowed token non-finite
    *best = -__builtin_inff();
    return true;
  }
  *best = D::value(static_cast<typename D::Bits>(bits_of_key16(km)));
  const float zmax = *best * inv_t;
  const auto mass = [&](uint32_t k) {
    return fixed_mass(D::value(static_cast<typename D::Bits>(bits_of_key16(k))), inv_t, zmax);
  };

  // ---- the cuts: a radix select over the list (the high digit of the
  // 16-bit key, then the low one under the chosen prefix), top-k by counts,
  // top-p by masses; the first digit's mass histogram holds every
  // candidate, so its total is Z
  const bool do_k = use_k && static_cast<uint32_t>(top_k) <= ntot;  // k beyond the candidates keeps all
  if (!do_k && !use_p) return true;
  if (t == 0) s_ss = SelectState{0u, static_cast<uint32_t>(top_k), 0ull, 0u};
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 8 : 0;
    const uint32_t pmask = pass == 0 ? 0u : 0xFF00u;
    uint32_t* h_n = hn + 256 * pass;
    unsigned long long* h_m = hm + 256 * pass;
    const uint32_t pk = pass == 0 ? 0u : s_ss.prefix_k, pp = pass == 0 ? 0u : s_ss.prefix_p;
    for (uint32_t i = static_cast<uint32_t>(lane); i < nw; i += 64u) {
      const uint32_t key = lkey[region + i];
      const uint32_t d = (key >> shift) & 255u;
      if (do_k && (key & pmask) == pk) atomicAdd(&h_n[d], 1u);
      if (use_p && (key & pmask) == pp) {
        const uint32_t m = mass(key);
        if (m) atomicAdd(&h_m[d], static_cast<unsigned long long>(m));
      }
    }
    __syncthreads();
    if (do_k && wave == 0) {
      const WaveSuffix<uint32_t> ws(h_n);
      int d;
      uint32_t ab;
      ws.pick(s_ss.need_k, &d, &ab);
      if (lane == 0) {
        s_ss.prefix_k |= static_cast<uint32_t>(d) << shift;
        s_ss.need_k -= ab;
      }
    }
    if (use_p && wave == 1) {
      const WaveSuffix<unsigned long long> ws(h_m);
      unsigned long long need = s_ss.need_p;
      if (pass == 0) {
        // p <= 0 keeps just the largest value, as p = 0 does: any mass reaches it
        const double pz = fmax(static_cast<double>(top_p), 0.0) * static_cast<double>(ws.total());
        const unsigned long long target = static_cast<unsigned long long>(ceil(pz));
        need = target ? target : 1ull;
      }
      int d;
      unsigned long long ab;
      ws.pick(need, &d, &ab);
      if (lane == 0) {
        s_ss.prefix_p |= static_cast<uint32_t>(d) << shift;
        s_ss.need_p = need - ab;
      }
    }
    __syncthreads();
  }
  *cut16 = max(do_k ? s_ss.prefix_k : 0u, use_p ? s_ss.prefix_p : 0u);
  return true;
}

// ---- fp32 rows with top-k or top-p, in 1024-thread blocks: the cut from one
// coarse pass and a list of the tokens in the bucket that holds it.
//
// The coarse pass counts every candidate (for top-k) and sums its fixed-point
// mass (for top-p) under the top 12 bits of its order key: 4096 buckets of an
// eighth of a binade, in LDS.  A search over them finds each cut's bucket and
// the count or mass above it.  The draw pass then keeps every candidate above
// the higher of the two buckets whatever the rest of its key is, drops every
// candidate below it, and lists the candidates inside it (order key and
// index) in LDS; a radix select over the list's low 20 key bits, three
// digits, gives the exact cut, and the listed tokens at or above it join the
// draw.  Two passes over the row for top-k and top-p alike -- against five and
// three for a radix search over the row: where top-p or min-p needs the row's
// maximum, the coarse pass finds it too, summing each bucket's masses
// relative to the bucket's largest value (edge_mass) and rescaling the sums
// to the maximum afterwards (edge_to_max_units).  A bucket holding more
// candidates than the list has room for sends the row to the radix search.
constexpr int kCoarseBuckets = 4096;
constexpr uint32_t kCoarseShift = 20;  // bucket = order key >> 20
// The list: one region per wave of the 1024-thread block, each wave appending
// to its own (no atomics); a wave that fills its region sends the row to the
// radix search.
constexpr uint32_t kCoarseListWaves = 16;
constexpr uint32_t kCoarseListPerWave = 960;
constexpr uint32_t kCoarseListCap = kCoarseListWaves * kCoarseListPerWave;  // 15360 keys and indices, 120 KB

// Dynamic LDS of the fp32 1024-thread kernel this path uses (it has the
// 131 KB of the 16-bit search): the coarse masses and counts (48 KB), then,
// reusing the space, the list and the list search's 256-bin histograms.
constexpr size_t coarse_lds_bytes() {
  const size_t hist = static_cast<size_t>(kCoarseBuckets) * (sizeof(unsigned long long) + sizeof(uint32_t));
  const size_t list = static_cast<size_t>(kCoarseListCap) * 2 * sizeof(uint32_t) + 256 * (sizeof(unsigned long long) + sizeof(uint32_t));
  return hist > list ? hist : list;
}

// The float whose order key is k (the inverse of order_key; the key of -0 is
// that of +0 and maps back to +0).
__device__ __forceinline__ float value_of_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// A candidate's softmax mass relative to the largest value e of its coarse
// bucket, in fixed point: 2^45 exp((x - e) / T), computed as the hardware
// base-2 exponential of (x - e) log2(e) / T.  x - e is exact (the two share
// a binade).  A mass of at most 2^45 summed over at most 2^18 candidates
// stays below 2^63.
constexpr int kEdgeMassBits = 45;
constexpr int32_t kEdgeMassMaxTokens = 1 << 18;
__device__ __forceinline__ unsigned long long edge_mass(float x, float e, float c) {
  // f in [0, 1]; floor(2^45 f) is its 24-bit significand placed 32 bits up
  // and shifted right by 10 - (f's exponent): a shift past 63 (f below
  // 2^-53, a subnormal or 0, or NaN) leaves 0
  const uint32_t b = __float_as_uint(__builtin_amdgcn_exp2f((x - e) * c));
  const uint32_t sh = 137u - (b >> 23);
  const unsigned long long sig = static_cast<unsigned long long>((b & 0x7FFFFFu) | 0x800000u) << 32;
  return sh < 64u ? sig >> sh : 0ull;
}

// One pass over an fp32 row: every candidate (mask bit set, finite) adds 1
// to cc[bucket] when use_k and its fixed-point mass to cm[bucket] when use_p,
// from a cleared start.  The mass is 2^31 exp(z - z_max) (fixed_mass) when
// the maximum is known (edge == false), else edge_mass, relative to the
// largest value of the candidate's own bucket, and the pass also finds the
// largest candidate.  Returns the order key of the largest candidate (0 when
// there is none; edge mode only).  Ends with a barrier.
template <int THREADS>
__device__ __forceinline__ uint32_t coarse_hist32(const RowView<F32Bits>& rv, unsigned long long* cm, uint32_t* cc,
                                                  bool use_k, bool use_p, float inv_t, float zmax, bool edge) {
  __shared__ uint32_t s_kmax[THREADS / 64];
  const int t = static_cast<int>(threadIdx.x);
  for (int i = t; i < kCoarseBuckets; i += THREADS) {
    cm[i] = 0ull;
    cc[i] = 0u;
  }
  __syncthreads();
  const float c = inv_t * 1.4426950408889634f;
  uint32_t kmax = 0;  // every finite value's key is at least 0x00800000
  const auto add = [&](uint32_t xb, uint32_t bit) {
    const float x = __uint_as_float(xb);
    const uint32_t key = order_key(x);
    if (bit && finite_key(key)) {
      const uint32_t b = key >> kCoarseShift;
      if (edge) kmax = max(kmax, key);
      if (use_k) atomicAdd(&cc[b], 1u);
      if (use_p) {
        if (edge) {
          const unsigned long long m = edge_mass(x, value_of_key(key | ((1u << kCoarseShift) - 1u)), c);
          if (m) atomicAdd(&cm[b], m);
        } else {
          const uint32_t m = fixed_mass(x, inv_t, zmax);  // one that truncates to 0 adds nothing
          if (m) atomicAdd(&cm[b], static_cast<unsigned long long>(m));
        }
      }
    }
  };
  walk_row_raw<128, THREADS>(rv, [&](int32_t g, const typename RowView<F32Bits>::Raw& raw, bool full) {
    const uint32_t bits = rv.mask_bits(raw, g, full);
#pragma unroll
    for (int q = 0; q < 8; ++q) add(raw.v[q], (bits >> q) & 1u);
  });
  if ((rv.V & 7) && t == 0) {  // the partial last group, by plain loads
    for (int32_t i = rv.V & ~7; i < rv.V; ++i)
      add(rv.row[i], rv.has_mask ? (load_word(rv.rm, (i >> 5) * 4) >> (i & 31)) & 1u : 1u);
  }
  if (edge) {
    kmax = wave_max(kmax);
    if (lane_id() == 0) s_kmax[t >> 6] = kmax;
  }
  __syncthreads();
  if (edge) {
    kmax = 0;
    for (int w = 0; w < THREADS / 64; ++w) kmax = max(kmax, s_kmax[w]);
  }
  return kmax;
}

// After coarse_hist32 in edge mode, with the largest candidate xmax known:
// each bucket's mass sum rescaled to 2^31 exp(z - z_max) units, the units
// of fixed_mass, by exp((e_b - xmax) / T) 2^(31 - 45) in double precision
// (e_b the bucket's largest value), thread t of 1024 taking buckets 4t ..
// 4t + 3.  Ends with a barrier.
__device__ __forceinline__ void edge_to_max_units(unsigned long long* cm, float inv_t, float xmax) {
  const double c = static_cast<double>(inv_t * 1.4426950408889634f);
  const int t = static_cast<int>(threadIdx.x);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t b = 4u * static_cast<uint32_t>(t) + static_cast<uint32_t>(j);
    const unsigned long long m = cm[b];
    if (m) {
      const double e = static_cast<double>(value_of_key((b << kCoarseShift) | ((1u << kCoarseShift) - 1u)));
      const double f = exp2((e - static_cast<double>(xmax)) * c + static_cast<double>(31 - kEdgeMassBits));
      cm[b] = static_cast<unsigned long long>(static_cast<double>(m) * f);
    }
  }
  __syncthreads();
}

// Over h[0 .. 4095] (thread t of 1024 holds buckets 4t .. 4t + 3), with
// S(b) = h[b] + ... + h[4095] and need = need_of(S(0)): the largest b with
// S(b) >= need, and *above = S(b + 1); ~0u (no cut) when need is 0 or above
// S(0).  *need_out gets need.  Ends with a barrier.
template <typename T, typename NeedOf>
__device__ __forceinline__ uint32_t coarse_search(const T* h, NeedOf&& need_of, T* above, T* need_out) {
  constexpr int kWaves = 16;
  __shared__ T s_w[kWaves];
  __shared__ T s_ab;
  __shared__ uint32_t s_b;
  const int t = static_cast<int>(threadIdx.x);
  const int lane = lane_id(), wave = t >> 6;
  T hv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) hv[j] = h[4 * t + j];
  const T c = hv[0] + hv[1] + hv[2] + hv[3];
  T sc = c;  // suffix total from this thread's buckets up
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T v = __shfl_down(sc, o);
    if (lane + o < 64) sc += v;
  }
  if (lane == 0) s_w[wave] = sc;
  if (t == 0) {
    s_b = ~0u;
    s_ab = 0;
  }
  __syncthreads();
  T tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    tot += s_w[w];
    if (w > wave) sc += s_w[w];
  }
  const T need = need_of(tot);
  if (need != 0 && need <= tot && sc >= need && sc - c < need) {  // one thread: sc falls with t
    T acc = sc - c;  // S(4t + 4)
    uint32_t b = 4u * static_cast<uint32_t>(t);
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (acc + hv[j] >= need) {
        b = 4u * static_cast<uint32_t>(t) + static_cast<uint32_t>(j);
        break;
      }
      acc += hv[j];
    }
    s_b = b;
    s_ab = acc;
  }
  __syncthreads();
  *above = s_ab;
  *need_out = need;
  return s_b;
}

// ---- Filtered 16-bit rows split over several blocks (few rows).
//
// A batch of a few rows with top-k, top-p or min-p would otherwise keep one
// compute unit per row busy while the rest idle.  Such rows are instead
// spread over a caller's workspace in three launches, between split_clear
// (which zeroes it and the output words) and finish_tokens:
//   split_hist    one 1024-thread block per segment of a row counts the
//                 segment's allowed tokens under their 16-bit keys (LDS,
//                 16-bit counters: a segment holds fewer than 65536 tokens)
//                 and adds its nonzero counts into the row's histogram of
//                 65536 32-bit counts in the workspace, two adjacent keys per
//                 64-bit atomic (a count stays below 2^28, so the low one
//                 never carries into the high one); it also marks each run
//                 of 64 keys that received a count in the row's 1024-bit map;
//   split_search  one block per row finds the maximum and the top-k / top-p
//                 cuts from those counts, exactly as fine_search does from
//                 its LDS histogram (same counts, same fixed-point masses, so
//                 the same cut), reading only the marked runs, and stores the
//                 result per row;
//   sample_rows   one block per segment draws over its segment with that
//                 cut, the segments merging through the row's output word.
// Workspace layout: every row's histogram (65536 words, key k at word k),
// then every row's run map (32 words), then one SplitInfo per row.

// The split search's result for one row.
struct SplitInfo {
  uint32_t cut16;  // keep the candidates whose 16-bit key is at least cut16 (0: every one)
  float best;      // the largest candidate; -inf when the row has none
  uint32_t kept;   // the candidates the cut keeps
  uint32_t pad;
};
constexpr int64_t kSplitHistWords = 65536;
constexpr int64_t kSplitMapWords = 32;
constexpr int64_t split_workspace_bytes(int64_t rows) {
  return rows * ((kSplitHistWords + kSplitMapWords) * 4 + static_cast<int64_t>(sizeof(SplitInfo)));
}

// Whether row r takes the split filtered path: a positive temperature with
// top-k, top-p or min-p in force (the same tests sample_rows makes).
__device__ __forceinline__ bool split_filtered_row(const SampleArgs& a, int64_t r) {
  const float temp = a.temperature ? a.temperature[r] : a.temperature_all;
  const int32_t top_k = a.top_k ? a.top_k[r] : a.top_k_all;
  const float top_p = a.top_p ? a.top_p[r] : a.top_p_all;
  const float min_p = a.min_p ? a.min_p[r] : a.min_p_all;
  const float inv_t = 1.0f / temp;
  return temp > 0.f && ((top_k > 0 && inv_t > 0.f) || (top_p < 1.0f && inv_t > 0.f) || min_p > 0.f);
}

// Before a split filtered launch: the histograms, run maps and output words
// at 0.  A kernel rather than a memset, so graphs replay it.
__global__ void split_clear(uint4* __restrict__ ws, int64_t n16, int64_t* __restrict__ out, int64_t rows) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    ws[i] = make_uint4(0u, 0u, 0u, 0u);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < rows) out[i] = 0;
}

// One segment of a filtered row: its 16-bit key counts, added into the row's
// workspace histogram (hist, rows x 65536 words) and run map (map, rows x 32
// words).  Block b is segment b % nseg of row b / nseg; seg_len is a
// multiple of 256 below 65536.
template <typename D>
__global__ __launch_bounds__(1024) void split_hist(const typename D::Bits* __restrict__ logits, int64_t ls,
                                                   const uint32_t* __restrict__ mask, int64_t ms, int32_t V,
                                                   SampleArgs a, int32_t nseg, int32_t seg_len,
                                                   uint32_t* __restrict__ hist, uint32_t* __restrict__ map) {
  extern __shared__ unsigned long long s_dyn[];
  const int64_t r = blockIdx.x / nseg;
  const int32_t tok0 = static_cast<int32_t>(blockIdx.x % nseg) * seg_len;
  if (!split_filtered_row(a, r) || tok0 >= V) return;  // uniform across the block
  const RowView<D> rv(logits + r * ls + tok0, mask ? mask + r * ms + tok0 / 32 : nullptr, min(seg_len, V - tok0));
  uint32_t* fine = reinterpret_cast<uint32_t*>(s_dyn);
  const typename RowView<D>::Raw pre[4] = {};
  count_keys<D, 64, 1024, 16>(rv, fine, pre, false);  // 4 groups in flight: a segment holds few per thread
  // Word 1024 j + t (keys 2 (1024 j + t) and the next) is added by thread
  // t, so the nonzero words, which crowd a narrow range of keys, spread over
  // every thread.  Its run of 64 keys, 32 j + t / 32, is bit t / 32 of map
  // word j: a wave marks its two runs per j by one ballot, in an LDS copy
  // of the map first.
  __shared__ uint32_t s_map[32];
  const int t = static_cast<int>(threadIdx.x);
  const int wave = t >> 6;
  if (t < 32) s_map[t] = 0u;
  __syncthreads();
  unsigned long long* h2 = reinterpret_cast<unsigned long long*>(hist + r * kSplitHistWords);
  uint32_t w[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) w[j] = fine[j * 1024 + t];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint64_t b = __ballot(w[j] != 0u);
    if (lane_id() == 0 && b)
      atomicOr(&s_map[j], ((static_cast<uint32_t>(b) ? 1u : 0u) << (2 * wave)) |
                              ((static_cast<uint32_t>(b >> 32) ? 1u : 0u) << (2 * wave + 1)));
    if (w[j]) atomicAdd(h2 + j * 1024 + t, (static_cast<unsigned long long>(w[j] >> 16) << 32) | (w[j] & 0xFFFFu));
  }
  __syncthreads();
  if (t < 32 && s_map[t]) atomicOr(map + r * kSplitMapWords + t, s_map[t]);
}

// One block per row of the split batch: the largest candidate and the top-k
// and top-p cuts from the row's workspace histogram, into info[r].  The
// same search as fine_search, on 32-bit counts that never wrap; thread t
// holds keys [64t, 64t + 64) and reads them only when the run map marks
// them.
template <typename D>
__global__ __launch_bounds__(1024) void split_search(SampleArgs a, const uint32_t* __restrict__ hist,
                                                     const uint32_t* __restrict__ map,
                                                     SplitInfo* __restrict__ info) {
  using Bits = typename D::Bits;
  constexpr int kWaves = 16;
  constexpr uint32_t kSpan = D::kKey16Hi - D::kKey16Lo;
  static_assert(D::kKey16Lo % 64 == 0 && (D::kKey16Hi + 1) % 64 == 0, "a thread's keys are all finite or none");
  __shared__ uint32_t s_kmax[kWaves], s_c[kWaves], s_cut[2], s_cross[2], s_above_n[2], s_kept[2];
  __shared__ unsigned long long s_m[kWaves], s_above[2];
  const int64_t r = blockIdx.x;
  if (!split_filtered_row(a, r)) return;  // uniform across the block
  const float temp = a.temperature ? a.temperature[r] : a.temperature_all;
  const int32_t top_k = a.top_k ? a.top_k[r] : a.top_k_all;
  const float top_p = a.top_p ? a.top_p[r] : a.top_p_all;
  const float inv_t = 1.0f / temp;
  const bool use_k = top_k > 0 && inv_t > 0.f;
  const bool use_p = top_p < 1.0f && inv_t > 0.f;
  const uint32_t* h = hist + r * kSplitHistWords;
  const int t = static_cast<int>(threadIdx.x);
  const int lane = lane_id(), wave = t >> 6;
  const uint32_t k0 = 64u * static_cast<uint32_t>(t);
  const auto in_range = [](uint32_t k) { return k - D::kKey16Lo <= kSpan; };
  const bool marked = (map[r * kSplitMapWords + (t >> 5)] >> (t & 31)) & 1u;
  const uint4* h4 = reinterpret_cast<const uint4*>(h + k0);
  if (t < 2) {
    s_cut[t] = 0u;
    s_cross[t] = ~0u;  // no crossing: keep every candidate
  }

  // ---- this thread's candidates and highest candidate key, all 64 counts
  // loaded at once
  uint32_t c = 0, ktop = 0;
  if (marked) {
    uint4 q[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) q[u] = h4[u];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t n4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = k0 + 4u * u + e;
        if (n4[e] && in_range(k)) {
          c += n4[e];
          ktop = k + 1;
        }
      }
    }
  }
  uint32_t sc = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t vc = static_cast<uint32_t>(__shfl_down(static_cast<int>(sc), o));
    if (lane + o < 64) sc += vc;
    ktop = max(ktop, static_cast<uint32_t>(__shfl_xor(static_cast<int>(ktop), o)));
  }
  if (lane == 0) {
    s_c[wave] = sc;
    s_kmax[wave] = ktop;
  }
  __syncthreads();
  uint32_t tot_c = 0;
  ktop = 0;
  for (int w = 0; w < kWaves; ++w) {
    tot_c += s_c[w];
    ktop = max(ktop, s_kmax[w]);
    if (w > wave) sc += s_c[w];
  }
  if (tot_c == 0) {
    if (t == 0) info[r] = SplitInfo{0u, -__builtin_inff(), 0u, 0u};
    return;
  }
  const float best = D::value(static_cast<Bits>(bits_of_key16(ktop - 1)));
  const float zmax = best * inv_t;
  const auto mass = [&](uint32_t k) { return fixed_mass(D::value(static_cast<Bits>(bits_of_key16(k))), inv_t, zmax); };

  // ---- top-p masses per thread (the counts read again), then their suffix totals
  unsigned long long m = 0, sm = 0, tot_m = 0;
  if (use_p) {
    if (marked && c) {  // c > 0: the thread's 64 keys are finite (they share one sign and finiteness)
      uint4 q[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) q[u] = h4[u];
      // raw bits run from k0's up (a positive value) or down (a negative one)
      const uint32_t b0 = bits_of_key16(k0), step = (k0 & 0x8000u) ? 1u : ~0u;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint32_t n4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n4[e])
            m += static_cast<unsigned long long>(n4[e]) *
                 fixed_mass(D::value(static_cast<Bits>(b0 + (4u * u + e) * step)), inv_t, zmax);
        }
      }
    }
    sm = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long vm = __shfl_down(sm, o);
      if (lane + o < 64) sm += vm;
    }
    if (lane == 0) s_m[wave] = sm;
    __syncthreads();
    for (int w = 0; w < kWaves; ++w) {
      tot_m += s_m[w];
      if (w > wave) sm += s_m[w];
    }
  }

  // ---- the crossing thread posts itself; one wave per search then takes
  // its 64 keys, one per lane (top-k on wave 0, top-p on wave 1)
  const uint32_t need_k = static_cast<uint32_t>(top_k);  // more than the candidates: keep all
  const double pz = fmax(static_cast<double>(top_p), 0.0) * static_cast<double>(tot_m);
  const unsigned long long target = static_cast<unsigned long long>(ceil(pz));
  const unsigned long long need_p = target ? target : 1ull;  // p <= 0 keeps just the largest value
  if (t == 0) s_kept[0] = s_kept[1] = tot_c;  // a search without a crossing keeps every candidate
  if (use_k && need_k <= tot_c && sc >= need_k && sc - c < need_k) {
    s_cross[0] = static_cast<uint32_t>(t);
    s_above[0] = sc - c;
    s_above_n[0] = sc - c;
  }
  if (use_p && need_p <= tot_m && sm >= need_p && sm - m < need_p) {
    s_cross[1] = static_cast<uint32_t>(t);
    s_above[1] = sm - m;
    s_above_n[1] = sc - c;
  }
  __syncthreads();
  const int which = wave;
  if (which < 2 && (which == 0 ? use_k : use_p) && s_cross[which] != ~0u) {
    const uint32_t kx = 64u * s_cross[which] + static_cast<uint32_t>(lane);
    const uint32_t n = in_range(kx) ? h[kx] : 0u;
    unsigned long long v = which == 0 ? n : (n ? static_cast<unsigned long long>(n) * mass(kx) : 0ull);
    uint32_t vn = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long u = __shfl_down(v, o);
      const uint32_t un = static_cast<uint32_t>(__shfl_down(static_cast<int>(vn), o));
      if (lane + o < 64) {
        v += u;
        vn += un;
      }
    }
    const unsigned long long total = v + s_above[which];
    const uint64_t hit = __ballot(total >= (which == 0 ? static_cast<unsigned long long>(need_k) : need_p));
    const int L = 63 - __clzll(static_cast<long long>(hit));
    const uint32_t at_cut = static_cast<uint32_t>(__shfl(static_cast<int>(vn), L)) + s_above_n[which];
    if (lane == 0) {
      s_cut[which] = 64u * s_cross[which] + static_cast<uint32_t>(L);
      s_kept[which] = at_cut;
    }
  }
  __syncthreads();
  if (t == 0) {
    const uint32_t kept = min(use_k ? s_kept[0] : tot_c, use_p ? s_kept[1] : tot_c);
    info[r] = SplitInfo{max(s_cut[0], s_cut[1]), best, kept, 0u};
  }
}

// The row's largest candidate and the lowest index holding it (-inf and
// 0x7FFFFFFF when there is none), in every thread; every thread of the
// block calls it (barriers).
//
// Fast form: each group's tokens are gated by their mask bits (others
// -inf) and reduced by a max tree; a thread keeps its best value and the
// words of the group holding it, and decodes that one group at the end
// for the lowest index with that value.  A group maximum that is NaN or
// +inf (possible only for rows holding such logits, which are not
// candidates) sends the whole block through the exact per-token form.
template <int BYTES, int THREADS, typename D>
__device__ __forceinline__ void row_max(const RowView<D>& rv, float* best_out, int32_t* besti_out) {
  constexpr int kWaves = THREADS / 64;
  __shared__ float s_best[kWaves];
  __shared__ int32_t s_besti[kWaves];
  const int t = static_cast<int>(threadIdx.x);
  float best = -__builtin_inff();
  int32_t besti = 0x7FFFFFFF;
  int32_t bestg = -1;
  typename RowView<D>::Raw braw{};  // the best group's words, kept so it need not be read again
  bool odd = false;
  walk_row_raw<BYTES, THREADS>(rv, [&](int32_t g, const typename RowView<D>::Raw& raw, bool full) {
    float xv[8];
    rv.gated(raw, g, full, xv);
    const float gm = fmaxf(fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3])),
                           fmaxf(fmaxf(xv[4], xv[5]), fmaxf(xv[6], xv[7])));
    odd |= !(gm < __builtin_inff()) && gm != -__builtin_inff();  // NaN or +inf
    if (gm > best) {  // strictly greater: each thread sees its groups in order
      best = gm;
      bestg = g;
      braw = raw;
    }
  });
  const int32_t tail_g = rv.V >> 3;  // the partial last group, if V % 8 != 0 (thread 0's)
  float tx[8] = {};
  const uint32_t tok = (rv.V & 7) && t == 0 ? rv.load_tail(tx) : 0u;
  if (tok) {
    float gm = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if ((tok >> q) & 1u) gm = fmaxf(gm, tx[q]);
    if (gm > best) {
      best = gm;
      bestg = tail_g;
    }
  }
  if (__syncthreads_or(odd)) {
    best = -__builtin_inff();
    walk_row<BYTES, THREADS>(rv, [&](int32_t i0, const float* x, uint32_t ok) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (((ok >> q) & 1u) && x[q] > best) {
          best = x[q];
          besti = i0 + q;
        }
    });
  } else if (bestg >= 0) {
    float x[8];
    uint32_t ok;
    if (bestg == tail_g && (rv.V & 7)) {
      ok = tok;
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = tx[q];
    } else {
      ok = rv.decode(braw, bestg, true, x);
    }
    for (int q = 7; q >= 0; --q)  // the lowest index holding the best value
      if (((ok >> q) & 1u) && x[q] == best) besti = 8 * bestg + q;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int32_t oi = __shfl_xor(besti, o);
    if (ob > best || (ob == best && oi < besti)) {
      best = ob;
      besti = oi;
    }
  }
  if (lane_id() == 0) {
    s_best[t >> 6] = best;
    s_besti[t >> 6] = besti;
  }
  __syncthreads();
  best = s_best[0];
  besti = s_besti[0];
  for (int w = 1; w < kWaves; ++w) {
    if (s_best[w] > best || (s_best[w] == best && s_besti[w] < besti)) {
      best = s_best[w];
      besti = s_besti[w];
    }
  }
  *best_out = best;
  *besti_out = besti;
}

// Greedy rows only (no row has a positive temperature): the max pass of
// sample_rows alone, in a kernel without the filtered paths, so it holds
// few registers and keeps BYTES of logits in flight per thread.  The same
// rows, segments, output and atomic merge as sample_rows.
template <typename D, int BYTES, int THREADS>
__global__ __launch_bounds__(THREADS) void greedy_rows(const typename D::Bits* __restrict__ logits, int64_t ls,
                                                       const uint32_t* __restrict__ mask, int64_t ms, int32_t V,
                                                       int64_t* __restrict__ out, int32_t nseg, int32_t seg_len) {
  const bool split = nseg > 1;
  const int64_t r = split ? blockIdx.x / nseg : blockIdx.x;
  const int32_t tok0 = split ? static_cast<int32_t>(blockIdx.x % nseg) * seg_len : 0;  // segment start
  const RowView<D> rv(logits + r * ls + tok0, mask ? mask + r * ms + tok0 / 32 : nullptr,
                      split ? min(seg_len, V - tok0) : V);
  float best;
  int32_t besti;
  row_max<BYTES, THREADS>(rv, &best, &besti);
  if (threadIdx.x == 0) {
    const bool none = best == -__builtin_inff();  // candidates are finite
    if (!split) {
      out[r] = none ? -1 : besti;
    } else if (!none) {
      const unsigned long long packed = (static_cast<unsigned long long>(order_key(best)) << 32) |
                                        static_cast<uint32_t>(~static_cast<uint32_t>(tok0 + besti));
      atomicMax(reinterpret_cast<unsigned long long*>(out) + r, packed);
    }
  }
}

// ---- Heavy rows first, for large filtered batches.  A block's time on a
// filtered row grows with what its mask allows: a row allowing more than
// kSparseMax tokens builds the full key histogram and, under top-p or
// min-p, may draw over most of its tokens, while a sparse row lists a few
// thousand candidates.  With more rows than resident blocks, blocks start
// in grid order and the hardware fills each compute unit's slots as they
// free up, so in a batch that mixes the two kinds at random some units get
// two heavy rows at once, or a heavy row late, and set the launch's end.
// row_classes marks the heavy rows; sample_rows then hands them out first,
// in row order, then the rest.  Rows are independent, so the tokens do not
// change with the order.

// Bit r of the flags (32-bit words, bit r % 32 of word r / 32) = row r's
// mask allows more than kSparseMax tokens below V.  One wave per row, 8
// rows to a 512-thread block, which stores their 8 bits as one byte.  A
// wave requests 64 PER_LANE mask words at once (PER_LANE 16: 32768 tokens,
// 32: 65536, 64: 131072) through a buffer resource that ends at the row's
// last word (loads past it return 0), and a longer row in further such
// batches until its count passes kSparseMax.
template <int PER_LANE>
__global__ __launch_bounds__(512) void row_classes(const uint32_t* __restrict__ mask, int64_t ms, int32_t V,
                                                   int32_t rows, uint8_t* __restrict__ flags) {
  __shared__ uint32_t s_flag[8];
  const int32_t wave = static_cast<int32_t>(threadIdx.x >> 6);
  const int32_t r = static_cast<int32_t>(blockIdx.x) * 8 + wave;
  const int32_t lane = static_cast<int32_t>(threadIdx.x & 63u);
  const int32_t W = (V + 31) / 32;
  // a wave past the last row reads nothing (a resource of size 0)
  const Rsrc rm = make_rsrc(r < rows ? mask + static_cast<int64_t>(r) * ms : mask,
                            r < rows ? static_cast<uint32_t>(W) * 4u : 0u);
  const uint32_t tail = (V & 31) ? (1u << (V & 31)) - 1u : ~0u;  // bits of the last word below V
  uint32_t total = 0;
  for (int32_t base = 0; base < W && total <= kSparseMax; base += 64 * PER_LANE) {  // uniform in the wave
    uint32_t x[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) x[j] = load_word(rm, (base + lane + 64 * j) * 4);
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) n += __builtin_popcount(base + lane + 64 * j == W - 1 ? x[j] & tail : x[j]);
    total += lane63(wave_prefix_sum(n));
  }
  if (lane == 0) s_flag[wave] = total > kSparseMax ? 1u : 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t bits = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) bits |= s_flag[w] << w;
    flags[blockIdx.x] = static_cast<uint8_t>(bits);
  }
}

// Bytes of the flags of n rows as row_classes stores them.
constexpr int64_t row_class_bytes(int64_t n) { return (n + 7) / 8; }

// The row block b takes when the heavy rows go first: the b-th heavy row
// of the n, or the (b - heavy rows)-th of the others, each in row order.
// Every wave works it out alone from the flag words (n <= 8192: lane l
// reads words 4 l to 4 l + 3, rows 128 l to 128 l + 127, as one 16-byte
// load; bits at or past n are ignored), with one wave prefix sum, so the
// block needs no barrier.  The result is the same in every lane and kept
// scalar, so that the row's addresses stay in scalar registers.  *dense
// says whether the row is a heavy one (its mask allows more than
// kSparseMax tokens).
__device__ __forceinline__ int64_t heavy_first_row(const uint32_t* __restrict__ flags, uint32_t n, uint32_t b,
                                                   bool* dense) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint4 f = load16(make_rsrc(flags, static_cast<uint32_t>((row_class_bytes(n) + 15) / 16 * 16)),
                         static_cast<int32_t>(16u * lane));
  const uint32_t lo = min(n, 128u * lane);
  const uint32_t w[4] = {f.x, f.y, f.z, f.w};
  uint32_t m[4], c = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t valid = min(32u, n - min(n, lo + 32u * k));  // rows of word k below n
    m[k] = valid == 32u ? ~0u : (1u << valid) - 1u;
    c += static_cast<uint32_t>(__builtin_popcount(w[k] & m[k]));
  }
  const uint32_t rows_here = min(n, lo + 128u) - lo;
  const uint32_t incl = wave_prefix_sum(c);
  const uint32_t total = lane63(incl), hb = incl - c;  // heavy rows in all, and below lo
  const bool heavy = b < total;
  *dense = heavy;
  const uint32_t j = heavy ? b - hb : b - total - (lo - hb);  // rank among this lane's heavy / light rows
  const bool mine = heavy ? (hb <= b && b < incl) : (b >= total && lo - hb <= b - total && j < rows_here - c);
  // this lane's j-th heavy (or light) row
  uint32_t row = 0, k_left = j;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t x = (heavy ? w[k] : ~w[k]) & m[k];
    const uint32_t cnt = static_cast<uint32_t>(__builtin_popcount(x));
    if (k_left < cnt && row == 0u) {
      for (uint32_t q = k_left; q; --q) x &= x - 1u;
      row = lo + 32u * k + static_cast<uint32_t>(__builtin_ctz(x)) + 1u;  // + 1: found
    }
    k_left = k_left >= cnt ? k_left - cnt : 0u;
  }
  const unsigned long long owner = __ballot(mine);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(row), __builtin_ctzll(owner))) - 1u;
}

// One block of THREADS threads per row, 128 bytes of logits in flight per
// thread: 1024 threads when each compute unit holds one row at a time; 256
// so several rows share a compute unit when there are many rows.  The draw,
// whose per-group work is heavy, keeps half as much in flight.
//
// With nseg > 1 (rows with neither top-k, top-p nor min-p), each row is
// split into nseg segments of seg_len tokens (a multiple of 256), one block
// each: a block finds its segment's greedy argmax or Gumbel-max and posts it
// to out[r] as one 64-bit atomic maximum of (order key of the value or the
// Gumbel key, inverted token index), so the largest wins and ties go to the
// lowest index.  out must hold 0 beforehand (clear_tokens) and is turned
// into token numbers afterwards (finish_tokens).
template <typename D, int BYTES, int THREADS, bool SPLITF = false, bool HEAVY = false>
__global__ __launch_bounds__(THREADS) void sample_rows(const typename D::Bits* __restrict__ logits, int64_t ls,
                                                              const uint32_t* __restrict__ mask, int64_t ms,
                                                              int32_t V, SampleArgs a, int64_t row_base,
                                                              int64_t* __restrict__ out, int32_t nseg,
                                                              int32_t seg_len, const SplitInfo* __restrict__ info,
                                                              const uint32_t* __restrict__ heavy) {
  constexpr int kWaves = THREADS / 64;
  __shared__ float s_best[kWaves];
  __shared__ int32_t s_besti[kWaves];
  __shared__ SelectState s_sel;
  __shared__ unsigned long long s_bin[256];  // last radix pass: best (key, token) per digit of the bucket
  // per-wave histograms in dynamic LDS (present only when a filter may run)
  extern __shared__ unsigned long long s_dyn[];
  auto hist_m = reinterpret_cast<unsigned long long(*)[256]>(s_dyn);
  auto hist_n = reinterpret_cast<uint32_t(*)[256]>(s_dyn + kWaves * 256);

  // HEAVY: heavy rows first, by the flags of row_classes (one block per
  // row); a separate instantiation, so that the other launches carry none
  // of its code
  int64_t r;
  bool known_dense = false;  // the row allows more than kSparseMax tokens (from row_classes)
  if constexpr (HEAVY) r = heavy_first_row(heavy, gridDim.x, blockIdx.x, &known_dense);
  else r = nseg > 1 ? blockIdx.x / nseg : blockIdx.x;
  const int32_t tok0 = nseg > 1 ? static_cast<int32_t>(blockIdx.x % nseg) * seg_len : 0;  // segment start
  const bool split = nseg > 1;
  const int t = static_cast<int>(threadIdx.x);
  const int wave = t >> 6;
  const typename D::Bits* row = logits + r * ls + tok0;
  const RowView<D> rv(row, mask ? mask + r * ms + tok0 / 32 : nullptr, split ? min(seg_len, V - tok0) : V);
  // one block's answer for row r: its own token (or -1), or a share of the
  // row's atomic maximum when the row is split
  const auto post = [&](uint32_t key, int32_t i) {
    const unsigned long long packed = (static_cast<unsigned long long>(key) << 32) |
                                      static_cast<uint32_t>(~static_cast<uint32_t>(tok0 + i));
    atomicMax(reinterpret_cast<unsigned long long*>(out) + r, packed);
  };

  const float temp = a.temperature ? a.temperature[r] : a.temperature_all;
  const int32_t top_k = a.top_k ? a.top_k[r] : a.top_k_all;
  const float top_p = a.top_p ? a.top_p[r] : a.top_p_all;
  const float min_p = a.min_p ? a.min_p[r] : a.min_p_all;

  // ---- pass 1: max and argmax (lowest index) over the candidates.  Greedy
  // rows need the argmax, top-p and min-p need the max logit (their masses
  // and cutoffs are relative to it); without those the pass is skipped: the
  // Gumbel keys need no max, and top-k needs no count of candidates (a k at
  // or above it comes out of the radix search as "keep all" (row_max).
  const bool first_pass = !(temp > 0.f) || top_p < 1.0f || min_p > 0.f;
  const float inv_t = 1.0f / temp;  // used only when temp > 0
  // An infinite temperature makes every z equal: each filter then keeps all
  // candidates (ties are kept), so top-k and top-p have nothing to do.
  const bool use_k = temp > 0.f && top_k > 0 && inv_t > 0.f;
  const bool use_p = temp > 0.f && top_p < 1.0f && inv_t > 0.f;
  float best = -__builtin_inff();
  bool have_best = false;  // the largest candidate is known
  bool have_cut = false;   // the top-k / top-p cut is known
  uint32_t cut = 0;        // keep tokens with order_key(x) >= cut
  uint32_t n_kept = 0;     // with the cut from the 16-bit search: candidates at or above it
  uint32_t cut16 = 0;      // and that cut as a 16-bit key (0: keep all)
  // A filtered row split over several blocks (SPLITF, nseg > 1): its
  // maximum and cut come from split_search, over the whole row.
  const bool from_split = SPLITF && temp > 0.f && (use_k || use_p || min_p > 0.f);
  if (from_split) {
    const SplitInfo si = info[r];
    if (si.best == -__builtin_inff()) {  // no candidate: the row's word keeps 0 (token -1)
      if (!split && t == 0) out[r] = -1;
      return;
    }
    best = si.best;
    have_best = true;
    if (use_k || use_p) {
      have_cut = true;
      cut16 = si.cut16;
      cut = cut16 ? order_key(D::value(static_cast<typename D::Bits>(bits_of_key16(cut16)))) : 0u;
      n_kept = si.kept;
    }
  }
  // A 16-bit row with a filter and at most 4 groups per thread is loaded once
  // into registers: the histogram pass and the draw both use these words.
  typename RowView<D>::Raw pre[4] = {};
  bool sparse = false;     // the cuts came from sparse_search, whose list the draw walks
  uint32_t sparse_nw = 0;  // that list's entries in this wave's region
  const bool preloaded = kFineSearch<D, THREADS> && (use_k || use_p) && !from_split && rv.V <= 4 * 8 * THREADS;
  if constexpr (kFineSearch<D, THREADS>) {
    if (preloaded) {
      const int32_t nfull = rv.V >> 3;
      if (rv.aligned) {
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[j] = rv.template load_raw<true>(j * THREADS + t, j * THREADS + t < nfull);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[j] = rv.template load_raw<false>(j * THREADS + t, j * THREADS + t < nfull);
      }
    }
    // a sparse row: the cuts from a list of its candidates, which the draw
    // then walks (sparse_search)
    if constexpr (THREADS == 512 || THREADS == 1024) {
      // (a row row_classes found dense would fail its count: skip it)
      if ((use_k || use_p) && !from_split && !preloaded && rv.has_mask && !known_dense) {
        sparse = sparse_search<D, THREADS>(rv, reinterpret_cast<uint32_t*>(s_dyn), inv_t, use_k, top_k, use_p, top_p,
                                           &best, &cut16, &sparse_nw);
        if (sparse) {
          have_cut = true;
          have_best = true;
          if (best == -__builtin_inff()) {  // no candidate
            if (t == 0) out[r] = -1;
            return;
          }
          cut = cut16 ? order_key(D::value(static_cast<typename D::Bits>(bits_of_key16(cut16)))) : 0u;
        }
      }
    }
    // 16-bit rows with a filter: one pass gives the maximum and both cuts
    if ((use_k || use_p) && !from_split && !sparse) {
      have_cut = fine_search<D, BYTES, THREADS>(rv, reinterpret_cast<uint32_t*>(s_dyn), inv_t, use_k, top_k, use_p,
                                                top_p, &best, &cut, &cut16, &n_kept, pre, preloaded);
      if (have_cut) {  // else the radix search below, after the first pass if the row needs the maximum
        have_best = true;
        if (best == -__builtin_inff()) {  // no candidate
          if (t == 0) out[r] = -1;
          return;
        }
      }
    }
  }
  // fp32 rows with top-k or top-p in 1024-thread blocks that need the
  // maximum (top-p, min-p): the coarse pass finds it too (coarse_hist32 in
  // edge mode)
  const bool fused_max = first_pass && sizeof(typename D::Bits) == 4 && THREADS == 1024 && (use_k || use_p) &&
                         !have_cut && !split && rv.V <= kEdgeMassMaxTokens;
  if (first_pass && !have_best && !fused_max) {
    int32_t besti;
    row_max<BYTES, THREADS>(rv, &best, &besti);
    // candidates are finite, so the max is -inf only when there is none
    const bool none = best == -__builtin_inff();
    if (none || !(temp > 0.f)) {  // no candidate, or greedy
      if (t == 0) {
        if (!split) out[r] = none ? -1 : besti;
        else if (!none) post(order_key(best), besti);
      }
      return;
    }
  }

  float zmax = best * inv_t;  // used only when the maximum is known (set again after a fused maximum)
  const bool use_min_p = min_p > 0.f;
  // min_p >= 1 keeps just the largest value and its ties (the cut never passes z_max)
  const float ln_min_p = use_min_p ? fminf(logf(min_p), 0.f) : 0.f;

  // Gumbel-max over the kept tokens: the token with the largest
  // z - ln(-ln u), u from the token's Philox word; sink(q, key) receives
  // each kept token's key.  The key is kept in base 2: since ln(-ln u) =
  // ln 2 (log2(-log2 u) + log2(ln 2)), z - ln(-ln u) is a positive multiple
  // of z log2(e) - log2(-log2 u) plus a constant, so both pick the same
  // token, and the base-2 form takes the two hardware logarithms and one
  // fma.  Clamped so an overflowed z (a tiny temperature) still draws a
  // token.
  const float inv_t_log2e = inv_t * 1.4426950408889634f;
  const auto gumbel_key = [&](float x, uint32_t word) {
    return fmaxf(fmaf(x, inv_t_log2e, -__log2f(-__log2f(unit_uniform(word)))), -__FLT_MAX__);
  };
  const auto gumbel_group = [&](int32_t i0, const float* x, uint32_t kept, auto&& sink) {
    uint32_t c0[4] = {static_cast<uint32_t>((tok0 + i0) >> 2), static_cast<uint32_t>(row_base + r), a.offset_lo,
                      a.offset_hi};
    uint32_t c1[4] = {static_cast<uint32_t>((tok0 + i0) >> 2) + 1u, static_cast<uint32_t>(row_base + r), a.offset_lo,
                      a.offset_hi};
    if (kept & 0x0Fu) philox4x32_10(c0, a.seed_lo, a.seed_hi);
    if (kept & 0xF0u) philox4x32_10(c1, a.seed_lo, a.seed_hi);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if ((kept >> q) & 1u) sink(q, gumbel_key(x[q], q < 4 ? c0[q] : c1[q - 4]));
  };
  const auto min_p_keep = [&](const float* x, uint32_t bits) {
    if (use_min_p) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (x[q] * inv_t - zmax < ln_min_p) bits &= ~(1u << q);
    }
    return bits;
  };

  float bk = -__builtin_inff();  // this thread's best Gumbel key so far, and its token
  int32_t bi = 0x7FFFFFFF;
  const auto offer = [&](float key, int32_t i) {
    if (key > bk || (key == bk && i < bi)) {
      bk = key;
      bi = i;
    }
  };
  // Gumbel-max over the kept tokens of one group, into (bk, bi), for a
  // thread that sees its tokens by increasing index (a token replaces the
  // best on a strictly larger key).  `dense` (the same in every lane of the
  // wave) computes every token's key and selects the kept ones without
  // branches; otherwise each token is a branch, which the wave skips when
  // none of its lanes keeps that token.
  const auto gumbel_best = [&](int32_t i0, const float* x, uint32_t kept, bool dense) {
    if (!dense) {
      gumbel_group(i0, x, kept, [&](int q, float key) {
        if (key > bk) {
          bk = key;
          bi = i0 + q;
        }
      });
      return;
    }
    uint32_t c0[4] = {static_cast<uint32_t>((tok0 + i0) >> 2), static_cast<uint32_t>(row_base + r), a.offset_lo,
                      a.offset_hi};
    uint32_t c1[4] = {static_cast<uint32_t>((tok0 + i0) >> 2) + 1u, static_cast<uint32_t>(row_base + r), a.offset_lo,
                      a.offset_hi};
    if (kept & 0x0Fu) philox4x32_10(c0, a.seed_lo, a.seed_hi);
    if (kept & 0xF0u) philox4x32_10(c1, a.seed_lo, a.seed_hi);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float key = gumbel_key(x[q], q < 4 ? c0[q] : c1[q - 4]);
      const bool take = ((kept >> q) & 1u) && key > bk;
      bk = take ? key : bk;
      bi = take ? i0 + q : bi;
    }
  };
  // whether at least half the wave's lanes keep a token of their group
  const auto dense_group = [](uint32_t kept) { return __popcll(__ballot(kept != 0u)) >= 32; };

  // Whether the last radix pass draws as it counts: fp32 only.  A 16-bit row
  // reaches the radix passes only when a key holds 65536 tokens or more (the
  // histogram search covers the rest), and a separate draw keeps the
  // kernel's register count down for the common path.
  constexpr bool kFuseDraw = sizeof(typename D::Bits) == 4;
  bool drawn = false;
  // fp32 rows with top-k or top-p in 1024-thread blocks: the coarse pass, then
  // a draw that lists the candidates of the cut's bucket (coarse_hist32)
  if constexpr (sizeof(typename D::Bits) == 4 && THREADS == 1024) {
    if ((use_k || use_p) && !have_cut) {
      unsigned long long* cm = reinterpret_cast<unsigned long long*>(s_dyn);
      uint32_t* cc = reinterpret_cast<uint32_t*>(cm + kCoarseBuckets);
      if (fused_max) {
        const uint32_t kmax = coarse_hist32<THREADS>(rv, cm, cc, use_k, use_p, inv_t, 0.f, true);
        if (kmax == 0u) {  // no candidate
          if (t == 0) out[r] = -1;
          return;
        }
        best = value_of_key(kmax);
        zmax = best * inv_t;
        // the bucket holding the maximum: its sum is rescaled by exp((e - xmax) / T)
        // >= 1, so its rounding error grows by that factor; past 2^14 (the
        // precision fixed_mass gives) the pass runs again relative to z_max
        const float e_top = value_of_key(kmax | ((1u << kCoarseShift) - 1u));
        if (use_p && (static_cast<double>(e_top) - static_cast<double>(best)) *
                             static_cast<double>(inv_t * 1.4426950408889634f) > 14.0) {
          __syncthreads();  // every thread has read the pass's results
          coarse_hist32<THREADS>(rv, cm, cc, use_k, use_p, inv_t, zmax, false);
        } else if (use_p) {
          edge_to_max_units(cm, inv_t, best);
        }
      } else {
        coarse_hist32<THREADS>(rv, cm, cc, use_k, use_p, inv_t, zmax, false);
      }
      uint32_t n_above = 0, need_k = 0;
      unsigned long long m_above = 0, need_p = 0;
      const uint32_t bk_ = use_k ? coarse_search<uint32_t>(
                                       cc, [&](uint32_t tot) { return static_cast<uint32_t>(top_k) <= tot ? static_cast<uint32_t>(top_k) : 0u; },
                                       &n_above, &need_k)
                                 : ~0u;
      const uint32_t bp_ = use_p ? coarse_search<unsigned long long>(
                                       cm,
                                       [&](unsigned long long tot) {
                                         // p <= 0 keeps just the largest value, as p = 0 does: any mass reaches it
                                         const double pz = fmax(static_cast<double>(top_p), 0.0) * static_cast<double>(tot);
                                         const unsigned long long target = static_cast<unsigned long long>(ceil(pz));
                                         return target ? target : 1ull;
                                       },
                                       &m_above, &need_p)
                                 : ~0u;
      // the higher of the two crossing buckets (~0u: that search keeps every candidate)
      const uint32_t bh = bk_ == ~0u ? bp_ : (bp_ == ~0u ? bk_ : max(bk_, bp_));
      have_cut = true;  // with bh == ~0u the cut is 0: every candidate is kept
      if (bh != ~0u) {
        // ---- draw: candidates above bucket bh by the walk, those inside listed
        uint32_t* lkey = reinterpret_cast<uint32_t*>(s_dyn);
        uint32_t* lidx = lkey + kCoarseListCap;
        __syncthreads();  // the searches' reads of cm and cc are done before the list overwrites them
        const int lane = lane_id();
        uint32_t* wkey = lkey + wave * kCoarseListPerWave;  // this wave's region
        uint32_t* widx = lidx + wave * kCoarseListPerWave;
        uint32_t nw = 0;  // entries this wave has listed (the same in every lane)
        const auto group = [&](int32_t i0, const float* x, uint32_t bits) {
          uint32_t above = 0, inside = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t key = order_key(x[q]);
            if (((bits >> q) & 1u) && finite_key(key)) {
              const uint32_t b = key >> kCoarseShift;
              above |= (b > bh ? 1u : 0u) << q;
              inside |= (b == bh ? 1u : 0u) << q;
            }
          }
          if (__ballot(inside != 0u)) {  // every lane of the wave takes this branch or none
            // this lane's entries go after those of the lanes below it
            const uint32_t cnt = static_cast<uint32_t>(__builtin_popcount(inside));
            const uint32_t incl = wave_prefix_sum(cnt);
            uint32_t pos = nw + incl - cnt;
            nw += lane63(incl);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              if ((inside >> q) & 1u) {
                if (pos < kCoarseListPerWave) {
                  wkey[pos] = order_key(x[q]);
                  widx[pos] = static_cast<uint32_t>(i0 + q);
                }
                ++pos;
              }
            }
          }
          // the branch-free form when the wave's groups keep many tokens (the
          // top-p sets of fp32 rows often do): 90.3 -> 86.5 us at B=256 top-p
          // 0.9; in the other draws it measured no better
          const uint32_t kept = min_p_keep(x, above);
          const bool dense = dense_group(kept);
          if (kept) gumbel_best(i0, x, kept, dense);  // each thread sees its tokens in order
        };
        walk_row_raw<BYTES / 2, THREADS>(rv, [&](int32_t g, const typename RowView<D>::Raw& raw, bool full) {
          float x[8];
          rv.values(raw, x);
          group(8 * g, x, rv.mask_bits(raw, g, full));
        });
        if (rv.V & 7) {  // the partial last group: exact candidate bits from the plain loads
          float x[8] = {};
          const uint32_t ok = t == 0 ? rv.load_tail(x) : 0u;
          group(rv.V & ~7, x, ok);
        }
        const bool over = __syncthreads_or(nw > kCoarseListPerWave);
        if (over) {
          // the bucket holds more candidates than the list: the radix search below
          // takes the row over, and its draw replaces this one
          have_cut = false;
          bk = -__builtin_inff();
          bi = 0x7FFFFFFF;
        } else {
          // ---- the exact cuts inside bucket bh: a radix select over the list's
          // low 20 key bits (digits at bits 19..12, 11..4, 3..0), counting for
          // top-k and summing masses for top-p, as the radix passes do over the row
          const bool rk = use_k && bk_ == bh, rp = use_p && bp_ == bh;
          unsigned long long* lh_m = reinterpret_cast<unsigned long long*>(lidx + kCoarseListCap);
          uint32_t* lh_n = reinterpret_cast<uint32_t*>(lh_m + 256);
          if (t == 0) s_sel = SelectState{bh << kCoarseShift, need_k - n_above, need_p - m_above, bh << kCoarseShift};
          uint32_t pmask = ~0u << kCoarseShift;
          for (int shift = 12; shift >= 0; shift = shift == 12 ? 4 : (shift == 4 ? 0 : -1)) {
            for (int b = t; b < 256; b += THREADS) {
              lh_n[b] = 0u;
              lh_m[b] = 0ull;
            }
            __syncthreads();
            const uint32_t pk = s_sel.prefix_k, pp = s_sel.prefix_p;
            for (uint32_t i = static_cast<uint32_t>(lane); i < nw; i += 64u) {  // this wave's entries
              const uint32_t key = wkey[i];
              const uint32_t d = (key >> shift) & 255u;
              if (rk && (key & pmask) == pk) atomicAdd(&lh_n[d], 1u);
              if (rp && (key & pmask) == pp) {
                const uint32_t m = fixed_mass(value_of_key(key), inv_t, zmax);
                if (m) atomicAdd(&lh_m[d], static_cast<unsigned long long>(m));
              }
            }
            __syncthreads();
            if (rk && wave == 0) {
              const WaveSuffix<uint32_t> ws(lh_n);
              int d;
              uint32_t ab;
              ws.pick(s_sel.need_k, &d, &ab);
              if (lane == 0) {
                s_sel.prefix_k |= static_cast<uint32_t>(d) << shift;
                s_sel.need_k -= ab;
              }
            }
            if (rp && wave == 1) {
              const WaveSuffix<unsigned long long> ws(lh_m);
              int d;
              unsigned long long ab;
              ws.pick(s_sel.need_p, &d, &ab);
              if (lane == 0) {
                s_sel.prefix_p |= static_cast<uint32_t>(d) << shift;
                s_sel.need_p -= ab;
              }
            }
            __syncthreads();
            pmask |= 255u << shift;
          }
          cut = max(rk ? s_sel.prefix_k : 0u, rp ? s_sel.prefix_p : 0u);
          // the listed candidates at or above the cut join the draw (min-p aside)
          for (uint32_t i = static_cast<uint32_t>(lane); i < nw; i += 64u) {  // this wave's entries
            const uint32_t key = wkey[i];
            const float x = value_of_key(key);
            if (key >= cut && !(use_min_p && x * inv_t - zmax < ln_min_p)) {
              const int32_t idx = static_cast<int32_t>(widx[i]);
              uint32_t c4[4] = {static_cast<uint32_t>((tok0 + idx) >> 2), static_cast<uint32_t>(row_base + r),
                                a.offset_lo, a.offset_hi};
              philox4x32_10(c4, a.seed_lo, a.seed_hi);
              const int32_t w4 = (tok0 + idx) & 3;
              const uint32_t word = w4 == 0 ? c4[0] : w4 == 1 ? c4[1] : w4 == 2 ? c4[2] : c4[3];
              offer(gumbel_key(x, word), idx);
            }
          }
          drawn = true;
        }
      }
    }
  }
  if ((use_k || use_p) && !have_cut) {
    // ---- top-k and top-p cuts: radix passes over 8-bit digits of the key,
    // high to low, both searches in the same passes.  The first mass
    // histogram covers every candidate, so its total is the softmax mass Z.
    //
    // For fp16 and fp32 the last pass also draws.  Before it, every token
    // whose key is above the bucket of the higher of the two prefixes is
    // kept whatever the last digit turns out to be, and every token below
    // that bucket is cut; the final cut lies inside the bucket.  So that
    // pass computes the Gumbel key of each token above or in the bucket: a
    // token above goes to the thread's running best, a token in the bucket
    // to a per-digit best in LDS; once the digit is known, the bins at or
    // above it join the draw.
    if (t == 0) s_sel = SelectState{0u, static_cast<uint32_t>(top_k), 0ull, 0u};
    // Digits below kLastShift lie in the type's always-zero low bits: every
    // token of a prefix shares them (all 0 under a positive prefix, all 1
    // under a negative one, the key complementing negatives), so they are
    // filled in after the passes instead of counted.
    constexpr int kLastShift = (D::kZeroLowBits / 8) * 8;
    // The draw may ride on the last pass only when that pass's bucket is
    // narrow (a 16-bit prefix or finer).  For bf16 the last pass is the
    // second digit and its bucket a whole binade, often thousands of tokens,
    // which would all pay for the generator.
    static_assert(!kFuseDraw || kLastShift < 16, "a fused draw needs a narrow last bucket");
    // one radix pass; `last` (a compile-time flag) also draws, with half as
    // many bytes in flight to leave registers for the generator
    const auto radix_pass = [&](int shift, uint32_t pmask, auto last_tag) {
      constexpr bool last = decltype(last_tag)::value;
      for (int b = t; b < kWaves * 256; b += THREADS) {
        (&hist_n[0][0])[b] = 0u;
        (&hist_m[0][0])[b] = 0ull;
      }
      if constexpr (last)
        for (int b = t; b < 256; b += THREADS) s_bin[b] = 0ull;
      __syncthreads();
      const uint32_t pk = s_sel.prefix_k, pp = s_sel.prefix_p;
      const uint32_t phi = max(use_k ? pk : 0u, use_p ? pp : 0u);
      // One group: `bits` are its mask bits; a token is a candidate when its
      // bit is set and its key is that of a finite value.
      const auto group = [&](int32_t i0, const float* x, uint32_t bits) {
        uint32_t above = 0, inside = 0;
        uint32_t digit[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t key = order_key(x[q]);
          const uint32_t d = (key >> shift) & 255u;
          digit[q] = d;
          if (((bits >> q) & 1u) && finite_key(key)) {
            if (use_k && (key & pmask) == pk) atomicAdd(&hist_n[wave][d], 1u);
            if (use_p && (key & pmask) == pp) {
              const uint32_t m = fixed_mass(x[q], inv_t, zmax);  // one that truncates to 0 adds nothing
              if (m) atomicAdd(&hist_m[wave][d], static_cast<unsigned long long>(m));
            }
            if constexpr (last) {
              if ((key & pmask) > phi) above |= 1u << q;
              else if ((key & pmask) == phi) inside |= 1u << q;
            }
          }
        }
        if constexpr (!last) return;
        const uint32_t kept = min_p_keep(x, above | inside);
        if (!kept) return;
        gumbel_group(i0, x, kept, [&](int q, float key) {
          if ((above >> q) & 1u) {
            offer(key, i0 + q);
          } else {
            // larger key first, then the lower token index
            const unsigned long long packed = (static_cast<unsigned long long>(order_key(key)) << 32) |
                                              static_cast<uint32_t>(~static_cast<uint32_t>(i0 + q));
            atomicMax(&s_bin[digit[q]], packed);
          }
        });
      };
      walk_row_raw<last ? BYTES / 2 : BYTES, THREADS>(
          rv, [&](int32_t g, const typename RowView<D>::Raw& raw, bool full) {
            float x[8];
            rv.values(raw, x);
            group(8 * g, x, rv.mask_bits(raw, g, full));
          });
      if (rv.V & 7) {  // the partial last group: exact candidate bits from the plain loads
        float x[8] = {};
        const uint32_t ok = t == 0 ? rv.load_tail(x) : 0u;
        group(rv.V & ~7, x, ok);
      }
      __syncthreads();
      // fold the per-wave histograms into row 0
      for (int b = t; b < 256; b += THREADS) {
        uint32_t n = 0;
        unsigned long long m = 0;
        for (int w = 0; w < kWaves; ++w) {
          n += hist_n[w][b];
          m += hist_m[w][b];
        }
        hist_n[0][b] = n;
        hist_m[0][b] = m;
      }
      __syncthreads();
      // both searches pick their digit at once: top-k on wave 0, top-p on
      // wave 1 (different fields of s_sel)
      if (use_k && wave == 0) {
        const WaveSuffix<uint32_t> ws(&hist_n[0][0]);
        int d;
        uint32_t ab;
        ws.pick(s_sel.need_k, &d, &ab);
        if (lane_id() == 0) {
          s_sel.prefix_k |= static_cast<uint32_t>(d) << shift;
          s_sel.need_k -= ab;
        }
      }
      if (use_p && wave == 1) {
        const WaveSuffix<unsigned long long> ws(&hist_m[0][0]);
        unsigned long long need = s_sel.need_p;
        if (shift == 24) {  // every candidate is in this histogram: its total is Z
          // p <= 0 keeps just the largest value, as p = 0 does: any mass reaches it
          const double pz = fmax(static_cast<double>(top_p), 0.0) * static_cast<double>(ws.total());
          const unsigned long long target = static_cast<unsigned long long>(ceil(pz));
          need = target ? target : 1ull;
        }
        int d;
        unsigned long long ab;
        ws.pick(need, &d, &ab);
        if (lane_id() == 0) {
          s_sel.prefix_p |= static_cast<uint32_t>(d) << shift;
          s_sel.need_p = need - ab;
        }
      }
      __syncthreads();
    };
    uint32_t pmask = 0;
    for (int shift = 24; shift > kLastShift; shift -= 8) {
      radix_pass(shift, pmask, std::false_type{});
      pmask |= 255u << shift;
    }
    radix_pass(kLastShift, pmask, std::integral_constant<bool, kFuseDraw>{});
    constexpr uint32_t kLow = (1u << kLastShift) - 1u;
    const auto complete = [&](uint32_t prefix) { return prefix | ((prefix & 0x80000000u) ? 0u : kLow); };
    if (use_k) cut = max(cut, complete(s_sel.prefix_k));
    if (use_p) cut = max(cut, complete(s_sel.prefix_p));
    if constexpr (kFuseDraw) {
      // the bucket's tokens at or above the cut's last digit are kept
      const uint32_t dcut = (cut >> kLastShift) & 255u;
      for (int b = t; b < 256; b += THREADS) {
        const unsigned long long packed = s_bin[b];
        if (static_cast<uint32_t>(b) >= dcut && packed) {
          const uint32_t k = static_cast<uint32_t>(packed >> 32);
          offer(__uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k),
                static_cast<int32_t>(~static_cast<uint32_t>(packed)));
        }
      }
    }
  }
  // ---- draw after the 16-bit search
  constexpr uint32_t kFineWordsHere = static_cast<uint32_t>(fine_words(THREADS));
  constexpr uint32_t kListPerWave = kFineWordsHere / (THREADS / 64);
  if constexpr (kFineSearch<D, THREADS>) {
    if (have_cut) {
      // The kept test on 16-bit keys of the raw words, two per operation:
      // a candidate (mask bit set, finite value) at or above the cut.  The
      // keys of -0 and +0 differ by one; a cut at +0 keeps -0 too.
      const uint32_t lo16 = cut16 == 0u ? D::kKey16Lo : (cut16 == 0x8000u ? 0x7FFFu : cut16);
      const uint32_t span16 = D::kKey16Hi - lo16;
      const auto keep_of = [&](const typename RowView<D>::Raw& raw, uint32_t bits, float x[8]) {
        uint32_t keep = 0;
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          const uint32_t k2 = order_key16x2(raw.v[p2]);
          keep |= ((k2 & 0xFFFFu) - lo16 <= span16 ? 1u : 0u) << (2 * p2);
          keep |= ((k2 >> 16) - lo16 <= span16 ? 1u : 0u) << (2 * p2 + 1);
        }
        keep &= bits;
        if (keep) {
          rv.values(raw, x);
          keep = min_p_keep(x, keep);
        }
        return keep;
      };
      // every group of the row, the partial last one included (its words
      // loaded by thread 0 alone), through f(i0, raw, mask bits)
      if (sparse) {
        // ---- draw over the listed candidates at or above the cut (min-p aside)
        const SparseList<THREADS> sl(reinterpret_cast<const uint32_t*>(s_dyn));
        const uint32_t region = static_cast<uint32_t>(wave) * SparseList<THREADS>::kPerWave;
        for (uint32_t i = static_cast<uint32_t>(lane_id()); i < sparse_nw; i += 64u) {
          const uint32_t k16 = sl.key[region + i];
          if (k16 - lo16 > span16) continue;
          const float x = D::value(static_cast<typename D::Bits>(bits_of_key16(k16)));
          if (use_min_p && x * inv_t - zmax < ln_min_p) continue;
          const int32_t idx = static_cast<int32_t>(sl.idx[region + i]);
          uint32_t c4[4] = {static_cast<uint32_t>((tok0 + idx) >> 2), static_cast<uint32_t>(row_base + r), a.offset_lo,
                            a.offset_hi};
          philox4x32_10(c4, a.seed_lo, a.seed_hi);
          const int32_t w4 = (tok0 + idx) & 3;
          const uint32_t word = w4 == 0 ? c4[0] : w4 == 1 ? c4[1] : w4 == 2 ? c4[2] : c4[3];
          offer(gumbel_key(x, word), idx);
        }
        drawn = true;
      }
      const auto walk16 = [&](auto&& f) {
        if (preloaded) {
          const int32_t nfull = rv.V >> 3;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int32_t g = j * THREADS + t;
            f(8 * g, pre[j], rv.mask_bits(pre[j], g, g < nfull));
          }
        } else {
          walk_row_raw<BYTES / 2, THREADS>(rv, [&](int32_t g, const typename RowView<D>::Raw& raw, bool full) {
            f(8 * g, raw, rv.mask_bits(raw, g, full));
          });
        }
        if (rv.V & 7) {
          typename RowView<D>::Raw raw{};
          uint32_t bits = 0;
          const int32_t i0 = rv.V & ~7;
          if (t == 0) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const int32_t i = i0 + q;
              if (i < rv.V) {
                raw.v[q >> 1] |= static_cast<uint32_t>(row[i]) << (16 * (q & 1));
                bits |= (rv.has_mask ? (load_word(rv.rm, (i >> 5) * 4) >> (i & 31)) & 1u : 1u) << q;
              }
            }
          }
          f(i0, raw, bits);
        }
      };
      if (!drawn && (n_kept >= 256u || rv.V <= 64 * THREADS) && n_kept >= 1u && n_kept <= static_cast<uint32_t>(rv.V) / 6u &&
          n_kept <= kFineWordsHere - 4096u) {
        // Many kept tokens (the search counted them): list them first (LDS, where
        // the histogram was, one region per wave), then run the generator on the
        // list alone, every lane busy; a walk would run it for every group in
        // which any lane of the wave keeps a token.  With fewer than 256 on a long
        // row, most of a wave's groups keep none, and the walk skips those; on a
        // row of at most 8 groups per thread most of them keep one somewhere in
        // the wave, and the list still pays.  The list pays one generator call per
        // kept token, the walk one per 4 tokens of every group it runs it for, so
        // the list is taken for at most V / 6 kept tokens; and at most 4096 fewer
        // than the histogram's words (28672 or 12288), which leaves each wave's
        // region room for its share plus 256 (or 512).
        uint32_t* list = reinterpret_cast<uint32_t*>(s_dyn) + wave * kListPerWave;
        uint32_t nw = 0;  // the same in every lane of the wave
        // per group: one prefix sum of the lanes' kept counts places each
        // lane's entries, then each lane writes its own kept tokens, so a
        // group costs its wave one step per kept token of its busiest lane
        // (the draw below does not depend on the list's order)
        walk16([&](int32_t i0, const typename RowView<D>::Raw& raw, uint32_t bits) {
          float x[8];
          const uint32_t keep = keep_of(raw, bits, x);
          const uint32_t cnt = static_cast<uint32_t>(__builtin_popcount(keep));
          if (!__ballot(cnt != 0u)) return;
          const uint32_t incl = wave_prefix_sum(cnt);
          uint32_t pos = nw + incl - cnt;
          nw += lane63(incl);
          for (uint32_t c = keep; c != 0u; c &= c - 1u) {
            if (pos < kListPerWave) list[pos] = static_cast<uint32_t>(i0 + __builtin_ctz(c));
            ++pos;
          }
        });
        // a wave whose region filled up sends the row through the walk below
        drawn = !__syncthreads_or(nw > kListPerWave);
        if (drawn) {
          // four entries per lane at a time, their logits loaded together
          for (uint32_t e0 = static_cast<uint32_t>(lane_id()); e0 < nw; e0 += 4u * 64u) {
            int32_t idx[4];
            uint32_t h[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint32_t e = e0 + 64u * u;
              idx[u] = e < nw ? static_cast<int32_t>(list[e]) : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
              h[u] = __builtin_amdgcn_raw_buffer_load_b16(rv.rl, idx[u] >= 0 ? idx[u] * 2 : kSkip, 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              if (idx[u] < 0) continue;
              const int32_t i = idx[u];
              uint32_t c4[4] = {static_cast<uint32_t>((tok0 + i) >> 2), static_cast<uint32_t>(row_base + r), a.offset_lo,
                                a.offset_hi};
              philox4x32_10(c4, a.seed_lo, a.seed_hi);
              const int32_t w4 = (tok0 + i) & 3;
              const uint32_t word = w4 == 0 ? c4[0] : w4 == 1 ? c4[1] : w4 == 2 ? c4[2] : c4[3];
              offer(gumbel_key(D::value(static_cast<typename D::Bits>(h[u])), word), i);
            }
          }
        }
      }
      if (!drawn) {
        // ---- draw: Gumbel-max over the tokens at or above the cut, by a walk
        walk16([&](int32_t i0, const typename RowView<D>::Raw& raw, uint32_t bits) {
          float x[8];
          const uint32_t keep = keep_of(raw, bits, x);
          if (!keep) return;
          gumbel_group(i0, x, keep, [&](int q, float key) { offer(key, i0 + q); });
        });
        drawn = true;
      }
    }
  }
  if ((use_k || use_p) && !drawn) {
    if (have_cut || !kFuseDraw) {
      // ---- draw: Gumbel-max over the tokens at or above the cut
      walk_row<BYTES / 2, THREADS>(rv, [&](int32_t i0, const float* x, uint32_t ok) {
        uint32_t at_or_above = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (((ok >> q) & 1u) && order_key(x[q]) >= cut) at_or_above |= 1u << q;
        const uint32_t kept = min_p_keep(x, at_or_above);
        if (!kept) return;
        gumbel_group(i0, x, kept, [&](int q, float key) {
          if (key > bk) {  // strictly greater: each thread sees its tokens in order
            bk = key;
            bi = i0 + q;
          }
        });
      });
    }
  } else if (!drawn) {
    // ---- draw: Gumbel-max over every candidate (min-p aside)
    walk_row<BYTES / 2, THREADS>(rv, [&](int32_t i0, const float* x, uint32_t ok) {
      const uint32_t kept = min_p_keep(x, ok);
      if (!kept) return;
      gumbel_group(i0, x, kept, [&](int q, float key) {
        if (key > bk) {  // strictly greater: each thread sees its tokens in order
          bk = key;
          bi = i0 + q;
        }
      });
    });
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
    for (int w = 1; w < kWaves; ++w)
      if (s_best[w] > bk || (s_best[w] == bk && s_besti[w] < bi)) {
        bk = s_best[w];
        bi = s_besti[w];
      }
    // every kept token has a key above -inf, and a row with a candidate
    // keeps at least its largest logit: bi is unset only without candidates
    if (!split) out[r] = bi == 0x7FFFFFFF ? -1 : bi;
    else if (bi != 0x7FFFFFFF) post(order_key(bk), bi);
  }
}

// Before a split launch: every row's answer word at 0, below any posted
// (key, index) pair (keys of finite values and of clamped Gumbel keys are at
// least 0x00800000).  A kernel rather than a memset, so graphs replay it.
__global__ void clear_tokens(int64_t* __restrict__ out, int64_t rows) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r < rows) out[r] = 0;
}

// After a split launch: the token number from each row's maximum, -1 where
// no segment posted one.
__global__ void finish_tokens(int64_t* __restrict__ out, int64_t rows) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r < rows) {
    const unsigned long long packed = static_cast<unsigned long long>(out[r]);
    out[r] = packed ? static_cast<int64_t>(~static_cast<uint32_t>(packed)) : -1;
  }
}

}  // namespace mi
