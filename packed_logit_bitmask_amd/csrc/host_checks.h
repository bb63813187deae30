// Host-side helpers shared by the library's entry points (internal): the
// thread-local error message, size limits, the vocab-size rule, the fill
// conversion, buffer extents and overlap, and the argument checks common to
// every device entry point.  Everything here runs on the host before the
// first HIP call of an entry point.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mi_bitmask.h"

#define MI_API extern "C" __attribute__((visibility("default")))

namespace mi_abi {

inline thread_local char g_message[512] = "";

inline mi_status_t fail(mi_status_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_message, sizeof g_message, fmt, ap);
  va_end(ap);
  return status;
}

// Limits keep every index computation inside int32 (within a row) and
// int64 (across rows), and the grid inside what one launch can carry.
constexpr int64_t kMaxCols = int64_t(1) << 30;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxPitch = int64_t(1) << 40;
constexpr int64_t kMaxBytes = int64_t(1) << 56;

inline int elem_bytes(mi_dtype_t d) { return d == MI_DTYPE_F32 ? 4 : 2; }

inline bool valid_dtype(int d) { return d == MI_DTYPE_F32 || d == MI_DTYPE_F16 || d == MI_DTYPE_BF16; }

// Round a double once, to nearest-even, into a binary format with `ebits`
// exponent and `mbits` fraction bits; returns the pattern in the low bits.
// Works on the double's fields: drop the low bits of the 53-bit significand
// (more of them below the target's normal range), round on the dropped
// part, then re-encode, carrying into the exponent and overflowing to inf.
inline uint32_t round_to_format(double x, int ebits, int mbits) {
  uint64_t b;
  std::memcpy(&b, &x, sizeof b);
  const int width = 1 + ebits + mbits;
  const uint32_t sbit = static_cast<uint32_t>(b >> 63) << (width - 1);
  const uint32_t exp_all = (1u << ebits) - 1u;
  const int dexp = static_cast<int>((b >> 52) & 0x7FF);
  const uint64_t frac = b & ((uint64_t(1) << 52) - 1);
  if (dexp == 0x7FF)  // inf, or NaN -> quiet NaN without payload
    return frac ? (sbit | (exp_all << mbits) | (1u << (mbits - 1))) : (sbit | (exp_all << mbits));
  if (dexp == 0) return sbit;  // zero or a double subnormal: far below every target's subnormals
  const int bias = (1 << (ebits - 1)) - 1;
  const int emin = 1 - bias;
  int e = dexp - 1023;                                   // x = sig * 2^(e - 52)
  const uint64_t sig = frac | (uint64_t(1) << 52);
  const int drop = 52 - mbits + (e < emin ? emin - e : 0);
  if (drop > 63) return sbit;
  uint64_t kept = sig >> drop;
  const uint64_t rem = sig & ((uint64_t(1) << drop) - 1);
  const uint64_t half = uint64_t(1) << (drop - 1);
  if (rem > half || (rem == half && (kept & 1u))) ++kept;
  if (e < emin)  // subnormal; a carry to 2^mbits is the smallest normal, same integer
    return sbit | static_cast<uint32_t>(kept);
  if (kept == (uint64_t(1) << (mbits + 1))) {
    kept >>= 1;
    ++e;
  }
  const int ef = e + bias;
  if (ef >= static_cast<int>(exp_all)) return sbit | (exp_all << mbits);
  return sbit | (static_cast<uint32_t>(ef) << mbits) | static_cast<uint32_t>(kept - (uint64_t(1) << mbits));
}

inline uint32_t fill_pattern(double v, mi_dtype_t d) {
  switch (d) {
    case MI_DTYPE_F32: return round_to_format(v, 8, 23);
    case MI_DTYPE_F16: return round_to_format(v, 5, 10);
    default: return round_to_format(v, 8, 7);
  }
}

struct ByteRange {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

inline bool extent(const void* p, int64_t rows, int64_t width, int64_t pitch, int64_t esize, ByteRange* out) {
  *out = ByteRange{};
  if (rows <= 0 || width <= 0) return true;
  int64_t n, bytes;
  if (__builtin_mul_overflow(rows - 1, pitch, &n) || __builtin_add_overflow(n, width, &n) ||
      __builtin_mul_overflow(n, esize, &bytes) || bytes > kMaxBytes)
    return false;
  out->lo = reinterpret_cast<uintptr_t>(p);
  out->hi = out->lo + static_cast<uintptr_t>(bytes);
  return out->hi > out->lo;
}

inline bool overlaps(const ByteRange& a, const ByteRange& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

inline mi_status_t resolve_vocab(int64_t cols, int64_t mask_cols, int64_t vocab_size, int64_t* V) {
  if (cols < 0 || mask_cols < 0) return fail(MI_ERR_BAD_SHAPE, "negative width (cols %lld, mask_cols %lld)",
                                             (long long)cols, (long long)mask_cols);
  if (cols > kMaxCols || mask_cols > kMaxCols)
    return fail(MI_ERR_BAD_SHAPE, "width above the limit 2^30 (cols %lld, mask_cols %lld)",
                (long long)cols, (long long)mask_cols);
  const int64_t limit = std::min(cols, 32 * mask_cols);
  if (vocab_size == -1) {
    *V = limit;
    return MI_OK;
  }
  if (vocab_size < 0 || vocab_size > limit)
    return fail(MI_ERR_BAD_VOCAB, "vocab_size %lld outside [0, min(cols %lld, 32 * mask_cols %lld) = %lld]",
                (long long)vocab_size, (long long)cols, (long long)mask_cols, (long long)limit);
  *V = vocab_size;
  return MI_OK;
}

// Everything the kernels need after validation.
struct Plan {
  int64_t V = 0, W = 0;       // vocab and words per row actually used
  int64_t R = 0;              // processed row slots
  int64_t row_limit = 0;      // valid row numbers for an index list
  int esize = 0;
  uint32_t fill = 0;
  ByteRange logits, mask, indices;
};

inline mi_status_t check_common(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t ls,
                         const int32_t* mask, int64_t mask_rows, int64_t mask_cols, int64_t ms,
                         int64_t vocab_size, const int32_t* indices, int64_t num_indices,
                         double fill_value, Plan* p) {
  // An empty tensor may carry a NULL data pointer; a non-empty one may not.
  if (!logits && rows > 0 && cols > 0) return fail(MI_ERR_NULL_POINTER, "logits is NULL");
  if (!mask && mask_rows > 0 && mask_cols > 0) return fail(MI_ERR_NULL_POINTER, "mask is NULL");
  if (!indices && num_indices > 0) return fail(MI_ERR_NULL_POINTER, "indices is NULL but num_indices is %lld",
                                              (long long)num_indices);
  if (!valid_dtype(static_cast<int>(dtype))) return fail(MI_ERR_BAD_DTYPE, "unknown dtype %d", (int)dtype);
  if (rows < 0 || cols < 0 || mask_rows < 0 || mask_cols < 0)
    return fail(MI_ERR_BAD_SHAPE, "negative size (rows %lld, cols %lld, mask_rows %lld, mask_cols %lld)",
                (long long)rows, (long long)cols, (long long)mask_rows, (long long)mask_cols);
  if (rows > kMaxRows || mask_rows > kMaxRows)
    return fail(MI_ERR_BAD_SHAPE, "row count above the limit 2^31 - 1");
  if (ls < cols || ls > kMaxPitch)
    return fail(MI_ERR_BAD_SHAPE, "logits_row_stride %lld must be in [cols %lld, 2^40]", (long long)ls,
                (long long)cols);
  if (ms < mask_cols || ms > kMaxPitch)
    return fail(MI_ERR_BAD_SHAPE, "mask_row_stride %lld must be in [mask_cols %lld, 2^40]", (long long)ms,
                (long long)mask_cols);
  mi_status_t st = resolve_vocab(cols, mask_cols, vocab_size, &p->V);
  if (st != MI_OK) return st;
  if (num_indices < 0 || num_indices > kMaxRows)
    return fail(MI_ERR_BAD_INDICES, "num_indices %lld outside [0, 2^31 - 1]", (long long)num_indices);
  if (indices) {
    p->R = num_indices;
    p->row_limit = std::min(rows, mask_rows);
  } else {
    if (mask_rows < rows)
      return fail(MI_ERR_BAD_SHAPE, "mask has %lld rows for %lld logits rows (no index list)",
                  (long long)mask_rows, (long long)rows);
    p->R = rows;
    p->row_limit = rows;
  }
  p->esize = elem_bytes(dtype);
  if (reinterpret_cast<uintptr_t>(logits) % p->esize)
    return fail(MI_ERR_MISALIGNED, "logits not aligned to its %d-byte elements", p->esize);
  if (reinterpret_cast<uintptr_t>(mask) % 4) return fail(MI_ERR_MISALIGNED, "mask not 4-byte aligned");
  if (indices && reinterpret_cast<uintptr_t>(indices) % 4)
    return fail(MI_ERR_MISALIGNED, "indices not 4-byte aligned");
  if (!extent(logits, rows, cols, ls, p->esize, &p->logits) ||
      !extent(mask, mask_rows, mask_cols, ms, 4, &p->mask) ||
      !extent(indices, indices ? 1 : 0, num_indices, num_indices, 4, &p->indices))
    return fail(MI_ERR_BAD_SHAPE, "buffer extent overflows");
  p->W = (p->V + 31) / 32;
  p->fill = fill_pattern(fill_value, dtype);
  return MI_OK;
}

inline mi_status_t after_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MI_OK;
}

}  // namespace mi_abi
