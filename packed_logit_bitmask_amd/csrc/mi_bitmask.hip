// Host side of the packed-bitmask apply: argument checks, vocab-size rule,
// fill conversion, variant choice and kernel launches.  The C ABI is
// declared (and documented) in include/mi_bitmask.h.
//
// Nothing here allocates, synchronises or touches device memory; every
// check runs before the first HIP call, so a rejected call enqueues nothing.

#include "mi_bitmask.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "apply_kernels.h"
#include "host_apply.h"
#include "sample_kernel.h"

#define MI_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_message[512] = "";

mi_status_t fail(mi_status_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_message, sizeof g_message, fmt, ap);
  va_end(ap);
  return status;
}

// Limits keep every index computation inside int32 (within a row) and
// int64 (across rows), and the grid inside what one launch can carry.
constexpr int64_t kMaxCols = int64_t(1) << 30;
constexpr int64_t kMaxSampleVocab = int64_t(1) << 28;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxPitch = int64_t(1) << 40;
constexpr int64_t kMaxBytes = int64_t(1) << 56;
constexpr int64_t kMaxBlocksPerLaunch = (int64_t(1) << 24) - 1;  // blocks * 256 < 2^32

// Shape of the 16-byte-vector kernels: vectors per lane (unroll) and the
// store cache policy.  Picked from measurements on MI355X, cold from HBM,
// in place:
//  - below 48 MB of writes, two vectors per lane with device-scope
//    write-through stores (the output streams out during the kernel instead
//    of in one end-of-kernel L2 writeback);
//  - from 48 MB to 1 GB, two vectors per lane with write-through
//    non-temporal stores: 3-5 % ahead of one vector per lane up to 128 MB
//    and 14-25 % ahead on rows of mixed kinds (all-ones, sparse, empty), at
//    most 4 % behind one vector per lane on 256-512 MB of uniform density;
//  - from 1 GB, four vectors per lane, non-temporal: 1-4 % ahead on the
//    large mixed-kind workloads.  One vector per lane is never used: it
//    launches 4x the blocks, which cost 36-40 % on rows that need little
//    work.
// Out of place, two vectors per lane with write-through non-temporal stores
// was best at every size measured.
struct VecShape {
  int unroll;
  int policy;
};

constexpr int64_t kSmallWriteBytes = int64_t(48) << 20;
constexpr int64_t kLargeWriteBytes = int64_t(1) << 30;

VecShape inplace_shape(int64_t write_bytes) {
  if (write_bytes < kSmallWriteBytes) return {2, mi::kStoreDevice};
  if (write_bytes < kLargeWriteBytes) return {2, mi::kStoreDeviceStream};
  return {4, mi::kStoreDeviceStream};
}

constexpr VecShape kOutShape{2, mi::kStoreDeviceStream};

int elem_bytes(mi_dtype_t d) { return d == MI_DTYPE_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == MI_DTYPE_F32 || d == MI_DTYPE_F16 || d == MI_DTYPE_BF16; }

// Round a double once, to nearest-even, into a binary format with `ebits`
// exponent and `mbits` fraction bits; returns the pattern in the low bits.
// Works on the double's fields: drop the low bits of the 53-bit significand
// (more of them below the target's normal range), round on the dropped
// part, then re-encode, carrying into the exponent and overflowing to inf.
uint32_t round_to_format(double x, int ebits, int mbits) {
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

uint32_t fill_pattern(double v, mi_dtype_t d) {
  switch (d) {
    case MI_DTYPE_F32: return round_to_format(v, 8, 23);
    case MI_DTYPE_F16: return round_to_format(v, 5, 10);
    default: return round_to_format(v, 8, 7);
  }
}

struct ByteRange {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

bool extent(const void* p, int64_t rows, int64_t width, int64_t pitch, int64_t esize, ByteRange* out) {
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

bool overlaps(const ByteRange& a, const ByteRange& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

mi_status_t resolve_vocab(int64_t cols, int64_t mask_cols, int64_t vocab_size, int64_t* V) {
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

mi_status_t check_common(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t ls,
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

mi_status_t after_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MI_OK;
}

// Launch over `slots` row slots, `chunks` blocks per slot, splitting into
// several launches when one grid would be too large.  With `extra_per_slot`
// set, each launch also carries one extra block per slot (the per-row report
// blocks, placed first); launch() gets (first slot, blocks, chunks, extra).
template <typename Launch>
mi_status_t launch_slots(int64_t slots, int64_t chunks, Launch&& launch, bool extra_per_slot = false) {
  const int64_t per_slot = chunks + (extra_per_slot ? 1 : 0);
  const int64_t per = std::max<int64_t>(1, kMaxBlocksPerLaunch / per_slot);
  for (int64_t s0 = 0; s0 < slots; s0 += per) {
    const int64_t n = std::min(per, slots - s0);
    launch(s0, static_cast<uint32_t>(n * per_slot), static_cast<uint32_t>(chunks),
           static_cast<uint32_t>(extra_per_slot ? n : 0));
  }
  return MI_OK;
}

template <typename T>
mi_status_t run_inplace(void* logits_v, int64_t ls, const int32_t* mask_i, int64_t ms, const int32_t* indices,
                        const Plan& p, mi_variant_t variant, hipStream_t stream, const int8_t* gate = nullptr,
                        uint8_t* any_out = nullptr) {
  T* logits = static_cast<T*>(logits_v);
  const uint32_t* mask = reinterpret_cast<const uint32_t*>(mask_i);
  const mi::RowMap map{indices, p.row_limit, gate};
  const T fill = static_cast<T>(p.fill);
  const int32_t V = static_cast<int32_t>(p.V), W = static_cast<int32_t>(p.W);
  (void)hipGetLastError();  // report only what this call's launches raise
  switch (variant) {
    case MI_VARIANT_SCALAR: {
      const int64_t chunks = (p.V + mi::kBlock * 8 - 1) / (mi::kBlock * 8);
      launch_slots(p.R, chunks, [&](int64_t s0, uint32_t blocks, uint32_t ch, uint32_t) {
        mi::inplace_scalar<T><<<blocks, mi::kBlock, 0, stream>>>(logits, ls, mask, ms, V, map, s0, ch, fill);
      });
      return after_launch("inplace_scalar");
    }
    case MI_VARIANT_VEC: {
      constexpr int VW = mi::Bits16B<T>::VW;
      const VecShape shape = inplace_shape(p.R * p.V * static_cast<int64_t>(sizeof(T)));
      const int64_t per = int64_t(mi::kBlock) * shape.unroll;
      const int64_t chunks = std::max<int64_t>(1, (p.V / VW + per - 1) / per);
      launch_slots(p.R, chunks, [&](int64_t s0, uint32_t blocks, uint32_t ch, uint32_t nrep) {
#define MI_INPLACE_VEC(UNROLL, POLICY)                                                            \
  mi::inplace_vec<T, UNROLL, POLICY><<<blocks, mi::kBlock, 0, stream>>>(logits, ls, mask, ms, V, W, map, s0, \
                                                                        ch, fill, any_out, nrep)
        // exactly the shapes inplace_shape returns
        if (shape.unroll == 2 && shape.policy == mi::kStoreDevice) MI_INPLACE_VEC(2, mi::kStoreDevice);
        else if (shape.unroll == 2) MI_INPLACE_VEC(2, mi::kStoreDeviceStream);
        else MI_INPLACE_VEC(4, mi::kStoreDeviceStream);
#undef MI_INPLACE_VEC
      }, any_out != nullptr);
      return after_launch("inplace_vec");
    }
    case MI_VARIANT_VEC_RESIDENT: {
      // cache-resident logits: keep the written lines in L2 (write-back) and
      // give each lane 16 vectors
      constexpr int VW = mi::Bits16B<T>::VW;
      const int64_t per = int64_t(mi::kBlock) * 16;
      const int64_t chunks = std::max<int64_t>(1, (p.V / VW + per - 1) / per);
      launch_slots(p.R, chunks, [&](int64_t s0, uint32_t blocks, uint32_t ch, uint32_t nrep) {
        mi::inplace_vec<T, 16, mi::kStoreWriteBack><<<blocks, mi::kBlock, 0, stream>>>(
            logits, ls, mask, ms, V, W, map, s0, ch, fill, any_out, nrep);
      }, any_out != nullptr);
      return after_launch("inplace_vec");
    }
    case MI_VARIANT_WRONLY: {
      const int64_t chunks = (p.W + 255) / 256;
      launch_slots(p.R, chunks, [&](int64_t s0, uint32_t blocks, uint32_t ch, uint32_t) {
        mi::inplace_wronly<T><<<blocks, mi::kBlock, 0, stream>>>(logits, ls, mask, ms, V, W, map, s0, ch, fill);
      });
      return after_launch("inplace_wronly");
    }
    default:
      return fail(MI_ERR_BAD_VARIANT, "variant %d", (int)variant);
  }
}

// Out of place over every row: apply != 0 masks [0, V), apply == 0 copies.
template <typename T>
mi_status_t run_out(void* out_v, int64_t os, const void* in_v, int64_t ls, const int32_t* mask_i, int64_t ms,
                    int64_t rows, int64_t cols, const Plan& p, int32_t apply, bool vec, hipStream_t stream) {
  T* out = static_cast<T*>(out_v);
  const T* in = static_cast<const T*>(in_v);
  const uint32_t* mask = reinterpret_cast<const uint32_t*>(mask_i);
  const T fill = static_cast<T>(p.fill);
  const int32_t V = static_cast<int32_t>(p.V), W = static_cast<int32_t>(p.W), C = static_cast<int32_t>(cols);
  (void)hipGetLastError();
  if (vec) {
    constexpr int VW = mi::Bits16B<T>::VW;
    const int64_t per = int64_t(mi::kBlock) * kOutShape.unroll;
    const int64_t chunks = std::max<int64_t>(1, (cols / VW + per - 1) / per);
    launch_slots(rows, chunks, [&](int64_t s0, uint32_t blocks, uint32_t ch, uint32_t) {
      mi::out_vec<T, kOutShape.unroll, kOutShape.policy><<<blocks, mi::kBlock, 0, stream>>>(
          out, os, in, ls, mask, ms, V, W, C, apply, s0, ch, fill);
    });
    return after_launch("out_vec");
  }
  const int64_t chunks = (cols + mi::kBlock * 8 - 1) / (mi::kBlock * 8);
  launch_slots(rows, chunks, [&](int64_t s0, uint32_t blocks, uint32_t ch, uint32_t) {
    mi::out_scalar<T><<<blocks, mi::kBlock, 0, stream>>>(out, os, in, ls, mask, ms, V, C, apply, s0, ch, fill);
  });
  return after_launch("out_scalar");
}

mi_variant_t auto_inplace(mi_dtype_t) { return MI_VARIANT_VEC; }

mi_status_t inplace_impl(void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t ls,
                         const int32_t* mask, int64_t mask_rows, int64_t mask_cols, int64_t ms, int64_t vocab_size,
                         const int32_t* indices, int64_t num_indices, double fill_value, mi_variant_t variant,
                         hipStream_t stream) {
  Plan p;
  mi_status_t st = check_common(logits, dtype, rows, cols, ls, mask, mask_rows, mask_cols, ms, vocab_size, indices,
                                num_indices, fill_value, &p);
  if (st != MI_OK) return st;
  if (overlaps(p.mask, p.logits)) return fail(MI_ERR_ALIAS, "mask overlaps logits");
  if (overlaps(p.indices, p.logits)) return fail(MI_ERR_ALIAS, "indices overlap logits");
  if (variant == MI_VARIANT_AUTO) variant = auto_inplace(dtype);
  if (variant != MI_VARIANT_SCALAR && variant != MI_VARIANT_VEC && variant != MI_VARIANT_WRONLY &&
      variant != MI_VARIANT_VEC_RESIDENT)
    return fail(MI_ERR_BAD_VARIANT, "unknown in-place variant %d", (int)variant);
  if (p.V == 0 || p.R == 0) return MI_OK;
  if (p.esize == 4) return run_inplace<uint32_t>(logits, ls, mask, ms, indices, p, variant, stream);
  return run_inplace<uint16_t>(logits, ls, mask, ms, indices, p, variant, stream);
}

mi_status_t out_impl(void* out, int64_t os, const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                     int64_t ls, const int32_t* mask, int64_t mask_rows, int64_t mask_cols, int64_t ms,
                     int64_t vocab_size, const int32_t* indices, int64_t num_indices, double fill_value,
                     mi_variant_t variant, hipStream_t stream) {
  if (!out && rows > 0 && cols > 0) return fail(MI_ERR_NULL_POINTER, "out is NULL");
  if (variant != MI_VARIANT_AUTO && variant != MI_VARIANT_SCALAR && variant != MI_VARIANT_VEC)
    return fail(MI_ERR_BAD_VARIANT, "variant %d has no out-of-place form", (int)variant);
  Plan p;
  mi_status_t st = check_common(logits, dtype, rows, cols, ls, mask, mask_rows, mask_cols, ms, vocab_size, indices,
                                num_indices, fill_value, &p);
  if (st != MI_OK) return st;
  if (os < cols || os > kMaxPitch)
    return fail(MI_ERR_BAD_SHAPE, "out_row_stride %lld must be in [cols %lld, 2^40]", (long long)os, (long long)cols);
  if (reinterpret_cast<uintptr_t>(out) % p.esize)
    return fail(MI_ERR_MISALIGNED, "out not aligned to its %d-byte elements", p.esize);
  ByteRange ob;
  if (!extent(out, rows, cols, os, p.esize, &ob)) return fail(MI_ERR_BAD_SHAPE, "out extent overflows");
  if (out == logits && os == ls) {  // the output is the input: this is the in-place apply
    return inplace_impl(out, dtype, rows, cols, ls, mask, mask_rows, mask_cols, ms, vocab_size, indices,
                        num_indices, fill_value, variant, stream);
  }
  if (overlaps(ob, p.logits)) return fail(MI_ERR_ALIAS, "out overlaps logits");
  if (overlaps(ob, p.mask)) return fail(MI_ERR_ALIAS, "out overlaps mask");
  if (overlaps(ob, p.indices)) return fail(MI_ERR_ALIAS, "out overlaps indices");
  if (rows == 0 || cols == 0) return MI_OK;

  // 16-byte vectors need out and logits rows at the same offset modulo 16.
  const bool same_phase =
      (reinterpret_cast<uintptr_t>(out) - reinterpret_cast<uintptr_t>(logits)) % 16 == 0 &&
      (rows == 1 || ((os - ls) * p.esize) % 16 == 0);
  const bool vec = variant == MI_VARIANT_SCALAR ? false : same_phase;
  // Without an index list every row is processed in one fused pass.  With one,
  // out first becomes a copy of logits and the listed rows are then masked in
  // place on out (rows outside the list stay copies).
  const int32_t apply = (indices == nullptr && p.V > 0) ? 1 : 0;
  st = p.esize == 4 ? run_out<uint32_t>(out, os, logits, ls, mask, ms, rows, cols, p, apply, vec, stream)
                    : run_out<uint16_t>(out, os, logits, ls, mask, ms, rows, cols, p, apply, vec, stream);
  if (st != MI_OK || indices == nullptr || p.V == 0 || p.R == 0) return st;
  const mi_variant_t iv = variant == MI_VARIANT_SCALAR ? MI_VARIANT_SCALAR : auto_inplace(dtype);
  return p.esize == 4 ? run_inplace<uint32_t>(out, os, mask, ms, indices, p, iv, stream)
                      : run_inplace<uint16_t>(out, os, mask, ms, indices, p, iv, stream);
}

mi_status_t rows_impl(void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t ls, const int32_t* mask,
                      int64_t mask_rows, int64_t mask_cols, int64_t ms, int64_t vocab_size, const int8_t* gate,
                      uint8_t* any_out, double fill_value, hipStream_t stream) {
  Plan p;
  mi_status_t st = check_common(logits, dtype, rows, cols, ls, mask, mask_rows, mask_cols, ms, vocab_size, nullptr,
                                0, fill_value, &p);
  if (st != MI_OK) return st;
  ByteRange gb, ab;
  if (!extent(gate, gate ? 1 : 0, rows, rows, 1, &gb) || !extent(any_out, any_out ? 1 : 0, rows, rows, 1, &ab))
    return fail(MI_ERR_BAD_SHAPE, "row flag extent overflows");
  if (overlaps(p.mask, p.logits)) return fail(MI_ERR_ALIAS, "mask overlaps logits");
  if (overlaps(gb, p.logits)) return fail(MI_ERR_ALIAS, "row_needs_mask overlaps logits");
  if (overlaps(ab, p.logits) || overlaps(ab, p.mask) || overlaps(ab, gb))
    return fail(MI_ERR_ALIAS, "row_any_allowed overlaps an input");
  if (p.R == 0 || (p.V == 0 && !any_out)) return MI_OK;
  // The per-row report lives in the vector kernel (its first block per row).
  if (p.esize == 4) return run_inplace<uint32_t>(logits, ls, mask, ms, nullptr, p, MI_VARIANT_VEC, stream, gate, any_out);
  return run_inplace<uint16_t>(logits, ls, mask, ms, nullptr, p, MI_VARIANT_VEC, stream, gate, any_out);
}

}  // namespace

MI_API mi_status_t mi_apply_bitmask_rows(void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                         int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                         int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                         const int8_t* row_needs_mask, uint8_t* row_any_allowed, double fill_value,
                                         hipStream_t stream) {
  return rows_impl(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols, mask_row_stride,
                   vocab_size, row_needs_mask, row_any_allowed, fill_value, stream);
}

MI_API mi_status_t mi_apply_bitmask_inplace(void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                            int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                            int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                            const int32_t* indices, int64_t num_indices, double fill_value,
                                            hipStream_t stream) {
  return inplace_impl(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols, mask_row_stride,
                      vocab_size, indices, num_indices, fill_value, MI_VARIANT_AUTO, stream);
}

MI_API mi_status_t mi_apply_bitmask_inplace_ex(void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                               int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                               int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                               const int32_t* indices, int64_t num_indices, double fill_value,
                                               mi_variant_t variant, hipStream_t stream) {
  return inplace_impl(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols, mask_row_stride,
                      vocab_size, indices, num_indices, fill_value, variant, stream);
}

MI_API mi_status_t mi_apply_bitmask_out(void* out, int64_t out_row_stride, const void* logits, mi_dtype_t dtype,
                                        int64_t rows, int64_t cols, int64_t logits_row_stride, const int32_t* mask,
                                        int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
                                        int64_t vocab_size, const int32_t* indices, int64_t num_indices,
                                        double fill_value, hipStream_t stream) {
  return out_impl(out, out_row_stride, logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols,
                  mask_row_stride, vocab_size, indices, num_indices, fill_value, MI_VARIANT_AUTO, stream);
}

MI_API mi_status_t mi_apply_bitmask_out_ex(void* out, int64_t out_row_stride, const void* logits, mi_dtype_t dtype,
                                           int64_t rows, int64_t cols, int64_t logits_row_stride, const int32_t* mask,
                                           int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
                                           int64_t vocab_size, const int32_t* indices, int64_t num_indices,
                                           double fill_value, mi_variant_t variant, hipStream_t stream) {
  return out_impl(out, out_row_stride, logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols,
                  mask_row_stride, vocab_size, indices, num_indices, fill_value, variant, stream);
}

// ---------------------------------------------------------------------------
// Host-memory entry points (CPU tensors)
// ---------------------------------------------------------------------------

namespace {

int resolve_threads(int threads, int64_t elements) {
  if (elements < (int64_t(1) << 20)) return 1;  // spawning threads costs more than small rows
  if (threads > 0) return threads;
  const unsigned hc = std::thread::hardware_concurrency();
  return hc > 1 ? static_cast<int>(hc / 2) : 1;
}

mi_status_t host_rows(const Plan& p, int64_t rows, const int32_t* indices, std::vector<int64_t>* out) {
  out->clear();
  if (!indices) {
    out->resize(rows);
    for (int64_t i = 0; i < rows; ++i) (*out)[i] = i;
    return MI_OK;
  }
  out->reserve(p.R);
  for (int64_t i = 0; i < p.R; ++i) {  // host memory: the values can be checked
    const int64_t r = indices[i];
    if (r < 0 || r >= p.row_limit)
      return fail(MI_ERR_BAD_INDICES, "index %lld outside [0, %lld)", (long long)r, (long long)p.row_limit);
    out->push_back(r);
  }
  return MI_OK;
}

template <typename T>
void host_apply(void* logits, int64_t ls, const int32_t* mask, int64_t ms, const Plan& p,
                const std::vector<int64_t>& rows, int threads) {
  mi_host::apply_parallel(static_cast<T*>(logits), ls, reinterpret_cast<const uint32_t*>(mask), ms, p.V,
                          rows.data(), static_cast<int64_t>(rows.size()), static_cast<T>(p.fill),
                          resolve_threads(threads, static_cast<int64_t>(rows.size()) * p.V));
}

}  // namespace

MI_API mi_status_t mi_apply_bitmask_inplace_host(void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                                 int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                                 int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                                 const int32_t* indices, int64_t num_indices, double fill_value,
                                                 int num_threads) {
  Plan p;
  mi_status_t st = check_common(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols,
                                mask_row_stride, vocab_size, indices, num_indices, fill_value, &p);
  if (st != MI_OK) return st;
  if (overlaps(p.mask, p.logits)) return fail(MI_ERR_ALIAS, "mask overlaps logits");
  if (overlaps(p.indices, p.logits)) return fail(MI_ERR_ALIAS, "indices overlap logits");
  if (p.V == 0 || p.R == 0) return MI_OK;
  std::vector<int64_t> rs;
  st = host_rows(p, rows, indices, &rs);
  if (st != MI_OK) return st;
  if (p.esize == 4) host_apply<uint32_t>(logits, logits_row_stride, mask, mask_row_stride, p, rs, num_threads);
  else host_apply<uint16_t>(logits, logits_row_stride, mask, mask_row_stride, p, rs, num_threads);
  return MI_OK;
}

MI_API mi_status_t mi_apply_bitmask_out_host(void* out, int64_t out_row_stride, const void* logits, mi_dtype_t dtype,
                                             int64_t rows, int64_t cols, int64_t logits_row_stride,
                                             const int32_t* mask, int64_t mask_rows, int64_t mask_cols,
                                             int64_t mask_row_stride, int64_t vocab_size, const int32_t* indices,
                                             int64_t num_indices, double fill_value, int num_threads) {
  if (!out && rows > 0 && cols > 0) return fail(MI_ERR_NULL_POINTER, "out is NULL");
  Plan p;
  mi_status_t st = check_common(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols,
                                mask_row_stride, vocab_size, indices, num_indices, fill_value, &p);
  if (st != MI_OK) return st;
  if (out_row_stride < cols || out_row_stride > kMaxPitch)
    return fail(MI_ERR_BAD_SHAPE, "out_row_stride %lld must be in [cols %lld, 2^40]", (long long)out_row_stride,
                (long long)cols);
  if (reinterpret_cast<uintptr_t>(out) % p.esize)
    return fail(MI_ERR_MISALIGNED, "out not aligned to its %d-byte elements", p.esize);
  ByteRange ob;
  if (!extent(out, rows, cols, out_row_stride, p.esize, &ob)) return fail(MI_ERR_BAD_SHAPE, "out extent overflows");
  if (out == logits && out_row_stride == logits_row_stride)
    return mi_apply_bitmask_inplace_host(out, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols,
                                         mask_row_stride, vocab_size, indices, num_indices, fill_value, num_threads);
  if (overlaps(ob, p.logits)) return fail(MI_ERR_ALIAS, "out overlaps logits");
  if (overlaps(ob, p.mask)) return fail(MI_ERR_ALIAS, "out overlaps mask");
  if (overlaps(ob, p.indices)) return fail(MI_ERR_ALIAS, "out overlaps indices");
  std::vector<int64_t> rs;
  st = host_rows(p, rows, indices, &rs);  // check the index list before writing anything
  if (st != MI_OK) return st;
  for (int64_t r = 0; r < rows; ++r)
    std::memcpy(static_cast<char*>(out) + r * out_row_stride * p.esize,
                static_cast<const char*>(logits) + r * logits_row_stride * p.esize, static_cast<size_t>(cols) * p.esize);
  if (p.V == 0 || p.R == 0) return MI_OK;
  if (p.esize == 4) host_apply<uint32_t>(out, out_row_stride, mask, mask_row_stride, p, rs, num_threads);
  else host_apply<uint16_t>(out, out_row_stride, mask, mask_row_stride, p, rs, num_threads);
  return MI_OK;
}

// ---------------------------------------------------------------------------
// Fused apply + sample
// ---------------------------------------------------------------------------

namespace {

// Checks for a call without a mask: every token below V takes part, and V
// defaults to cols.
mi_status_t check_logits_only(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t ls,
                              int64_t vocab_size, Plan* p) {
  if (!logits && rows > 0 && cols > 0) return fail(MI_ERR_NULL_POINTER, "logits is NULL");
  if (!valid_dtype(static_cast<int>(dtype))) return fail(MI_ERR_BAD_DTYPE, "unknown dtype %d", (int)dtype);
  if (rows < 0 || cols < 0) return fail(MI_ERR_BAD_SHAPE, "negative size (rows %lld, cols %lld)", (long long)rows,
                                        (long long)cols);
  if (rows > kMaxRows || cols > kMaxCols) return fail(MI_ERR_BAD_SHAPE, "size above the limits");
  if (ls < cols || ls > kMaxPitch)
    return fail(MI_ERR_BAD_SHAPE, "logits_row_stride %lld must be in [cols %lld, 2^40]", (long long)ls, (long long)cols);
  if (vocab_size < -1 || vocab_size > cols)
    return fail(MI_ERR_BAD_VOCAB, "vocab_size %lld outside [0, cols %lld] (or -1)", (long long)vocab_size,
                (long long)cols);
  p->V = vocab_size == -1 ? cols : vocab_size;
  p->W = (p->V + 31) / 32;
  p->R = rows;
  p->row_limit = rows;
  p->esize = elem_bytes(dtype);
  if (reinterpret_cast<uintptr_t>(logits) % p->esize)
    return fail(MI_ERR_MISALIGNED, "logits not aligned to its %d-byte elements", p->esize);
  if (!extent(logits, rows, cols, ls, p->esize, &p->logits)) return fail(MI_ERR_BAD_SHAPE, "buffer extent overflows");
  return MI_OK;
}

}  // namespace

MI_API mi_status_t mi_apply_bitmask_sample(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                           int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                           int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                           const mi_sample_params_t* params, int64_t* tokens, hipStream_t stream) {
  if (!params) return fail(MI_ERR_NULL_POINTER, "params is NULL");
  if (!tokens && rows > 0) return fail(MI_ERR_NULL_POINTER, "tokens is NULL");
  Plan p;
  mi_status_t st;
  if (mask) {
    st = check_common(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols, mask_row_stride,
                      vocab_size, nullptr, 0, 0.0, &p);
  } else {
    st = check_logits_only(logits, dtype, rows, cols, logits_row_stride, vocab_size, &p);
  }
  if (st != MI_OK) return st;
  // the kernel addresses a row through 32-bit byte offsets
  if (p.V > kMaxSampleVocab) return fail(MI_ERR_BAD_SHAPE, "vocab size above 2^28 (the sampler's limit)");
  ByteRange tb;
  if (!extent(tokens, tokens ? 1 : 0, rows, rows, 8, &tb)) return fail(MI_ERR_BAD_SHAPE, "tokens extent overflows");
  if (reinterpret_cast<uintptr_t>(tokens) % 8) return fail(MI_ERR_MISALIGNED, "tokens not 8-byte aligned");
  if (overlaps(tb, p.logits) || overlaps(tb, p.mask)) return fail(MI_ERR_ALIAS, "tokens overlap an input");
  for (const void* q : {static_cast<const void*>(params->temperature), static_cast<const void*>(params->top_k),
                        static_cast<const void*>(params->top_p), static_cast<const void*>(params->min_p)})
    if (reinterpret_cast<uintptr_t>(q) % 4) return fail(MI_ERR_MISALIGNED, "a per-row parameter array is not 4-byte aligned");
  if (rows == 0) return MI_OK;

  mi::SampleArgs a{params->temperature, params->top_k, params->top_p, params->min_p,
                   params->temperature_all, params->top_k_all, params->top_p_all, params->min_p_all,
                   static_cast<uint32_t>(params->seed), static_cast<uint32_t>(params->seed >> 32),
                   static_cast<uint32_t>(params->offset), static_cast<uint32_t>(params->offset >> 32)};
  const uint32_t* m = reinterpret_cast<const uint32_t*>(mask);
  const int32_t V = static_cast<int32_t>(p.V);
  (void)hipGetLastError();
  constexpr int64_t kRowsPerLaunch = int64_t(1) << 20;   // blocks * threads < 2^32
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const uint32_t n = static_cast<uint32_t>(std::min(kRowsPerLaunch, rows - r0));
    const int64_t mr0 = m ? r0 * mask_row_stride : 0;
    // per-row parameter arrays and the row counter of the generator start at r0
    mi::SampleArgs ar = a;
    if (ar.temperature) ar.temperature += r0;
    if (ar.top_k) ar.top_k += r0;
    if (ar.top_p) ar.top_p += r0;
    if (ar.min_p) ar.min_p += r0;
    const auto* lg = static_cast<const char*>(logits) + r0 * logits_row_stride * p.esize;
    const uint32_t* mk = m ? m + mr0 : nullptr;
    // Histogram LDS only when some row may filter; deep load pipeline when a
    // compute unit holds one row at a time (rows <= 256), shallow otherwise.
    const bool may_filter = ar.top_k || ar.top_p || ar.top_k_all > 0 || ar.top_p_all < 1.0f;
    const bool deep = n <= 256;
    const int threads = deep ? 1024 : 256;
    const size_t lds = may_filter ? mi::sample_hist_bytes(threads) : 0;
#define MI_SAMPLE(TAG, BITS, BYTES, THREADS)                                                                   \
  mi::sample_rows<TAG, BYTES, THREADS><<<n, THREADS, lds, stream>>>(reinterpret_cast<const BITS*>(lg),          \
                                                                    logits_row_stride, mk, mask_row_stride, V,   \
                                                                    ar, r0, tokens + r0)
    switch (dtype) {
      case MI_DTYPE_F32:
        if (deep) MI_SAMPLE(mi::F32Bits, uint32_t, 128, 1024); else MI_SAMPLE(mi::F32Bits, uint32_t, 64, 256);
        break;
      case MI_DTYPE_F16:
        if (deep) MI_SAMPLE(mi::F16Bits, uint16_t, 128, 1024); else MI_SAMPLE(mi::F16Bits, uint16_t, 64, 256);
        break;
      default:
        if (deep) MI_SAMPLE(mi::BF16Bits, uint16_t, 128, 1024); else MI_SAMPLE(mi::BF16Bits, uint16_t, 64, 256);
    }
#undef MI_SAMPLE
  }
  return after_launch("sample_rows");
}

MI_API mi_status_t mi_resolve_vocab_size(int64_t cols, int64_t mask_cols, int64_t vocab_size, int64_t* vocab_out) {
  if (!vocab_out) return fail(MI_ERR_NULL_POINTER, "vocab_out is NULL");
  return resolve_vocab(cols, mask_cols, vocab_size, vocab_out);
}

MI_API mi_status_t mi_fill_value_bits(double fill_value, mi_dtype_t dtype, uint32_t* bits_out) {
  if (!bits_out) return fail(MI_ERR_NULL_POINTER, "bits_out is NULL");
  if (!valid_dtype(static_cast<int>(dtype))) return fail(MI_ERR_BAD_DTYPE, "unknown dtype %d", (int)dtype);
  *bits_out = fill_pattern(fill_value, dtype);
  return MI_OK;
}

MI_API const char* mi_status_string(mi_status_t s) {
  switch (s) {
    case MI_OK: return "MI_OK";
    case MI_ERR_NULL_POINTER: return "MI_ERR_NULL_POINTER";
    case MI_ERR_BAD_DTYPE: return "MI_ERR_BAD_DTYPE";
    case MI_ERR_BAD_SHAPE: return "MI_ERR_BAD_SHAPE";
    case MI_ERR_BAD_VOCAB: return "MI_ERR_BAD_VOCAB";
    case MI_ERR_BAD_INDICES: return "MI_ERR_BAD_INDICES";
    case MI_ERR_ALIAS: return "MI_ERR_ALIAS";
    case MI_ERR_MISALIGNED: return "MI_ERR_MISALIGNED";
    case MI_ERR_BAD_VARIANT: return "MI_ERR_BAD_VARIANT";
    case MI_ERR_HIP: return "MI_ERR_HIP";
  }
  return "MI_ERR_UNKNOWN";
}

MI_API const char* mi_last_error_message(void) { return g_message; }
