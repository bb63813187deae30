// Host side of the packed-bitmask apply on the device: the kernel shape
// table, grid splitting and the launches of the apply kernels, and the
// device apply entry points.  The C ABI is declared (and documented) in
// include/mi_bitmask.h.
//
// Nothing here allocates, synchronises or touches device memory; every
// check runs before the first HIP call, so a rejected call enqueues nothing.

#include "mi_bitmask.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "apply_kernels.h"
#include "host_checks.h"

using namespace mi_abi;

namespace {

constexpr int64_t kMaxBlocksPerLaunch = (int64_t(1) << 24) - 1;  // blocks * 256 < 2^32

// Shape of the 16-byte-vector kernels: vectors per lane (unroll) and the
// store cache policy.  Picked from measurements on MI355X, cold from HBM
// (buffer sets rotated so that the bytes the launches touch cycle through
// more than twice the 256 MB Infinity Cache), in place:
//  - below 1 GB of writes, two vectors per lane with device-scope
//    write-through non-temporal stores.  On the 34.8 MB bf16 launch of 128
//    rows x 128000 tokens this took 13.9 us against 15.8 us with
//    write-through stores that are not marked non-temporal, and against
//    14.2-14.3 us with one or four vectors per lane; loads marked
//    non-temporal or system-coherent were 1-2 % slower;
//  - from 1 GB, four vectors per lane, non-temporal: 1-4 % ahead on the
//    large mixed-kind workloads.
// Out of place, two vectors per lane with write-through non-temporal stores
// was best at every size measured.
struct VecShape {
  int unroll;
  int policy;
};

constexpr int64_t kLargeWriteBytes = int64_t(1) << 30;

VecShape inplace_shape(int64_t write_bytes) {
  if (write_bytes < kLargeWriteBytes) return {2, mi::kStoreDeviceStream};
  return {4, mi::kStoreDeviceStream};
}

constexpr VecShape kOutShape{2, mi::kStoreDeviceStream};

// Out of place with an index list: one fused pass up to this many entries
// (each block compares its row with every entry), copy then in place beyond.
constexpr int64_t kFusedListMax = 1024;

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
        if (shape.unroll == 2) MI_INPLACE_VEC(2, mi::kStoreDeviceStream);
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

// Out of place over every row: apply != 0 masks [0, V), apply == 0 copies;
// with `listed` set, only the rows the list holds are masked.
template <typename T>
mi_status_t run_out(void* out_v, int64_t os, const void* in_v, int64_t ls, const int32_t* mask_i, int64_t ms,
                    int64_t rows, int64_t cols, const Plan& p, int32_t apply, const mi::ListedRows& listed, bool vec,
                    hipStream_t stream) {
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
          out, os, in, ls, mask, ms, V, W, C, apply, listed, s0, ch, fill);
    });
    return after_launch("out_vec");
  }
  const int64_t chunks = (cols + mi::kBlock * 8 - 1) / (mi::kBlock * 8);
  launch_slots(rows, chunks, [&](int64_t s0, uint32_t blocks, uint32_t ch, uint32_t) {
    mi::out_scalar<T><<<blocks, mi::kBlock, 0, stream>>>(out, os, in, ls, mask, ms, V, C, apply, listed, s0, ch, fill);
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
  // One fused pass over every row: without an index list each row is masked;
  // with a list of at most kFusedListMax entries each block finds whether the
  // list holds its row.  A longer list would cost every block a long scan:
  // out first becomes a copy of logits and the listed rows are then masked in
  // place on out (rows outside the list stay copies).
  const bool fused_list = indices != nullptr && p.V > 0 && num_indices > 0 && num_indices <= kFusedListMax;
  const int32_t apply = (indices == nullptr && p.V > 0) ? 1 : 0;
  mi::ListedRows listed;
  if (fused_list) listed = mi::ListedRows{indices, static_cast<int32_t>(num_indices), p.row_limit};
  st = p.esize == 4 ? run_out<uint32_t>(out, os, logits, ls, mask, ms, rows, cols, p, apply, listed, vec, stream)
                    : run_out<uint16_t>(out, os, logits, ls, mask, ms, rows, cols, p, apply, listed, vec, stream);
  if (st != MI_OK || indices == nullptr || fused_list || p.V == 0 || p.R == 0) return st;
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
