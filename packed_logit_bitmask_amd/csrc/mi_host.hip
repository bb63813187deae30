// Host-memory entry points (CPU tensors) and the library's small helpers:
// vocab-size rule, fill bits, status text, the last error message and the
// host loop in use.  Declared in include/mi_bitmask.h.

#include "mi_bitmask.h"

#include <cstdint>
#include <cstring>
#include <thread>

#include "host_apply.h"
#include "host_checks.h"

using namespace mi_abi;

namespace {

int resolve_threads(int threads, int64_t elements) {
  if (elements < (int64_t(1) << 20)) return 1;  // spawning threads costs more than small rows
  if (threads > 0) return threads;
  const unsigned hc = std::thread::hardware_concurrency();
  return hc > 1 ? static_cast<int>(hc / 2) : 1;
}

// Host memory can be read, so an index list is checked value by value
// before anything is written.
mi_status_t check_host_indices(const Plan& p, const int32_t* indices) {
  for (int64_t i = 0; indices && i < p.R; ++i) {
    const int64_t r = indices[i];
    if (r < 0 || r >= p.row_limit)
      return fail(MI_ERR_BAD_INDICES, "index %lld outside [0, %lld)", (long long)r, (long long)p.row_limit);
  }
  return MI_OK;
}

template <typename T>
void host_apply(void* logits, int64_t ls, const int32_t* mask, int64_t ms, const Plan& p, const int32_t* indices,
                int threads) {
  const uint32_t* m = reinterpret_cast<const uint32_t*>(mask);
  const int nt = resolve_threads(threads, p.R * p.V);
  if constexpr (sizeof(T) == 4)
    mi_host::apply_u32(static_cast<uint32_t*>(logits), ls, m, ms, p.V, indices, p.R, static_cast<uint32_t>(p.fill), nt);
  else
    mi_host::apply_u16(static_cast<uint16_t*>(logits), ls, m, ms, p.V, indices, p.R, static_cast<uint16_t>(p.fill), nt);
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
  st = check_host_indices(p, indices);
  if (st != MI_OK) return st;
  if (p.esize == 4) host_apply<uint32_t>(logits, logits_row_stride, mask, mask_row_stride, p, indices, num_threads);
  else host_apply<uint16_t>(logits, logits_row_stride, mask, mask_row_stride, p, indices, num_threads);
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
  st = check_host_indices(p, indices);  // before anything is written
  if (st != MI_OK) return st;
  for (int64_t r = 0; r < rows; ++r)
    std::memcpy(static_cast<char*>(out) + r * out_row_stride * p.esize,
                static_cast<const char*>(logits) + r * logits_row_stride * p.esize, static_cast<size_t>(cols) * p.esize);
  if (p.V == 0 || p.R == 0) return MI_OK;
  if (p.esize == 4) host_apply<uint32_t>(out, out_row_stride, mask, mask_row_stride, p, indices, num_threads);
  else host_apply<uint16_t>(out, out_row_stride, mask, mask_row_stride, p, indices, num_threads);
  return MI_OK;
}

// ---------------------------------------------------------------------------
// Fused apply + sample
// ---------------------------------------------------------------------------

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

MI_API const char* mi_host_isa(void) { return mi_host::isa(); }
