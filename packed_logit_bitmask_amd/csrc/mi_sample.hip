// Host side of the fused apply + sampler: argument checks and the launch of
// mi::sample_rows (sample_kernel.h).  Declared in include/mi_bitmask.h.

#include "mi_bitmask.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "host_checks.h"
#include "sample_kernel.h"

using namespace mi_abi;

namespace {

constexpr int64_t kMaxSampleVocab = int64_t(1) << 28;

// Segmented rows (no filter, no min-p): at most this many rows per launch
// (fewer when every row is greedy), about this many blocks in all, and at
// most this many segments per row (each posts one atomic to the row's word).
constexpr int64_t kSplitRows = 128;
constexpr int64_t kSplitRowsGreedy = 2;
constexpr int64_t kSplitBlocks = 512;
constexpr int64_t kMaxSegments = 32;

// Filtered 16-bit rows: more rows than this (the compute units) take the
// 8-bit-counter histogram in 512-thread blocks, two per unit, when a row has
// at most kFine8Vocab tokens.
constexpr int64_t kFine16Rows = 256;
constexpr int64_t kFine8Vocab = 65536;

// Filtered 16-bit rows, at most this many in a batch, split over several
// blocks when the caller gives a workspace (see split_hist in
// sample_kernel.h).  The histogram pass takes at most kSplitHistBlocks
// blocks in all (one per compute unit) and at most kMaxHistSegments per row
// (every segment adds its nonzero counts to the row's histogram by atomics,
// so fewer, longer segments contend less), each under 65536 tokens so its
// 16-bit counters cannot wrap.  The row limit is where the split stops
// paying: on MI355X at 128000 bf16 tokens a row, a batch of 32 rows draws
// faster split in every mode (top-k 30.4 against 32.1 us, top-p 37.7
// against 46.1), while from 40 rows on one block per row is up to 10 %
// faster for top-k and for the filters together, and ties for top-p.
constexpr int64_t kSplitFilteredRows = 32;
constexpr int64_t kSplitHistBlocks = 256;

// Filtered 16-bit batches of more rows than compute units, at most this
// many, hand out their heavy rows first (row_classes, heavy_first_row in
// sample_kernel.h) when the caller gives a workspace for one bit per row
// (rounded up to 256 bytes).  Every wave of sample_rows then ranks the
// batch's flags in its prologue, 128 rows per lane.
constexpr int64_t kOrderMaxRows = 8192;
constexpr int64_t kMaxHistSegments = 8;
constexpr int64_t kSplitHistMaxSeg = 65280;

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

// ---- Scratch of mi_apply_bitmask_sample_noalloc: the split path's workspace
// as a device array of the library, for callers that cannot allocate.  Each
// GPU holds its own copy (8.4 MB, enough for kNoAllocRows split rows) until
// the process ends.  Host code never passes the array's name to a kernel
// (on the host it stands for no device address): it takes each device's
// address once, through hipGetSymbolAddress, and uses that.
constexpr int64_t kNoAllocRows = 32;
constexpr int64_t kScratchBytes = kNoAllocRows * mi::split_workspace_bytes(1);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Whether a batch takes the split filtered path (filtered 16-bit rows spread
// over several blocks through the workspace): few rows, long enough to split.
bool split_filtered_batch(mi_dtype_t dtype, int64_t rows, int64_t V) {
  return dtype != MI_DTYPE_F32 && rows >= 1 && rows <= kSplitFilteredRows && V >= 8192;
}

// Whether a batch may order its rows heavy first through the workspace:
// 16-bit rows, more of them than kFine16Rows (so more than the compute
// units hold at once), longer than a 512-thread block holds in registers,
// so that a sparse row takes the listed search and costs far less than a
// dense one.  (At 8192 tokens, where every row is held in registers,
// ordering B=1024 fp16 rows cost 2.5 us more than it saved.)
bool ordered_batch(mi_dtype_t dtype, int64_t rows, int64_t V) {
  return dtype != MI_DTYPE_F32 && rows > kFine16Rows && rows <= kOrderMaxRows && V > 4 * 8 * 512;
}

// Workspace bytes a batch can use (0: none).
int64_t workspace_need(mi_dtype_t dtype, int64_t rows, int64_t V) {
  if (split_filtered_batch(dtype, rows, V)) return mi::split_workspace_bytes(rows);
  if (ordered_batch(dtype, rows, V)) return (mi::row_class_bytes(rows) + 255) / 256 * 256;
  return 0;
}

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the GPU that `stream` runs on (the
// current device for the null stream), looked up once per device with that
// device current: each GPU holds its own copy of the array.
mi_status_t scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(MI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(MI_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(MI_ERR_HIP, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return fail(MI_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (back != hipSuccess) return fail(MI_ERR_HIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(back));
    }
    if (e != hipSuccess || !p)
      return fail(MI_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MI_OK;
}

// use_scratch: take the split path's workspace from `scratch` (workspace and
// workspace_bytes are then ignored).
mi_status_t sample_impl(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
                        const int32_t* mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
                        int64_t vocab_size, const mi_sample_params_t* params, int64_t* tokens, void* workspace,
                        int64_t workspace_bytes, hipStream_t stream, bool use_scratch = false) {
  if (!params) return fail(MI_ERR_NULL_POINTER, "params is NULL");
  if (!tokens && rows > 0) return fail(MI_ERR_NULL_POINTER, "tokens is NULL");
  if (workspace_bytes < 0) return fail(MI_ERR_BAD_SHAPE, "negative workspace_bytes");
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
  // The workspace is used only when this batch can split its filtered rows
  // or order them heavy first, and it is large enough; then it must not
  // overlap anything else.
  const int64_t ws_need = workspace_need(dtype, rows, p.V);
  // whether any row may take a filter (only such batches use a workspace)
  const bool params_filter = params->top_k || params->top_p || params->min_p || params->top_k_all > 0 ||
                             params->top_p_all < 1.0f || params->min_p_all > 0.f;
  if (use_scratch) {
    // kNoAllocRows equals the split limit, and the flags of the largest
    // ordered batch take far less, so no batch needs more than the array
    // holds; the check guards the limits against drifting apart.
    static_assert((mi::row_class_bytes(kOrderMaxRows) + 255) / 256 * 256 <= kScratchBytes,
                  "the scratch holds the flags of the largest ordered batch");
    if (params_filter && ws_need > kScratchBytes)
      return fail(MI_ERR_BAD_SHAPE,
                  "%lld rows of %lld tokens need %lld bytes of scratch; the no-alloc entry point holds %lld "
                  "(%lld such rows): split the batch, or pass a workspace to mi_apply_bitmask_sample_ws",
                  (long long)rows, (long long)p.V, (long long)ws_need, (long long)kScratchBytes,
                  (long long)kNoAllocRows);
    workspace = nullptr;
    workspace_bytes = 0;
  }
  bool use_ws = workspace && ws_need > 0 && workspace_bytes >= ws_need;
  if (use_ws) {
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(MI_ERR_MISALIGNED, "workspace not 16-byte aligned");
    ByteRange wb;
    if (!extent(workspace, 1, ws_need, ws_need, 1, &wb)) return fail(MI_ERR_BAD_SHAPE, "workspace extent overflows");
    if (overlaps(wb, p.logits) || overlaps(wb, p.mask) || overlaps(wb, tb))
      return fail(MI_ERR_ALIAS, "workspace overlaps logits, mask or tokens");
    const void* per_row[4] = {params->temperature, params->top_k, params->top_p, params->min_p};
    for (const void* q : per_row) {
      ByteRange qb;
      if (q && extent(q, 1, rows * 4, rows * 4, 1, &qb) && overlaps(wb, qb))
        return fail(MI_ERR_ALIAS, "workspace overlaps a per-row parameter array");
    }
  }
  if (rows == 0) return MI_OK;
  if (use_scratch && params_filter && ws_need > 0) {  // every argument check has passed
    st = scratch_address(stream, &workspace);
    if (st != MI_OK) return st;
    workspace_bytes = ws_need;
    use_ws = true;
  }

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
    // Histogram LDS only when some row may filter; 1024-thread blocks when a
    // compute unit holds one row at a time (rows <= 256), 256-thread blocks
    // otherwise, 128 bytes in flight per thread either way (with 64 bytes
    // the 256-thread blocks took B=1024 fp16 greedy 7 % longer).
    // Filtered 16-bit rows search the full 16-bit key histogram: in
    // 1024-thread blocks with 16-bit counters (128 KB, most of a compute
    // unit's LDS) when there are at most as many rows as compute units, else
    // in 512-thread blocks with 8-bit counters (64 KB), two to a unit, for
    // rows of at most 65536 tokens (longer rows would more often hold 256
    // equal logits, which sends a row to the radix search).  The radix
    // histograms of that fallback share the space.
    const bool may_filter = ar.top_k || ar.top_p || ar.top_k_all > 0 || ar.top_p_all < 1.0f;
    const bool may_min_p = ar.min_p || ar.min_p_all > 0.f;
    const bool fine = may_filter && dtype != MI_DTYPE_F32;
    // Rows with neither a filter nor min-p need no whole-row state: with few
    // rows they are split into segments, one 256-thread block each, so every
    // compute unit has work (see sample_rows).
    // A launch of greedy rows alone gains only at one or two rows: one block
    // reads a row about as fast as a few blocks that then merge.
    const bool greedy_only = !ar.temperature && !(ar.temperature_all > 0.f);
    // With a workspace, a small batch that may filter splits its rows too
    // (split_hist, split_search, then a segmented draw).
    const bool split_filtered = use_ws && split_filtered_batch(dtype, rows, p.V) && (may_filter || may_min_p);
    int32_t nseg = 1, seg_len = V;
    if ((split_filtered || (!may_filter && !may_min_p && n <= (greedy_only ? kSplitRowsGreedy : kSplitRows))) &&
        V >= 8192) {
      nseg = static_cast<int32_t>(std::min<int64_t>({(kSplitBlocks + n - 1) / n, kMaxSegments, (V + 4095) / 4096}));
      seg_len = static_cast<int32_t>(((V + nseg - 1) / nseg + 255) / 256 * 256);
      nseg = (V + seg_len - 1) / seg_len;
    }
    const bool fine8 = fine && n > kFine16Rows && V <= kFine8Vocab;
    // heavy rows first, given a mask to tell dense rows from sparse ones:
    // rows of at most kFine8Vocab tokens (512-thread blocks, two to a unit)
    // with top-p or min-p, whose draws over a dense row may take most of its
    // tokens (with top-k alone the order measured 2.5 us slower); longer
    // rows (1024-thread blocks, one to a unit) with any filter: a dense one
    // of those costs far more than a sparse one even for top-k
    const bool may_p = ar.top_p || ar.top_p_all < 1.0f;
    const bool long_rows = fine && !fine8 && V > kFine8Vocab;
    const uint32_t* heavy = nullptr;
    if (use_ws && ordered_batch(dtype, rows, p.V) && nseg == 1 && mk &&
        ((fine8 && (may_p || may_min_p)) || long_rows)) {
      static_assert(kOrderMaxRows <= 128 * 64, "heavy_first_row reads at most 128 rows' flags per lane");
      uint8_t* flags = static_cast<uint8_t*>(workspace);
      // one batch of 16, 32 or 64 loads per lane, as the row needs; batches
      // of 64 beyond 131072 tokens
      if (V <= 64 * 16 * 32)
        mi::row_classes<16><<<(n + 7) / 8, 512, 0, stream>>>(mk, mask_row_stride, V, static_cast<int32_t>(n), flags);
      else if (V <= 64 * 32 * 32)
        mi::row_classes<32><<<(n + 7) / 8, 512, 0, stream>>>(mk, mask_row_stride, V, static_cast<int32_t>(n), flags);
      else
        mi::row_classes<64><<<(n + 7) / 8, 512, 0, stream>>>(mk, mask_row_stride, V, static_cast<int32_t>(n), flags);
      heavy = reinterpret_cast<const uint32_t*>(flags);
    }
    const bool deep = (n <= 256 || fine) && nseg == 1;
    const int threads = fine8 ? 512 : deep ? 1024 : 256;
    // the 16-bit counters: filtered 16-bit rows, and fp32 rows in 1024-thread
    // blocks (their coarse histogram and bucket list take less; see
    // coarse_hist32)
    static_assert(mi::coarse_lds_bytes() <= mi::sample_fine_bytes(1024), "the fp32 cut's LDS fits the 16-bit search's");
    const bool fine_lds = may_filter && nseg == 1 && (fine || threads == 1024);
    const size_t lds = fine_lds ? std::max(mi::sample_fine_bytes(threads), mi::sample_hist_bytes(threads))
                                : (may_filter ? mi::sample_hist_bytes(threads) : 0);
    const mi::SplitInfo* sinfo = nullptr;
    if (split_filtered && nseg > 1) {
      // the histogram pass: segments of a multiple of 256 tokens, fewer than
      // 65536, about kSplitHistBlocks blocks in all
      int64_t hseg = std::min<int64_t>({std::max<int64_t>(kSplitHistBlocks / n, 1), kMaxHistSegments, (V + 4095) / 4096});
      hseg = std::max<int64_t>(hseg, (V + kSplitHistMaxSeg - 1) / kSplitHistMaxSeg);
      const int64_t hlen = ((V + hseg - 1) / hseg + 255) / 256 * 256;
      hseg = (V + hlen - 1) / hlen;
      uint32_t* hist = static_cast<uint32_t*>(workspace);
      uint32_t* map = hist + static_cast<int64_t>(n) * mi::kSplitHistWords;
      mi::SplitInfo* info = reinterpret_cast<mi::SplitInfo*>(map + static_cast<int64_t>(n) * mi::kSplitMapWords);
      const int64_t n16 = static_cast<int64_t>(n) * (mi::kSplitHistWords + mi::kSplitMapWords) / 4;
      mi::split_clear<<<static_cast<uint32_t>((n16 + 255) / 256), 256, 0, stream>>>(reinterpret_cast<uint4*>(hist), n16,
                                                                                   tokens + r0, n);
      const uint32_t hblocks = static_cast<uint32_t>(n * hseg);
      if (dtype == MI_DTYPE_F16) {
        mi::split_hist<mi::F16Bits><<<hblocks, 1024, mi::sample_fine_bytes(1024), stream>>>(
            reinterpret_cast<const uint16_t*>(lg), logits_row_stride, mk, mask_row_stride, V, ar,
            static_cast<int32_t>(hseg), static_cast<int32_t>(hlen), hist, map);
        mi::split_search<mi::F16Bits><<<n, 1024, 0, stream>>>(ar, hist, map, info);
      } else {
        mi::split_hist<mi::BF16Bits><<<hblocks, 1024, mi::sample_fine_bytes(1024), stream>>>(
            reinterpret_cast<const uint16_t*>(lg), logits_row_stride, mk, mask_row_stride, V, ar,
            static_cast<int32_t>(hseg), static_cast<int32_t>(hlen), hist, map);
        mi::split_search<mi::BF16Bits><<<n, 1024, 0, stream>>>(ar, hist, map, info);
      }
      sinfo = info;
    } else if (nseg > 1) {
      mi::clear_tokens<<<(n + 255) / 256, 256, 0, stream>>>(tokens + r0, n);
    }
    if (greedy_only && !sinfo) {
      // every row greedy: the max pass alone, in its own kernel (greedy_rows),
      // 128 bytes in flight per thread; measured on MI355X (cold, graph
      // replay): one 512-thread block per row for at most 256 rows (B=256
      // bf16 18.1 -> 16.2 us, fp32 28.9 -> 26.4 us against the 1024-thread
      // sample_rows), 128-thread blocks beyond (B=1024 fp16 16.2 -> 15.8 us),
      // 256-thread blocks per segment of a split row
#define MI_GREEDY(TAG, BITS, THREADS)                                                                             \
  mi::greedy_rows<TAG, 128, THREADS><<<static_cast<uint32_t>(n) * nseg, THREADS, 0, stream>>>(                      \
      reinterpret_cast<const BITS*>(lg), logits_row_stride, mk, mask_row_stride, V, tokens + r0, nseg, seg_len)
#define MI_GREEDY_SHAPES(TAG, BITS)                    \
  if (nseg > 1) MI_GREEDY(TAG, BITS, 256);             \
  else if (n <= 256) MI_GREEDY(TAG, BITS, 512);        \
  else MI_GREEDY(TAG, BITS, 128)
      switch (dtype) {
        case MI_DTYPE_F32:
          MI_GREEDY_SHAPES(mi::F32Bits, uint32_t);
          break;
        case MI_DTYPE_F16:
          MI_GREEDY_SHAPES(mi::F16Bits, uint16_t);
          break;
        default:
          MI_GREEDY_SHAPES(mi::BF16Bits, uint16_t);
      }
#undef MI_GREEDY_SHAPES
#undef MI_GREEDY
      if (nseg > 1) mi::finish_tokens<<<(n + 255) / 256, 256, 0, stream>>>(tokens + r0, n);
      continue;
    }
#define MI_SAMPLE(TAG, BITS, BYTES, THREADS, SPLITF, HEAVY)                                                    \
  mi::sample_rows<TAG, BYTES, THREADS, SPLITF, HEAVY><<<static_cast<uint32_t>(n) * nseg, THREADS, lds, stream>>>( \
      reinterpret_cast<const BITS*>(lg), logits_row_stride, mk, mask_row_stride, V, ar, r0, tokens + r0, nseg,     \
      seg_len, sinfo, heavy)
    switch (dtype) {
      case MI_DTYPE_F32:
        if (deep) MI_SAMPLE(mi::F32Bits, uint32_t, 128, 1024, false, false);
        else MI_SAMPLE(mi::F32Bits, uint32_t, 128, 256, false, false);
        break;
      case MI_DTYPE_F16:
        if (sinfo) MI_SAMPLE(mi::F16Bits, uint16_t, 128, 256, true, false);
        else if (fine8 && heavy) MI_SAMPLE(mi::F16Bits, uint16_t, 128, 512, false, true);
        else if (fine8) MI_SAMPLE(mi::F16Bits, uint16_t, 128, 512, false, false);
        else if (deep && heavy) MI_SAMPLE(mi::F16Bits, uint16_t, 128, 1024, false, true);
        else if (deep) MI_SAMPLE(mi::F16Bits, uint16_t, 128, 1024, false, false);
        else MI_SAMPLE(mi::F16Bits, uint16_t, 128, 256, false, false);
        break;
      default:
        if (sinfo) MI_SAMPLE(mi::BF16Bits, uint16_t, 128, 256, true, false);
        else if (fine8 && heavy) MI_SAMPLE(mi::BF16Bits, uint16_t, 128, 512, false, true);
        else if (fine8) MI_SAMPLE(mi::BF16Bits, uint16_t, 128, 512, false, false);
        else if (deep && heavy) MI_SAMPLE(mi::BF16Bits, uint16_t, 128, 1024, false, true);
        else if (deep) MI_SAMPLE(mi::BF16Bits, uint16_t, 128, 1024, false, false);
        else MI_SAMPLE(mi::BF16Bits, uint16_t, 128, 256, false, false);
    }
#undef MI_SAMPLE
    if (nseg > 1) mi::finish_tokens<<<(n + 255) / 256, 256, 0, stream>>>(tokens + r0, n);
  }
  return after_launch("sample_rows");
}

}  // namespace

MI_API mi_status_t mi_apply_bitmask_sample(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                           int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                           int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                           const mi_sample_params_t* params, int64_t* tokens, hipStream_t stream) {
  return sample_impl(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols, mask_row_stride,
                     vocab_size, params, tokens, nullptr, 0, stream);
}

MI_API mi_status_t mi_apply_bitmask_sample_ws(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                              int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                              int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                              const mi_sample_params_t* params, int64_t* tokens, void* workspace,
                                              int64_t workspace_bytes, hipStream_t stream) {
  return sample_impl(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols, mask_row_stride,
                     vocab_size, params, tokens, workspace, workspace_bytes, stream);
}

MI_API mi_status_t mi_apply_bitmask_sample_noalloc(const void* logits, mi_dtype_t dtype, int64_t rows, int64_t cols,
                                                   int64_t logits_row_stride, const int32_t* mask, int64_t mask_rows,
                                                   int64_t mask_cols, int64_t mask_row_stride, int64_t vocab_size,
                                                   const mi_sample_params_t* params, int64_t* tokens,
                                                   hipStream_t stream) {
  return sample_impl(logits, dtype, rows, cols, logits_row_stride, mask, mask_rows, mask_cols, mask_row_stride,
                     vocab_size, params, tokens, nullptr, 0, stream, true);
}

MI_API int64_t mi_sample_workspace_bytes(mi_dtype_t dtype, int64_t rows, int64_t vocab) {
  if (!valid_dtype(static_cast<int>(dtype)) || rows < 0 || vocab < 0 || vocab > kMaxSampleVocab) return 0;
  return workspace_need(dtype, rows, vocab);
}
