// Device kernels of the packed-bitmask apply, written for gfx950 (CDNA4,
// wave64).
//
// The op is pure data movement: a logit is either kept bit for bit or
// replaced by the fill's bit pattern (XGrammar "Bitmask Operations",
// apply_token_bitmask_inplace; Modular MAX "apply_packed_bitmask").  So every
// kernel works on raw 16- or 32-bit patterns (fp16 and bf16 share the 16-bit
// kernels) and does no floating-point arithmetic at all; the only compute is
// a few integer ops per element to find and test the element's mask bit:
// bit (v % 32) of word v / 32 of the row, set = keep.
//
// Launch shape shared by all kernels: a 1-D grid of (row slot, chunk) blocks
// of 256 threads (four wave64s); block b serves slot slot_base + b / chunks,
// chunk b % chunks of that row.  A slot maps to a row through RowMap (the
// optional index list of XGrammar "Bitmask Operations", Notes: Indices).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi {

constexpr int kBlock = 256;

// Raw buffer resources (CDNA buffer addressing, stride 0).  An access whose
// byte offset is at or past the resource's size is range-checked by the
// hardware: a load returns 0 and a store is dropped.  The vector kernels use
// that as a branch-free predicate -- a skipped vector gets kSkip as its
// offset -- so the compiler emits straight-line code with one wait between
// the loads and the stores.  Every resource here is at most 2^27 bytes.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer, 32-bit data format
constexpr int kSkip = 0x7FFFFFF0;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy bits of a gfx950 vector memory instruction (the `aux`
// operand): SC0 = 1, NT = 2, SC1 = 16.  A store with SC1 set has device
// scope: it is written through the XCD's L2 instead of lying dirty there
// until the end-of-kernel writeback, so a kernel whose output does not fit
// the L2s streams its writes while it runs.  NT marks the data as
// non-temporal (streamed, not kept).
enum StorePolicy : int {
  kStoreWriteBack = 0,          // default: lines stay dirty in L2
  kStoreDevice = 16,            // SC1: write through L2
  kStoreDeviceStream = 16 | 2,  // SC1 + NT: write through, do not keep
};

__device__ __forceinline__ uint32_t load_word(Rsrc r, int32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}
__device__ __forceinline__ uint4 load16(Rsrc r, int32_t byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int POLICY>
__device__ __forceinline__ void store16(Rsrc r, int32_t byte_off, uint4 v) {
  u32x4 d;
  d.x = v.x; d.y = v.y; d.z = v.z; d.w = v.w;
  __builtin_amdgcn_raw_buffer_store_b128(d, r, byte_off, 0, POLICY);
}

// Slot -> row.  Without an index list the slot is the row.  With one, an
// entry outside [0, row_limit) is skipped: the host cannot check device
// memory, so the kernel defines that case as "no write".  An optional
// per-row gate (one byte per row; TensorRT-Edge-LLM "Guided Decoder": the
// apply leaves a row whose flag is zero alone) turns rows off.
struct RowMap {
  const int32_t* indices;
  int64_t row_limit;
  const int8_t* gate = nullptr;

  __device__ __forceinline__ bool row(int64_t slot, int64_t* r) const {
    const int64_t v = indices ? static_cast<int64_t>(indices[slot]) : slot;
    *r = v;
    return v >= 0 && v < row_limit;
  }
  __device__ __forceinline__ bool gated_off(int64_t r) const { return gate && gate[r] == 0; }
};

// Out of place with a short index list, in one pass over every row: a block
// masks its row only when the list holds it (XGrammar "Bitmask Operations",
// Notes: Indices), and copies it otherwise.  Every thread compares its share
// of the list with the row, and a block-wide OR decides; a listed value
// outside [0, row_limit) matches no row, as in the in-place apply.  Called
// by every thread of the block (it holds a barrier).
struct ListedRows {
  const int32_t* indices = nullptr;  // nullptr: no list (the caller's `apply` stands)
  int32_t count = 0;
  int64_t row_limit = 0;

  __device__ __forceinline__ int32_t holds(int64_t r) const {
    bool found = false;
    for (int32_t i = static_cast<int32_t>(threadIdx.x); i < count; i += kBlock)
      found |= static_cast<int64_t>(indices[i]) == r;
    return (__syncthreads_or(found) != 0 && r < row_limit) ? 1 : 0;
  }
};

// Per-row report for the gated apply: 1 when row r still admits one of its
// first V tokens (TensorRT-Edge-LLM "Guided Decoder": rowHasAnyToken; an
// all-zero row is unsatisfiable).  A gated-off row is not masked, so it
// admits a token whenever V > 0.  Called by every thread of one block (it
// ends with a block barrier); one thread writes the byte, so no
// atomics and no prior initialisation are needed.  Bits past V in the last
// word are masked off; words past it are never read.  The apply runs it in
// blocks of their own, one per row, alongside the apply blocks.
__device__ __forceinline__ void report_row(const uint32_t* __restrict__ mrow, int32_t V, int32_t W,
                                           bool gated_off, uint8_t* __restrict__ out_r) {
  constexpr int kBatch = 8;  // loads in flight per thread
  uint32_t acc = 0;
  if (!gated_off) {
    const Rsrc rm = make_rsrc(mrow, static_cast<uint32_t>(W) * 4u);
    const uint32_t tail = (V & 31) ? (1u << (V & 31)) - 1u : 0xFFFFFFFFu;
    const int t = static_cast<int>(threadIdx.x);
    for (int32_t base = 0; base < W; base += kBlock * kBatch) {
      uint32_t w[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) w[k] = load_word(rm, (base + k * kBlock + t) * 4);  // past W: 0
#pragma unroll
      for (int k = 0; k < kBatch; ++k) acc |= (base + k * kBlock + t == W - 1) ? (w[k] & tail) : w[k];
    }
  }
  const int any = __syncthreads_or(acc != 0u);
  if (threadIdx.x == 0) *out_r = gated_off ? static_cast<uint8_t>(V > 0) : static_cast<uint8_t>(any != 0);
}

template <typename T>
struct Bits16B {
  static constexpr int VW = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte vector
  static constexpr uint32_t FULL = (1u << VW) - 1u;
};

// Mask bits of tokens [e, e + VW) of one row, token e in bit 0.  Reads word
// e / 32 and, when the window crosses a word boundary, the next word -- but
// never word W or beyond (the caller forces bits of tokens >= V itself).
template <int VW>
__device__ __forceinline__ uint32_t window_bits(const uint32_t* __restrict__ mrow, int64_t e, int64_t W) {
  const int64_t wi = e >> 5;
  const uint32_t sh = static_cast<uint32_t>(e) & 31u;
  uint32_t b = mrow[wi] >> sh;
  if (sh + VW > 32u && wi + 1 < W) b |= mrow[wi + 1] << (32u - sh);
  return b & ((1u << VW) - 1u);
}

// Per-element select inside one 16-byte vector: element i keeps v's bits
// when bit i of `keep` is set, else takes the fill pattern.
template <typename T>
__device__ __forceinline__ uint4 select16(uint4 v, uint32_t keep, uint32_t fill_word) {
  uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m;  // 1-bits where the fill goes
    if constexpr (sizeof(T) == 2) {
      m = ((keep >> (2 * q)) & 1u ? 0u : 0x0000FFFFu) | ((keep >> (2 * q + 1)) & 1u ? 0u : 0xFFFF0000u);
    } else {
      m = ((keep >> q) & 1u) ? 0u : 0xFFFFFFFFu;
    }
    d[q] = (d[q] & ~m) | (fill_word & m);
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

template <typename T>
__device__ __forceinline__ uint32_t fill_word_of(T fill) {
  if constexpr (sizeof(T) == 2) return static_cast<uint32_t>(fill) | (static_cast<uint32_t>(fill) << 16);
  else return static_cast<uint32_t>(fill);
}

__device__ __forceinline__ bool token_kept(const uint32_t* __restrict__ mrow, int64_t v) {
  return (mrow[v >> 5] >> (static_cast<uint32_t>(v) & 31u)) & 1u;
}

// ---------------------------------------------------------------------------
// In place, one thread per element.  Chunk = 256 threads x 8 elements.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBlock) void inplace_scalar(
    T* __restrict__ logits, int64_t ls, const uint32_t* __restrict__ mask, int64_t ms,
    int32_t V, RowMap map, int64_t slot_base, uint32_t chunks, T fill) {
  const int64_t slot = slot_base + blockIdx.x / chunks;
  const int32_t chunk = static_cast<int32_t>(blockIdx.x % chunks);
  int64_t r;
  if (!map.row(slot, &r) || map.gated_off(r)) return;
  T* __restrict__ row = logits + r * ls;
  const uint32_t* __restrict__ mrow = mask + r * ms;
  const int32_t j0 = chunk * (kBlock * 8) + static_cast<int32_t>(threadIdx.x);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int32_t j = j0 + u * kBlock;
    if (j < V && !token_kept(mrow, j)) row[j] = fill;
  }
}

// ---------------------------------------------------------------------------
// In place, 16-byte vectors.  Each lane owns U vectors spaced one block
// apart, so every wave instruction covers 1 KiB of consecutive logits.
// Per 128-byte line: all kept -> nothing; otherwise every vector is written:
// all masked -> the fill vector, without reading; the others read, selected
// and written (kept elements get their own bits back).  Loads and stores are
// predicated through buffer range checks, not branches.
// The row's elements before the first 16-byte boundary (head) and after the
// last whole vector below V (tail) are done one element at a time by block 0
// of the row, so no store ever covers a column >= V or a byte of another
// row.  When the row start is not 16-byte aligned the mask window of a
// vector can straddle two words; a funnel shift joins them.
// ---------------------------------------------------------------------------
template <typename T, int U, int POLICY>
__global__ __launch_bounds__(kBlock) void inplace_vec(
    T* __restrict__ logits, int64_t ls, const uint32_t* __restrict__ mask, int64_t ms,
    int32_t V, int32_t W, RowMap map, int64_t slot_base, uint32_t chunks, T fill,
    uint8_t* __restrict__ any_out, uint32_t nrep) {
  constexpr int VW = Bits16B<T>::VW;
  constexpr uint32_t FULL = Bits16B<T>::FULL;
  // With a per-row report, the first `nrep` blocks of the grid are report
  // blocks, one per slot; they run beside the apply blocks, not before them.
  if (blockIdx.x < nrep) {
    int64_t rr;
    if (map.row(slot_base + blockIdx.x, &rr)) report_row(mask + rr * ms, V, W, map.gated_off(rr), any_out + rr);
    return;
  }
  const uint32_t b = blockIdx.x - nrep;
  const int64_t slot = slot_base + b / chunks;
  const int32_t chunk = static_cast<int32_t>(b % chunks);
  int64_t r;
  if (!map.row(slot, &r) || map.gated_off(r)) return;
  const uint32_t* __restrict__ mrow = mask + r * ms;
  T* __restrict__ row = logits + r * ls;

  const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row) & 15u);
  int32_t h = static_cast<int32_t>(((16u - mis) & 15u) / sizeof(T));
  if (h > V) h = V;
  const int32_t nvec = (V - h) / VW;
  const int32_t tail0 = h + nvec * VW;
  const int t = static_cast<int>(threadIdx.x);

  if (chunk == 0) {
    int32_t j = -1;
    if (t < h) j = t;
    else if (t >= 64 && t - 64 < V - tail0) j = tail0 + (t - 64);
    if (j >= 0 && !token_kept(mrow, j)) row[j] = fill;
  }

  const int32_t kbase = chunk * (kBlock * U);
  const int32_t nv = min(kBlock * U, nvec - kbase);
  if (nv <= 0) return;
  const Rsrc rl = make_rsrc(row + h + static_cast<int64_t>(kbase) * VW, static_cast<uint32_t>(nv) * 16u);
  const Rsrc rm = make_rsrc(mrow, static_cast<uint32_t>(W) * 4u);

  uint32_t lo[U], hi[U], keep[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t e = h + (kbase + u * kBlock + t) * VW;   // first token of the vector
    lo[u] = load_word(rm, (e >> 5) * 4);
    hi[u] = load_word(rm, h ? ((e >> 5) + 1) * 4 : kSkip);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t e = h + (kbase + u * kBlock + t) * VW;
    // lanes past the chunk's last vector count as all kept (nothing to write)
    const uint32_t past = u * kBlock + t < nv ? 0u : FULL;
    keep[u] = (__builtin_amdgcn_alignbit(hi[u], lo[u], static_cast<uint32_t>(e) & 31u) & FULL) | past;
  }
  // Line-complete writes: the (up to) 8 lanes whose vectors share a 128-byte
  // line decide together.  If any vector of the line needs a store, every
  // vector of the line is stored -- all-kept ones written back with their own
  // bits -- so the line leaves the L2 whole; a partly written line would cost
  // a read-modify-write at the memory side.  A vector is read unless it is
  // all masked (its line is being read anyway when a neighbour is).
  const int lane = t & 63;
  const int line_pos = static_cast<int>(((reinterpret_cast<uintptr_t>(row + h) >> 4) + kbase + t) & 7u);
  const int first = lane - line_pos;                      // lane holding the line's first vector
  const uint64_t line_lanes = first >= 0 ? (uint64_t(0xFF) << first) : (uint64_t(0xFF) >> -first);
  bool write[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t needs = __builtin_amdgcn_ballot_w64(keep[u] != FULL);
    write[u] = (needs & line_lanes) != 0;
  }
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    v[u] = load16(rl, (write[u] && keep[u] != 0u) ? (u * kBlock + t) * 16 : kSkip);
  const uint32_t fw = fill_word_of(fill);
#pragma unroll
  for (int u = 0; u < U; ++u)
    store16<POLICY>(rl, write[u] ? (u * kBlock + t) * 16 : kSkip, select16<T>(v[u], keep[u], fw));
}

// ---------------------------------------------------------------------------
// In place, write-only.  One lane per element: each wave takes 64 mask words
// (2048 tokens) with one coalesced load, then for each 64-token group reads
// its two words as wave-uniform values, skips the group when both are all
// ones, and otherwise stores the fill under the lane's bit.  Logits are
// never read, and alignment does not matter (element stores).
// Chunk = 4 waves x 64 words = 8192 tokens.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBlock) void inplace_wronly(
    T* __restrict__ logits, int64_t ls, const uint32_t* __restrict__ mask, int64_t ms,
    int32_t V, int32_t W, RowMap map, int64_t slot_base, uint32_t chunks, T fill) {
  const int64_t slot = slot_base + blockIdx.x / chunks;
  const int32_t chunk = static_cast<int32_t>(blockIdx.x % chunks);
  int64_t r;
  if (!map.row(slot, &r) || map.gated_off(r)) return;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int wave = static_cast<int>(threadIdx.x) >> 6;
  const int32_t wbase = chunk * 256 + wave * 64;
  if (wbase >= W) return;
  const uint32_t* __restrict__ mrow = mask + r * ms;
  const uint32_t mw = (wbase + lane < W) ? mrow[wbase + lane] : 0xFFFFFFFFu;
  T* __restrict__ p = logits + r * ls + static_cast<int64_t>(wbase) * 32;
  const int32_t nel = V - wbase * 32;
  const uint32_t sel = static_cast<uint32_t>(lane) & 31u;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const uint32_t lo = __builtin_amdgcn_readlane(mw, 2 * u);
    const uint32_t hi = __builtin_amdgcn_readlane(mw, 2 * u + 1);
    if ((lo & hi) != 0xFFFFFFFFu) {
      const uint32_t w = lane < 32 ? lo : hi;
      const int32_t e = u * 64 + lane;
      if (e < nel && !((w >> sel) & 1u)) p[e] = fill;
    }
  }
}

// ---------------------------------------------------------------------------
// Out of place, one thread per element, every row:  out = in where kept,
// fill where masked (only when `apply` is set and v < V), plain copy
// elsewhere.  Chunk = 256 threads x 8 elements over [0, cols).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBlock) void out_scalar(
    T* __restrict__ out, int64_t os, const T* __restrict__ in, int64_t ls,
    const uint32_t* __restrict__ mask, int64_t ms, int32_t V, int32_t cols, int32_t apply,
    ListedRows listed, int64_t slot_base, uint32_t chunks, T fill) {
  const int64_t r = slot_base + blockIdx.x / chunks;
  const int32_t chunk = static_cast<int32_t>(blockIdx.x % chunks);
  if (listed.indices) apply = listed.holds(r);
  T* __restrict__ orow = out + r * os;
  const T* __restrict__ irow = in + r * ls;
  const uint32_t* __restrict__ mrow = mask + r * ms;
  const int32_t j0 = chunk * (kBlock * 8) + static_cast<int32_t>(threadIdx.x);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int32_t j = j0 + u * kBlock;
    if (j < cols) {
      const bool masked = apply && j < V && !token_kept(mrow, j);
      orow[j] = masked ? fill : irow[j];
    }
  }
}

// ---------------------------------------------------------------------------
// Out of place, 16-byte vectors, every row, one fused pass over [0, cols).
// Needs out and in rows at the same offset modulo 16 bytes (the host checks).
// Per vector: all masked -> store the fill vector without reading the input;
// otherwise read, select (tokens >= V, and every token when `apply` is 0,
// count as kept), write.  Head and tail elements go one at a time.
// ---------------------------------------------------------------------------
template <typename T, int U, int POLICY>
__global__ __launch_bounds__(kBlock) void out_vec(
    T* __restrict__ out, int64_t os, const T* __restrict__ in, int64_t ls,
    const uint32_t* __restrict__ mask, int64_t ms, int32_t V, int32_t W, int32_t cols,
    int32_t apply, ListedRows listed, int64_t slot_base, uint32_t chunks, T fill) {
  constexpr int VW = Bits16B<T>::VW;
  constexpr uint32_t FULL = Bits16B<T>::FULL;
  const int64_t r = slot_base + blockIdx.x / chunks;
  const int32_t chunk = static_cast<int32_t>(blockIdx.x % chunks);
  if (listed.indices) apply = listed.holds(r);
  T* __restrict__ orow = out + r * os;
  const T* __restrict__ irow = in + r * ls;
  const uint32_t* __restrict__ mrow = mask + r * ms;

  const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(orow) & 15u);
  int32_t h = static_cast<int32_t>(((16u - mis) & 15u) / sizeof(T));
  if (h > cols) h = cols;
  const int32_t nvec = (cols - h) / VW;
  const int32_t tail0 = h + nvec * VW;
  const int t = static_cast<int>(threadIdx.x);

  if (chunk == 0) {
    int32_t j = -1;
    if (t < h) j = t;
    else if (t >= 64 && t - 64 < cols - tail0) j = tail0 + (t - 64);
    if (j >= 0) {
      const bool masked = apply && j < V && !token_kept(mrow, j);
      orow[j] = masked ? fill : irow[j];
    }
  }

  const int32_t kbase = chunk * (kBlock * U);
  const int32_t nv = min(kBlock * U, nvec - kbase);
  if (nv <= 0) return;
  const int64_t off0 = h + static_cast<int64_t>(kbase) * VW;
  const Rsrc ro = make_rsrc(orow + off0, static_cast<uint32_t>(nv) * 16u);
  const Rsrc ri = make_rsrc(irow + off0, static_cast<uint32_t>(nv) * 16u);
  const Rsrc rm = make_rsrc(mrow, static_cast<uint32_t>(W) * 4u);
  const int32_t Va = apply ? V : 0;   // tokens below Va are masked by their bit

  uint32_t keep[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t e = h + (kbase + u * kBlock + t) * VW;
    const bool any = e < Va;
    const uint32_t lo = load_word(rm, any ? (e >> 5) * 4 : kSkip);
    const uint32_t hi = (h && any) ? load_word(rm, ((e >> 5) + 1) * 4) : 0u;
    uint32_t b = __builtin_amdgcn_alignbit(hi, lo, static_cast<uint32_t>(e) & 31u) & FULL;
    const int32_t left = Va - e;  // tokens of this vector below Va
    if (left < VW) b |= FULL & ~((1u << (left > 0 ? left : 0)) - 1u);
    keep[u] = b;
  }
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = load16(ri, keep[u] != 0u ? (u * kBlock + t) * 16 : kSkip);
  const uint32_t fw = fill_word_of(fill);
#pragma unroll
  for (int u = 0; u < U; ++u) store16<POLICY>(ro, (u * kBlock + t) * 16, select16<T>(v[u], keep[u], fw));
}

}  // namespace mi
