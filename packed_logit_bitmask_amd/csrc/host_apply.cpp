// Host-memory apply (declared in host_apply.h).  Compiled as plain host C++.
//
// Two loops, chosen once per process:
//  - AVX-512 (F + BW): a mask word covers 32 tokens; its complement, cut to
//    the tokens below V, is the lane mask of one masked store of the fill
//    (32 16-bit lanes, or two stores of 16 32-bit lanes).  Masked-off lanes
//    are neither read nor written, and they raise no fault, so a word that
//    reaches past the end of a buffer is safe.
//  - portable: for every clear bit, one element store.
#include "host_apply.h"

#include <immintrin.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <thread>

namespace mi_host {
namespace {

// Bits of word w (of W) that name tokens to fill: the clear bits, without
// those at or past V in the last word.
inline uint32_t fill_bits(uint32_t word, int64_t w, int64_t W, uint32_t last) {
  const uint32_t m = ~word;
  return w == W - 1 ? (m & last) : m;
}

inline uint32_t last_word_bits(int64_t V) {
  return (V % 32) ? (1u << (V % 32)) - 1u : 0xFFFFFFFFu;
}

inline int64_t row_of(const int32_t* rows, int64_t i) { return rows ? rows[i] : i; }

template <typename T>
void rows_portable(T* logits, int64_t ls, const uint32_t* mask, int64_t ms, int64_t V, const int32_t* rows,
                   int64_t i0, int64_t i1, T fill) {
  const int64_t W = (V + 31) / 32;
  const uint32_t last = last_word_bits(V);
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t r = row_of(rows, i);
    T* row = logits + r * ls;
    const uint32_t* mrow = mask + r * ms;
    for (int64_t w = 0; w < W; ++w) {
      uint32_t m = fill_bits(mrow[w], w, W, last);
      T* p = row + w * 32;
      while (m) {
        p[__builtin_ctz(m)] = fill;
        m &= m - 1u;
      }
    }
  }
}

__attribute__((target("avx512f,avx512bw"))) void rows_avx512_u16(uint16_t* logits, int64_t ls,
                                                                  const uint32_t* mask, int64_t ms, int64_t V,
                                                                  const int32_t* rows, int64_t i0, int64_t i1,
                                                                  uint16_t fill) {
  const int64_t W = (V + 31) / 32;
  const uint32_t last = last_word_bits(V);
  const __m512i f = _mm512_set1_epi16(static_cast<short>(fill));
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t r = row_of(rows, i);
    uint16_t* row = logits + r * ls;
    const uint32_t* mrow = mask + r * ms;
    for (int64_t w = 0; w < W; ++w) {
      const uint32_t m = fill_bits(mrow[w], w, W, last);
      if (m) _mm512_mask_storeu_epi16(row + w * 32, static_cast<__mmask32>(m), f);
    }
  }
}

__attribute__((target("avx512f"))) void rows_avx512_u32(uint32_t* logits, int64_t ls, const uint32_t* mask,
                                                         int64_t ms, int64_t V, const int32_t* rows, int64_t i0, int64_t i1,
                                                         uint32_t fill) {
  const int64_t W = (V + 31) / 32;
  const uint32_t last = last_word_bits(V);
  const __m512i f = _mm512_set1_epi32(static_cast<int>(fill));
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t r = row_of(rows, i);
    uint32_t* row = logits + r * ls;
    const uint32_t* mrow = mask + r * ms;
    for (int64_t w = 0; w < W; ++w) {
      const uint32_t m = fill_bits(mrow[w], w, W, last);
      if (m & 0xFFFFu) _mm512_mask_storeu_epi32(row + w * 32, static_cast<__mmask16>(m & 0xFFFFu), f);
      if (m >> 16) _mm512_mask_storeu_epi32(row + w * 32 + 16, static_cast<__mmask16>(m >> 16), f);
    }
  }
}

bool use_avx512() {
  static const bool yes = [] {
    const char* env = std::getenv("MI_BITMASK_HOST_ISA");
    if (env && std::strcmp(env, "portable") == 0) return false;
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
  }();
  return yes;
}

constexpr int kMaxThreads = 256;

// fn(a, b) over [0, nrows) in `threads` even parts, one per thread; a part
// whose thread cannot be started runs on the calling thread.
template <typename Fn>
void split_rows(int64_t nrows, int threads, const Fn& fn) noexcept {
  threads = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>({threads, nrows, kMaxThreads})));
  const int64_t per = (nrows + threads - 1) / threads;
  std::thread pool[kMaxThreads];  // default-constructed threads own nothing
  for (int k = 1; k < threads; ++k) {
    const int64_t a = k * per, b = std::min(nrows, a + per);
    if (a >= b) break;
    try {
      pool[k] = std::thread([&fn, a, b] { fn(a, b); });
    } catch (...) {
      fn(a, b);
    }
  }
  fn(int64_t(0), std::min(nrows, per));
  for (auto& t : pool)
    if (t.joinable()) t.join();
}

}  // namespace

void apply_u16(uint16_t* logits, int64_t ls, const uint32_t* mask, int64_t ms, int64_t V, const int32_t* rows,
               int64_t nrows, uint16_t fill, int threads) noexcept {
  const bool wide = use_avx512();
  split_rows(nrows, threads, [=](int64_t a, int64_t b) {
    if (wide) rows_avx512_u16(logits, ls, mask, ms, V, rows, a, b, fill);
    else rows_portable(logits, ls, mask, ms, V, rows, a, b, fill);
  });
}

void apply_u32(uint32_t* logits, int64_t ls, const uint32_t* mask, int64_t ms, int64_t V, const int32_t* rows,
               int64_t nrows, uint32_t fill, int threads) noexcept {
  const bool wide = use_avx512();
  split_rows(nrows, threads, [=](int64_t a, int64_t b) {
    if (wide) rows_avx512_u32(logits, ls, mask, ms, V, rows, a, b, fill);
    else rows_portable(logits, ls, mask, ms, V, rows, a, b, fill);
  });
}

const char* isa() noexcept { return use_avx512() ? "avx512" : "portable"; }

}  // namespace mi_host
