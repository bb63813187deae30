// Host-memory implementation of the packed-bitmask apply, for tensors that
// live on the CPU (XGrammar "Bitmask Operations", Notes: Device -- CPU
// tensors get a CPU implementation).  Rows are split over std::threads; each
// row walks its mask words and writes the fill at every clear bit below V.
// Bit patterns only, as on the device.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <thread>
#include <vector>

namespace mi_host {

template <typename T>
void apply_rows(T* logits, int64_t ls, const uint32_t* mask, int64_t ms, int64_t V, const int64_t* rows,
                int64_t nrows, T fill) {
  const int64_t W = (V + 31) / 32;
  const uint32_t tail = static_cast<uint32_t>(V % 32);
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t r = rows[i];
    T* row = logits + r * ls;
    const uint32_t* mrow = mask + r * ms;
    for (int64_t w = 0; w < W; ++w) {
      uint32_t masked = ~mrow[w];                       // 1 = token to fill
      if (w == W - 1 && tail) masked &= (1u << tail) - 1u;  // bits past V are not used
      T* p = row + w * 32;
      while (masked) {
        const int b = __builtin_ctz(masked);
        p[b] = fill;
        masked &= masked - 1u;
      }
    }
  }
}

// Run apply_rows over `nrows` rows on up to `threads` threads (>= 1).
template <typename T>
void apply_parallel(T* logits, int64_t ls, const uint32_t* mask, int64_t ms, int64_t V, const int64_t* rows,
                    int64_t nrows, T fill, int threads) {
  threads = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(threads, nrows)));
  if (threads == 1) {
    apply_rows(logits, ls, mask, ms, V, rows, nrows, fill);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t per = (nrows + threads - 1) / threads;
  for (int k = 0; k < threads; ++k) {
    const int64_t a = k * per, b = std::min(nrows, a + per);
    if (a >= b) break;
    pool.emplace_back([=] { apply_rows(logits, ls, mask, ms, V, rows + a, b - a, fill); });
  }
  for (auto& t : pool) t.join();
}

}  // namespace mi_host
