// Host-side code of the library under the sanitizers (built by
// tests/test_sanitize_host.py with -fsanitize=address,undefined and, in a
// second build, -fsanitize=thread).  TEST INFRASTRUCTURE.
//
// It compiles the host entry points and helpers (mi_host.hip, with the
// argument checks and fill rounding of host_checks.h) into this file, links
// host_apply.cpp (the AVX-512 and portable loops and their thread split) and
// the oracle's C loop (oracle/apply_loop.c), and drives them:
//   - every rejection the host entry points make (NULL pointers, dtypes,
//     negative and oversized shapes, pitches, vocab sizes, misalignment,
//     overlapping buffers, bad index values), each with its status code;
//   - the fill conversion over doubles of every exponent, the special values
//     and the rounding midpoints;
//   - in-place and out-of-place applies over both element sizes, ragged
//     vocab tails, padded pitches, index lists, V = 0, empty buffers and 1 to
//     17 threads, each compared with the oracle's loop on the same inputs.
// Any sanitizer report aborts the run (-fno-sanitize-recover); a wrong result
// or status exits with code 1 and names the case.
#include "mi_host.hip"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
void oracle_apply_u32(uint32_t* logits, int64_t logits_row_stride, const int32_t* mask, int64_t mask_row_stride,
                      int64_t vocab_size, const int64_t* rowset, int64_t n_rows, uint32_t fill_bits);
void oracle_apply_u16(uint16_t* logits, int64_t logits_row_stride, const int32_t* mask, int64_t mask_row_stride,
                      int64_t vocab_size, const int64_t* rowset, int64_t n_rows, uint16_t fill_bits);
}

namespace {

int g_failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s (%s)\n", what, mi_last_error_message());
    ++g_failures;
  }
}

void expect_status(mi_status_t got, mi_status_t want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL: %s: status %s, want %s (%s)\n", what, mi_status_string(got), mi_status_string(want),
                 mi_last_error_message());
    ++g_failures;
  }
}

// Every argument check of the host entry points, one per call.
void rejections() {
  std::vector<uint16_t> logits(4 * 70);
  std::vector<int32_t> mask(4 * 3, -1);
  std::vector<int32_t> idx = {0, 3, 1};
  std::vector<uint16_t> out(4 * 70);
  void* L = logits.data();
  const int32_t* M = mask.data();
  const auto inplace = [&](void* l, int dtype, int64_t rows, int64_t cols, int64_t ls, const int32_t* m,
                           int64_t mrows, int64_t mcols, int64_t ms, int64_t vocab, const int32_t* ind, int64_t n) {
    return mi_apply_bitmask_inplace_host(l, static_cast<mi_dtype_t>(dtype), rows, cols, ls, m, mrows, mcols, ms, vocab,
                                         ind, n, -INFINITY, 2);
  };
  expect_status(inplace(nullptr, 2, 4, 70, 70, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_NULL_POINTER, "NULL logits");
  expect_status(inplace(L, 2, 4, 70, 70, nullptr, 4, 3, 3, -1, nullptr, 0), MI_ERR_NULL_POINTER, "NULL mask");
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, -1, nullptr, 2), MI_ERR_NULL_POINTER, "NULL indices, n > 0");
  expect_status(inplace(L, 7, 4, 70, 70, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_DTYPE, "dtype 7");
  expect_status(inplace(L, -1, 4, 70, 70, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_DTYPE, "dtype -1");
  expect_status(inplace(L, 2, -1, 70, 70, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_SHAPE, "negative rows");
  expect_status(inplace(L, 2, 4, -5, 70, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_SHAPE, "negative cols");
  expect_status(inplace(L, 2, 4, 70, 69, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_SHAPE, "pitch below cols");
  expect_status(inplace(L, 2, 4, 70, int64_t(1) << 41, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_SHAPE, "huge pitch");
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 2, -1, nullptr, 0), MI_ERR_BAD_SHAPE, "mask pitch below width");
  expect_status(inplace(L, 2, 4, int64_t(1) << 31, int64_t(1) << 31, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_SHAPE,
                "cols above 2^30");
  expect_status(inplace(L, 2, int64_t(1) << 32, 70, 70, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_SHAPE,
                "rows above 2^31");
  expect_status(inplace(L, 2, 5, 70, 70, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_BAD_SHAPE, "mask rows below rows");
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, 97, nullptr, 0), MI_ERR_BAD_VOCAB, "vocab above 32 * mask_cols");
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, 71, nullptr, 0), MI_ERR_BAD_VOCAB, "vocab above cols");
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, -2, nullptr, 0), MI_ERR_BAD_VOCAB, "vocab -2");
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, -1, idx.data(), -1), MI_ERR_BAD_INDICES, "negative count");
  expect_status(inplace(static_cast<char*>(L) + 1, 2, 4, 60, 60, M, 4, 3, 3, -1, nullptr, 0), MI_ERR_MISALIGNED,
                "odd logits address");
  expect_status(inplace(L, 0, 4, 30, 30, reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(M) + 2), 4,
                        1, 1, -1, nullptr, 0),
                MI_ERR_MISALIGNED, "misaligned mask");
  expect_status(inplace(L, 2, 4, 70, 70, reinterpret_cast<const int32_t*>(logits.data() + 8), 4, 3, 3, -1, nullptr,
                        0),
                MI_ERR_ALIAS, "mask inside logits");
  // index values: the host can read them
  std::vector<int32_t> bad = {0, 4};
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, -1, bad.data(), 2), MI_ERR_BAD_INDICES, "index = rows");
  bad = {-1};
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, -1, bad.data(), 1), MI_ERR_BAD_INDICES, "index -1");
  bad = {2};
  expect_status(inplace(L, 2, 4, 70, 70, M, 2, 3, 3, -1, bad.data(), 1), MI_ERR_BAD_INDICES, "index = mask rows");
  // out of place
  const auto outp = [&](void* o, int64_t os, const void* l) {
    return mi_apply_bitmask_out_host(o, os, l, MI_DTYPE_BF16, 4, 70, 70, M, 4, 3, 3, -1, nullptr, 0, -1.0, 3);
  };
  expect_status(outp(nullptr, 70, L), MI_ERR_NULL_POINTER, "NULL out");
  expect_status(outp(out.data(), 69, L), MI_ERR_BAD_SHAPE, "out pitch below cols");
  expect_status(outp(reinterpret_cast<char*>(out.data()) + 1, 70, L), MI_ERR_MISALIGNED, "odd out address");
  expect_status(outp(logits.data() + 10, 70, L), MI_ERR_ALIAS, "out overlaps logits");
  expect_status(outp(out.data(), 70, L), MI_OK, "out of place");
  expect_status(outp(L, 70, L), MI_OK, "out == logits is in place");
  // empty buffers: NULL allowed
  expect_status(inplace(nullptr, 2, 0, 70, 70, nullptr, 0, 3, 3, -1, nullptr, 0), MI_OK, "zero rows, NULL");
  expect_status(inplace(L, 2, 4, 70, 70, M, 4, 3, 3, 0, nullptr, 0), MI_OK, "V = 0");
  // helpers
  int64_t v = 0;
  expect_status(mi_resolve_vocab_size(50257, 1571, -1, &v), MI_OK, "default vocab");
  expect(v == 50257, "default vocab value");
  expect_status(mi_resolve_vocab_size(100, 3, -1, &v), MI_OK, "vocab limited by the mask");
  expect(v == 96, "vocab limited by the mask value");
  expect_status(mi_resolve_vocab_size(100, 3, -1, nullptr), MI_ERR_NULL_POINTER, "NULL vocab out");
  uint32_t bits = 0;
  expect_status(mi_fill_value_bits(0.0, static_cast<mi_dtype_t>(9), &bits), MI_ERR_BAD_DTYPE, "fill dtype");
  expect_status(mi_fill_value_bits(0.0, MI_DTYPE_F16, nullptr), MI_ERR_NULL_POINTER, "NULL fill out");
  for (int s = -1; s < 12; ++s) expect(std::strlen(mi_status_string(static_cast<mi_status_t>(s))) > 0, "status text");
}

// The fill conversion over every exponent of the double and the values
// around each target's limits; values only checked where a library does the
// same rounding (binary32 by the C cast), the rest for sanitizer reports.
void fills() {
  std::mt19937_64 rng(5);
  const double specials[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, -NAN, 65504.0, 65520.0, 65519.99, -65504.0,
                             5.960464477539063e-08, 2.9802322387695312e-08, 2.98023223876953125e-08,
                             3.4028234663852886e+38, 3.4028235677973366e+38, 1e-45, 1.4e-45, 7e-46, 1e-320,
                             -1e-320, 1.1754942e-38, 3.0e38, 3.3895313892515355e+38, 3.3961775292304957e+38};
  for (double x : specials)
    for (int d = 0; d < 3; ++d) {
      uint32_t b = 0;
      expect_status(mi_fill_value_bits(x, static_cast<mi_dtype_t>(d), &b), MI_OK, "fill special");
    }
  for (int i = 0; i < 200000; ++i) {
    uint64_t u = rng();
    double x;
    std::memcpy(&x, &u, sizeof x);
    uint32_t b32 = 0, b16 = 0, bb = 0;
    mi_fill_value_bits(x, MI_DTYPE_F32, &b32);
    mi_fill_value_bits(x, MI_DTYPE_F16, &b16);
    mi_fill_value_bits(x, MI_DTYPE_BF16, &bb);
    if (std::fabs(x) < 3.4e38) {  // in binary32's range: the cast rounds to nearest even, as the FPU does
      const float f = static_cast<float>(x);
      uint32_t want;
      std::memcpy(&want, &f, sizeof want);
      if (b32 != want) {
        std::fprintf(stderr, "FAIL: fp32 fill of %a: %08x, want %08x\n", x, b32, want);
        ++g_failures;
        return;
      }
    }
  }
}

template <typename T>
void apply_case(std::mt19937_64& rng, int rows, int cols, int pad, int mask_rows, int mask_cols, int64_t vocab,
                bool with_indices, bool out_of_place, int threads) {
  const int64_t ls = cols + pad, ms = mask_cols + 1;
  std::vector<T> logits(static_cast<size_t>(rows) * ls + 3), want, got;
  for (auto& e : logits) e = static_cast<T>(rng());
  std::vector<int32_t> mask(static_cast<size_t>(mask_rows) * ms);
  for (auto& w : mask) w = static_cast<int32_t>(rng());
  std::vector<int32_t> idx;
  std::vector<int64_t> rowset;
  const int limit = std::min(rows, mask_rows);
  if (with_indices) {
    for (int r = 0; r < limit; ++r)
      if (rng() % 3) idx.push_back(r);
    for (size_t i = idx.size(); i > 1; --i) std::swap(idx[i - 1], idx[rng() % i]);
    for (int32_t r : idx) rowset.push_back(r);
  } else {
    for (int r = 0; r < rows; ++r) rowset.push_back(r);
  }
  int64_t V = 0;
  mi_resolve_vocab_size(cols, mask_cols, vocab, &V);
  const mi_dtype_t dt = sizeof(T) == 4 ? MI_DTYPE_F32 : MI_DTYPE_BF16;
  uint32_t fb = 0;
  mi_fill_value_bits(-7.5, dt, &fb);
  want = logits;
  if (sizeof(T) == 4)
    oracle_apply_u32(reinterpret_cast<uint32_t*>(want.data()), ls, mask.data(), ms, V, rowset.data(),
                     static_cast<int64_t>(rowset.size()), fb);
  else
    oracle_apply_u16(reinterpret_cast<uint16_t*>(want.data()), ls, mask.data(), ms, V, rowset.data(),
                     static_cast<int64_t>(rowset.size()), static_cast<uint16_t>(fb));
  const int32_t* ip = with_indices ? (idx.empty() ? reinterpret_cast<const int32_t*>(mask.data()) : idx.data()) : nullptr;
  mi_status_t st;
  if (out_of_place) {
    got.assign(logits.size(), static_cast<T>(0x5A5A5A5A));
    st = mi_apply_bitmask_out_host(got.data(), ls, logits.data(), dt, rows, cols, ls, mask.data(), mask_rows,
                                   mask_cols, ms, vocab, ip, static_cast<int64_t>(idx.size()), -7.5, threads);
    // the output's window is compared; the slack after the last row is not part of it
    for (size_t i = static_cast<size_t>(rows) * ls; i < got.size(); ++i) got[i] = want[i];
    for (int r = 0; r < rows; ++r)
      for (int64_t c = cols; c < ls; ++c) got[r * ls + c] = want[r * ls + c];
  } else {
    got = logits;
    st = mi_apply_bitmask_inplace_host(got.data(), dt, rows, cols, ls, mask.data(), mask_rows, mask_cols, ms, vocab,
                                       ip, static_cast<int64_t>(idx.size()), -7.5, threads);
  }
  char what[160];
  std::snprintf(what, sizeof what, "%s %dx%d pad %d mask %dx%d V %lld idx %d threads %d", sizeof(T) == 4 ? "u32" : "u16",
                rows, cols, pad, mask_rows, mask_cols, static_cast<long long>(vocab), with_indices ? 1 : 0, threads);
  expect_status(st, MI_OK, what);
  expect(got == want, what);
}

void applies() {
  std::mt19937_64 rng(11);
  const int shapes[][5] = {{1, 1, 0, 1, 1}, {3, 31, 1, 3, 1}, {4, 33, 0, 5, 2}, {7, 100, 3, 7, 4},
                           {5, 1000, 0, 5, 32}, {9, 2049, 5, 10, 70}, {2, 65, 0, 2, 3}};
  for (auto& s : shapes)
    for (int64_t vocab : {int64_t(-1), int64_t(0), int64_t(s[1] / 2)})
      for (int ind = 0; ind < 2; ++ind)
        for (int oop = 0; oop < 2; ++oop) {
          apply_case<uint16_t>(rng, s[0], s[1], s[2], s[3], s[4], vocab, ind, oop, 2);
          apply_case<uint32_t>(rng, s[0], s[1], s[2], s[3], s[4], vocab, ind, oop, 3);
        }
  // large enough (>= 2^20 elements) for the thread split
  for (int threads : {1, 4, 17}) {
    apply_case<uint16_t>(rng, 40, 40001, 7, 40, 1251, -1, threads == 4, threads == 17, threads);
    apply_case<uint32_t>(rng, 33, 32770, 0, 35, 1025, 32769, threads == 1, false, threads);
  }
}

}  // namespace

int main() {
  std::printf("host loop: %s\n", mi_host_isa());
  rejections();
  fills();
  applies();
  if (g_failures) {
    std::fprintf(stderr, "%d failures\n", g_failures);
    return 1;
  }
  std::printf("sanitized host checks: ok\n");
  return 0;
}
