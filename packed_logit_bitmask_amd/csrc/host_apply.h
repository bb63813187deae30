// Host-memory implementation of the packed-bitmask apply, for tensors that
// live on the CPU (XGrammar "Bitmask Operations", Notes: Device -- CPU
// tensors get a CPU implementation).  Bit patterns only, as on the device:
// every token v < V of a listed row whose bit (v % 32 of word v / 32) is
// clear gets the fill; every other element is left untouched.  Defined in
// host_apply.cpp, which is compiled for the host only.
#pragma once

#include <stdint.h>

namespace mi_host {

// Apply to `nrows` rows on up to `threads` threads (>= 1), rows split
// evenly.  Row i is rows[i] when `rows` is given (values already checked),
// else i.  logits: [*, ls] elements; mask: [*, ms] words.  Allocates
// nothing and throws nothing: a worker thread that cannot be started leaves
// its rows to the calling thread.
void apply_u16(uint16_t* logits, int64_t ls, const uint32_t* mask, int64_t ms, int64_t V, const int32_t* rows,
               int64_t nrows, uint16_t fill, int threads) noexcept;
void apply_u32(uint32_t* logits, int64_t ls, const uint32_t* mask, int64_t ms, int64_t V, const int32_t* rows,
               int64_t nrows, uint32_t fill, int threads) noexcept;

// The instruction set the two calls use: "avx512" (one masked store per
// mask word) or "portable" (one store per masked token).  The environment
// variable MI_BITMASK_HOST_ISA=portable selects the portable loop, so it
// can be tested on machines that have AVX-512.
const char* isa() noexcept;

}  // namespace mi_host
