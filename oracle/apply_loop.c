/*
 * CPU oracle, compiled part: the literal double loop of the packed-bitmask
 * apply, on raw bit patterns.  TEST INFRASTRUCTURE -- only the tests, the
 * smoke check and the bench's CPU-baseline leg load this; the product never
 * does.
 *
 * What it follows:
 *   XGrammar "Bitmask Operations", apply_token_bitmask_inplace: for every row
 *   b of the processed row set and every token j below the vocab size, if the
 *   j-th bit of row b of the bitmask is 0, logits[b, j] becomes the fill
 *   (-inf there).  The same page's Indices note gives the row set as the index
 *   list when one is given.
 *   Modular MAX "apply_packed_bitmask": bit j % 32 of word j // 32 of the row,
 *   a set bit keeps the token, otherwise the caller's fill value is written.
 *
 * The words are int32 on the pages only because old PyTorch lacked uint32
 * (XGrammar "Bitmask Operations", allocate_token_bitmask); they are read as
 * uint32 here.  Logits are never interpreted as numbers: a masked entry gets
 * the fill's bit pattern, a kept one is not touched.
 *
 * No blocking, no vector tricks, no threads: one plain loop per definition.
 */
#include <stdint.h>

void oracle_apply_u32(uint32_t *logits, int64_t logits_row_stride,
                      const int32_t *mask, int64_t mask_row_stride,
                      int64_t vocab_size, const int64_t *rowset, int64_t n_rows,
                      uint32_t fill_bits)
{
    for (int64_t k = 0; k < n_rows; ++k) {
        int64_t b = rowset[k];
        for (int64_t j = 0; j < vocab_size; ++j) {
            uint32_t word = (uint32_t)mask[b * mask_row_stride + j / 32];
            if (((word >> (j % 32)) & 1u) == 0u)
                logits[b * logits_row_stride + j] = fill_bits;
        }
    }
}

void oracle_apply_u16(uint16_t *logits, int64_t logits_row_stride,
                      const int32_t *mask, int64_t mask_row_stride,
                      int64_t vocab_size, const int64_t *rowset, int64_t n_rows,
                      uint16_t fill_bits)
{
    for (int64_t k = 0; k < n_rows; ++k) {
        int64_t b = rowset[k];
        for (int64_t j = 0; j < vocab_size; ++j) {
            uint32_t word = (uint32_t)mask[b * mask_row_stride + j / 32];
            if (((word >> (j % 32)) & 1u) == 0u)
                logits[b * logits_row_stride + j] = fill_bits;
        }
    }
}

/*
 * Whether row r's mask admits at least one token below the vocab size
 * (TensorRT-Edge-LLM "Guided Decoder": a row whose mask admits no token is
 * unsatisfiable; rowHasAnyToken).  The same bit test as above, token by
 * token, stopping at the first allowed one.
 */
void oracle_rows_any_allowed(const int32_t *mask, int64_t mask_row_stride, int64_t vocab_size,
                             int64_t rows, uint8_t *out)
{
    for (int64_t b = 0; b < rows; ++b) {
        uint8_t any = 0;
        for (int64_t j = 0; j < vocab_size; ++j) {
            uint32_t word = (uint32_t)mask[b * mask_row_stride + j / 32];
            if ((word >> (j % 32)) & 1u) {
                any = 1;
                break;
            }
        }
        out[b] = any;
    }
}
