// pack.h -- host packers between canonical arrays and packed row records.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fmoe {

// Returns false if a code does not fit in `bits` bits.
bool pack_row(int bits, int cols, const uint8_t *codes, const uint16_t *scale, const uint16_t *bias,
              uint8_t *rec);
void unpack_row(int bits, int cols, const uint8_t *rec, uint8_t *codes, uint16_t *scale, uint16_t *bias);

// Record r of the matrix sits at blob + rec_offset + r * rec_stride.
bool pack_matrix(int bits, int rows, int cols, const uint8_t *codes, const uint16_t *scale,
                 const uint16_t *bias, uint8_t *blob, size_t rec_stride, size_t rec_offset);
void unpack_matrix(int bits, int rows, int cols, const uint8_t *blob, size_t rec_stride, size_t rec_offset,
                   uint8_t *codes, uint16_t *scale, uint16_t *bias);

}  // namespace fmoe
