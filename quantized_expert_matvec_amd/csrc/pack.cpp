// pack.cpp -- host conversion between the canonical layout (one uint8 code per
// weight, bf16 scale and bias per (row, group)) and the library's packed row
// records (layout.h). Pure C++; no device code.
#include <string.h>

#include "layout.h"
#include "pack.h"

namespace fmoe {

static inline void put32(uint8_t *p, uint32_t v) { memcpy(p, &v, 4); }
static inline uint32_t get32(const uint8_t *p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}

// One row record from canonical codes (cols) and per-group scale/bias (cols/64).
bool pack_row(int bits, int cols, const uint8_t *codes, const uint16_t *scale, const uint16_t *bias,
              uint8_t *rec) {
  const int ng = cols / kGroup;
  const uint8_t lim = (uint8_t)(1u << bits);
  for (int c = 0; c < cols; ++c)
    if (codes[c] >= lim) return false;
  if (bits == 4) {
    for (int g = 0; g < ng; ++g)
      for (int h = 0; h < 2; ++h)
        for (int w = 0; w < 4; ++w) {
          uint32_t word = 0;
          for (int k = 0; k < 4; ++k) {
            const int c = kGroup * g + 32 * h + 8 * w + k;
            const uint32_t byte = (uint32_t)codes[c] | ((uint32_t)codes[c + 4] << 4);
            word |= byte << (8 * k);
          }
          put32(rec + (size_t)h * ng * 16 + (size_t)g * 16 + 4 * w, word);
        }
  } else {
    for (int g = 0; g < ng; ++g)
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
        for (int k = 0; k < 4; ++k) {
          uint32_t byte = 0;
          for (int q = 0; q < 4; ++q) byte |= (uint32_t)codes[kGroup * g + 16 * w + 4 * q + k] << (2 * q);
          word |= byte << (8 * k);
        }
        put32(rec + (size_t)g * 16 + 4 * w, word);
      }
  }
  uint8_t *sb = rec + (size_t)ng * code_bytes(bits);
  for (int g = 0; g < ng; ++g) put32(sb + 4 * g, ((uint32_t)scale[g] << 16) | bias[g]);
  return true;
}

void unpack_row(int bits, int cols, const uint8_t *rec, uint8_t *codes, uint16_t *scale, uint16_t *bias) {
  const int ng = cols / kGroup;
  if (bits == 4) {
    for (int g = 0; g < ng; ++g)
      for (int h = 0; h < 2; ++h)
        for (int w = 0; w < 4; ++w) {
          const uint32_t word = get32(rec + (size_t)h * ng * 16 + (size_t)g * 16 + 4 * w);
          for (int k = 0; k < 4; ++k) {
            const int c = kGroup * g + 32 * h + 8 * w + k;
            const uint32_t byte = (word >> (8 * k)) & 0xFFu;
            codes[c] = (uint8_t)(byte & 15u);
            codes[c + 4] = (uint8_t)(byte >> 4);
          }
        }
  } else {
    for (int g = 0; g < ng; ++g)
      for (int w = 0; w < 4; ++w) {
        const uint32_t word = get32(rec + (size_t)g * 16 + 4 * w);
        for (int k = 0; k < 4; ++k) {
          const uint32_t byte = (word >> (8 * k)) & 0xFFu;
          for (int q = 0; q < 4; ++q) codes[kGroup * g + 16 * w + 4 * q + k] = (uint8_t)((byte >> (2 * q)) & 3u);
        }
      }
  }
  const uint8_t *sb = rec + (size_t)ng * code_bytes(bits);
  for (int g = 0; g < ng; ++g) {
    const uint32_t v = get32(sb + 4 * g);
    scale[g] = (uint16_t)(v >> 16);
    bias[g] = (uint16_t)(v & 0xFFFFu);
  }
}

bool pack_matrix(int bits, int rows, int cols, const uint8_t *codes, const uint16_t *scale,
                 const uint16_t *bias, uint8_t *blob, size_t first_rec_stride, size_t rec_offset) {
  // record r goes to blob + rec_offset + r * first_rec_stride
  const int ng = cols / kGroup;
  for (int r = 0; r < rows; ++r)
    if (!pack_row(bits, cols, codes + (size_t)r * cols, scale + (size_t)r * ng, bias + (size_t)r * ng,
                  blob + rec_offset + (size_t)r * first_rec_stride))
      return false;
  return true;
}

void unpack_matrix(int bits, int rows, int cols, const uint8_t *blob, size_t rec_stride, size_t rec_offset,
                   uint8_t *codes, uint16_t *scale, uint16_t *bias) {
  const int ng = cols / kGroup;
  for (int r = 0; r < rows; ++r)
    unpack_row(bits, cols, blob + rec_offset + (size_t)r * rec_stride, codes + (size_t)r * cols,
               scale + (size_t)r * ng, bias + (size_t)r * ng);
}

}  // namespace fmoe
