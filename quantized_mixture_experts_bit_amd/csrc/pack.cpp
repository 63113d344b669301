// Host-side packer: canonical MLX-style quantized matrices <-> the device tile format.
//
// Canonical 4-bit row: byte j holds column 2j in its low nibble and 2j+1 in its
// high nibble; (s, b) are bf16 per group of 64 columns (the affine 4-bit,
// group-64, BF16 scale+bias format the TurboFieldfare pages name: ai-heartland
// review "TurboFieldfareとは", system-design summary). The device format is the
// 64x64 tile layout documented in common.h; it is a pure permutation of the
// canonical bytes, so the unpackers recover them exactly.
#include <stdint.h>
#include <string.h>

#include "moe.h"

namespace {

constexpr int64_t kTile4 = 2304, kTile8 = 4352;

bool shape_ok(int32_t rows, int32_t cols) { return rows > 0 && cols > 0 && rows % 64 == 0 && cols % 64 == 0; }

// four canonical bytes (columns c0..c0+7) -> one device code word
inline uint32_t to_word(const uint8_t* src) {
  uint32_t w = 0;
  for (int i = 0; i < 4; ++i) {
    w |= (uint32_t)(src[i] & 0x0F) << (4 * i);        // column c0 + 2i
    w |= (uint32_t)(src[i] >> 4) << (16 + 4 * i);     // column c0 + 2i + 1
  }
  return w;
}

inline void from_word(uint32_t w, uint8_t* dst) {
  for (int i = 0; i < 4; ++i)
    dst[i] = (uint8_t)(((w >> (4 * i)) & 0x0F) | (((w >> (16 + 4 * i)) & 0x0F) << 4));
}

}  // namespace

extern "C" {

uint64_t moe_matrix4_bytes(int32_t rows, int32_t cols) {
  if (!shape_ok(rows, cols)) return 0;
  return (uint64_t)(rows / 64) * (uint64_t)(cols / 64) * kTile4;
}

uint64_t moe_matrix8_bytes(int32_t rows, int32_t cols) {
  if (!shape_ok(rows, cols)) return 0;
  return (uint64_t)(rows / 64) * (uint64_t)(cols / 64) * kTile8;
}

moe_status moe_pack_matrix4(const uint8_t* q, const uint16_t* s, const uint16_t* b, int32_t rows, int32_t cols,
                            uint8_t* out) {
  if (!q || !s || !b || !out) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols)) return MOE_ERR_UNSUPPORTED_SHAPE;
  const int64_t G = cols / 64, qrow = cols / 2;
  for (int64_t nb = 0; nb < rows / 64; ++nb)
    for (int64_t g = 0; g < G; ++g) {
      uint8_t* tile = out + (nb * G + g) * kTile4;
      for (int64_t r = 0; r < 64; ++r) {
        const int64_t n = nb * 64 + r;
        for (int h = 0; h < 2; ++h)
          for (int j = 0; j < 4; ++j) {
            const int64_t c0 = g * 64 + h * 32 + j * 8;
            uint32_t w = to_word(q + n * qrow + c0 / 2);
            memcpy(tile + h * 1024 + r * 16 + j * 4, &w, 4);
          }
        uint32_t sb = (uint32_t)s[n * G + g] | ((uint32_t)b[n * G + g] << 16);
        memcpy(tile + 2048 + r * 4, &sb, 4);
      }
    }
  return MOE_OK;
}

moe_status moe_unpack_matrix4(const uint8_t* in, int32_t rows, int32_t cols, uint8_t* q, uint16_t* s, uint16_t* b) {
  if (!q || !s || !b || !in) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols)) return MOE_ERR_UNSUPPORTED_SHAPE;
  const int64_t G = cols / 64, qrow = cols / 2;
  for (int64_t nb = 0; nb < rows / 64; ++nb)
    for (int64_t g = 0; g < G; ++g) {
      const uint8_t* tile = in + (nb * G + g) * kTile4;
      for (int64_t r = 0; r < 64; ++r) {
        const int64_t n = nb * 64 + r;
        for (int h = 0; h < 2; ++h)
          for (int j = 0; j < 4; ++j) {
            const int64_t c0 = g * 64 + h * 32 + j * 8;
            uint32_t w;
            memcpy(&w, tile + h * 1024 + r * 16 + j * 4, 4);
            from_word(w, q + n * qrow + c0 / 2);
          }
        uint32_t sb;
        memcpy(&sb, tile + 2048 + r * 4, 4);
        s[n * G + g] = (uint16_t)(sb & 0xFFFF);
        b[n * G + g] = (uint16_t)(sb >> 16);
      }
    }
  return MOE_OK;
}

moe_status moe_pack_matrix8(const uint8_t* q, const uint16_t* s, const uint16_t* b, int32_t rows, int32_t cols,
                            uint8_t* out) {
  if (!q || !s || !b || !out) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols)) return MOE_ERR_UNSUPPORTED_SHAPE;
  const int64_t G = cols / 64;
  for (int64_t nb = 0; nb < rows / 64; ++nb)
    for (int64_t g = 0; g < G; ++g) {
      uint8_t* tile = out + (nb * G + g) * kTile8;
      for (int64_t r = 0; r < 64; ++r) {
        const int64_t n = nb * 64 + r;
        for (int c = 0; c < 4; ++c) memcpy(tile + c * 1024 + r * 16, q + n * cols + g * 64 + c * 16, 16);
        uint32_t sb = (uint32_t)s[n * G + g] | ((uint32_t)b[n * G + g] << 16);
        memcpy(tile + 4096 + r * 4, &sb, 4);
      }
    }
  return MOE_OK;
}

moe_status moe_unpack_matrix8(const uint8_t* in, int32_t rows, int32_t cols, uint8_t* q, uint16_t* s, uint16_t* b) {
  if (!q || !s || !b || !in) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols)) return MOE_ERR_UNSUPPORTED_SHAPE;
  const int64_t G = cols / 64;
  for (int64_t nb = 0; nb < rows / 64; ++nb)
    for (int64_t g = 0; g < G; ++g) {
      const uint8_t* tile = in + (nb * G + g) * kTile8;
      for (int64_t r = 0; r < 64; ++r) {
        const int64_t n = nb * 64 + r;
        for (int c = 0; c < 4; ++c) memcpy(q + n * cols + g * 64 + c * 16, tile + c * 1024 + r * 16, 16);
        uint32_t sb;
        memcpy(&sb, tile + 4096 + r * 4, 4);
        s[n * G + g] = (uint16_t)(sb & 0xFFFF);
        b[n * G + g] = (uint16_t)(sb >> 16);
      }
    }
  return MOE_OK;
}

}  // extern "C"
