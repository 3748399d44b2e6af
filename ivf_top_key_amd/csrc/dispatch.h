// Compile-time instantiation of the (format, dimension, head-tile) variants.
//   fp32: d in {32, 64, 128};  bf16 / E4M3: d in {64, 128};  head tiles of 32: 1, 2 or 4.
#pragma once

#include "dev.h"

#define IVFTK_DISPATCH_HT(FN, DT_, D_, HT_, ...) \
  switch (HT_) {                                 \
    case 1: return FN<DT_, D_, 1>(__VA_ARGS__);  \
    case 2: return FN<DT_, D_, 2>(__VA_ARGS__);  \
    case 4: return FN<DT_, D_, 4>(__VA_ARGS__);  \
    default: return hipErrorInvalidValue;        \
  }

// One format's dimensions (a statement that returns when DIM matches).
#define IVFTK_DISPATCH_F32(FN, DIM, HT_, ...)                                    \
  if ((DIM) == 32) IVFTK_DISPATCH_HT(FN, ivftk::DT_F32, 32, HT_, __VA_ARGS__)    \
  if ((DIM) == 64) IVFTK_DISPATCH_HT(FN, ivftk::DT_F32, 64, HT_, __VA_ARGS__)    \
  if ((DIM) == 128) IVFTK_DISPATCH_HT(FN, ivftk::DT_F32, 128, HT_, __VA_ARGS__)
#define IVFTK_DISPATCH_BF16(FN, DIM, HT_, ...)                                   \
  if ((DIM) == 64) IVFTK_DISPATCH_HT(FN, ivftk::DT_BF16, 64, HT_, __VA_ARGS__)   \
  if ((DIM) == 128) IVFTK_DISPATCH_HT(FN, ivftk::DT_BF16, 128, HT_, __VA_ARGS__)
#define IVFTK_DISPATCH_E4M3(FN, DIM, HT_, ...)                                   \
  if ((DIM) == 64) IVFTK_DISPATCH_HT(FN, ivftk::DT_E4M3, 64, HT_, __VA_ARGS__)   \
  if ((DIM) == 128) IVFTK_DISPATCH_HT(FN, ivftk::DT_E4M3, 128, HT_, __VA_ARGS__)

#define IVFTK_DISPATCH(FN, DTYPE, DIM, HT_, ...)                                   \
  do {                                                                            \
    if ((DTYPE) == ivftk::DT_F32) {                                               \
      IVFTK_DISPATCH_F32(FN, DIM, HT_, __VA_ARGS__)                               \
    } else if ((DTYPE) == ivftk::DT_BF16) {                                       \
      IVFTK_DISPATCH_BF16(FN, DIM, HT_, __VA_ARGS__)                              \
    } else if ((DTYPE) == ivftk::DT_E4M3) {                                       \
      IVFTK_DISPATCH_E4M3(FN, DIM, HT_, __VA_ARGS__)                              \
    }                                                                             \
    return hipErrorInvalidValue;                                                  \
  } while (0)

// Same, without the head-tile parameter (clustering kernels).
#define IVFTK_DISPATCH_D(FN, DTYPE, DIM, ...)                                   \
  do {                                                                          \
    if ((DTYPE) == ivftk::DT_F32) {                                             \
      if ((DIM) == 32) return FN<ivftk::DT_F32, 32>(__VA_ARGS__);               \
      if ((DIM) == 64) return FN<ivftk::DT_F32, 64>(__VA_ARGS__);               \
      if ((DIM) == 128) return FN<ivftk::DT_F32, 128>(__VA_ARGS__);             \
    } else if ((DTYPE) == ivftk::DT_BF16) {                                     \
      if ((DIM) == 64) return FN<ivftk::DT_BF16, 64>(__VA_ARGS__);              \
      if ((DIM) == 128) return FN<ivftk::DT_BF16, 128>(__VA_ARGS__);            \
    } else if ((DTYPE) == ivftk::DT_E4M3) {                                     \
      if ((DIM) == 64) return FN<ivftk::DT_E4M3, 64>(__VA_ARGS__);              \
      if ((DIM) == 128) return FN<ivftk::DT_E4M3, 128>(__VA_ARGS__);            \
    }                                                                           \
    return hipErrorInvalidValue;                                                \
  } while (0)
