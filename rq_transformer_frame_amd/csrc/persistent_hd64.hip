// Persistent frame kernel instances for temporal head dim 64.
#include "persistent_variants.h"

using mk::bf16_t;

const PVariant *pvariants_hd64(int *n) {
  static const PVariant v[] = {
      pvariant<float, float, float, 64, 4, 1, 1, 1, 1>(MOSHI_BAND_F32),
      pvariant<bf16_t, bf16_t, float, 64, 4, 1, 1, 1, 1>(MOSHI_BAND_BF16),
      pvariant<int8_t, bf16_t, float, 64, 4, 1, 1, 1, 1>(MOSHI_BAND_I8),
      pvariant<mk::q4_t, bf16_t, float, 64, 4, 1, 1, 1, 1>(MOSHI_BAND_Q4),
      pvariant<mk::q8_t, bf16_t, float, 64, 4, 1, 1, 1, 1>(MOSHI_BAND_Q8),
  };
  *n = (int)(sizeof(v) / sizeof(v[0]));
  return v;
}
