// Persistent frame kernel instance: temporal head dim 128, bf16 weights, float32 KV.
#include "persistent_variants.h"

using mk::bf16_t;

PVariant pvariant_hd128_bf16_kvf32() { return pvariant<bf16_t, bf16_t, float, 128, 4, 2, 6, 1, 2>(MOSHI_BAND_BF16); }
