// Persistent frame kernel instance: temporal head dim 128, q8_0 weights, float32 KV.
#include "persistent_variants.h"

using mk::bf16_t;

PVariant pvariant_hd128_q8_kvf32() { return pvariant<mk::q8_t, bf16_t, float, 128, 4, 2, 6, 1, 2>(MOSHI_BAND_Q8); }
