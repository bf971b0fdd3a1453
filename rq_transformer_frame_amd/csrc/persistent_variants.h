// Compiled instances of the persistent frame kernel, one translation unit per group so they build
// in parallel.
#pragma once
#include <type_traits>

#include "frame_persistent.h"
#include "moshi_mi355x.h"

// One instance: (band, KV storage, temporal head dim, depformer head dim / 16, 16-byte staging
// loads per thread and pass for inputs of width D, F, Dd, Fd).  The staging counts only set how
// many loads each thread has in flight, so a shape without its own instance runs the generic one
// of its band, KV storage and head dims.
struct PVariant {
  int band, kv, hd, depl, ud, uf, udd, ufd;
  const void *fn;
};

template <typename WT, typename ET, typename KT, int HD, int DEPL, int UD, int UF, int UDd, int UFd>
PVariant pvariant(int band) {
  return PVariant{band, std::is_same<KT, float>::value ? MOSHI_KV_F32 : MOSHI_KV_BF16, HD, DEPL, UD, UF, UDd, UFd,
                  reinterpret_cast<const void *>(&mk::k_frame_persistent<WT, ET, KT, HD, DEPL, UD, UF, UDd, UFd>)};
}

// Temporal head dim 128 (the Moshi-7B shape: d4096 / ffn 11264, depformer d1024 / ffn 2816), one
// instance per translation unit: bf16 weights with float32 or bf16 KV, int8, Q4_0 and q8_0 weights.
PVariant pvariant_hd128_bf16_kvf32();
PVariant pvariant_hd128_bf16_kvbf16();
PVariant pvariant_hd128_i8_kvf32();
PVariant pvariant_hd128_q4_kvf32();
PVariant pvariant_hd128_q8_kvf32();
// Temporal head dim 64 (small shapes, one staging pass per 2048-wide input).
const PVariant *pvariants_hd64(int *n);
