// Device-side primitives shared by the frame-step kernels (gfx950, wave64).
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

constexpr int WAVE = 64;
constexpr int BLOCK = 256;
constexpr int NWAVES = BLOCK / WAVE;
constexpr int MAX_STREAMS = 33;  // 2 * dep_q + 1 upper bound (dep_q <= 16)

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u) return (bf16_t)((b >> 16) | ((b & 0xFFFFu) ? 0x40u : 0u));
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (bf16_t)(b >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// Cross-lane reductions on DPP moves (VALU, no LDS round trip per step).  A DPP move with full row
// and bank masks and bound_ctrl reads lane CTRL-selected within its row of 16.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over each row of 16 lanes: the two quad swaps (quad_perm [1,0,3,2], [2,3,0,1]), then the
// half-row mirror and the row mirror.  Each step adds two partial sums that are equal in both
// lanes of a pair (float addition commutes), so every lane of the row ends with identical bits.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

// Sum over the 64 lanes: row sums, then (row 0 + row 1) + (row 2 + row 3) from lanes 0, 16, 32, 48;
// every lane holds identical bits.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// Lane l's value combined with lane l ^ 32's (l ^ 16's) through the gfx950 lane swaps (VALU): with
// both operands v, the two results hold, in every lane, the two values of the pair, so their sum
// (max) has identical bits in both lanes -- the same value a shuffle-and-add gives.
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over 64 lanes with identical bits in every lane.
__device__ __forceinline__ float wave_sum_bcast(float v) { return wave_sum(v); }

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Block-wide sum: each wave's lane-0 sum goes to LDS, then every thread adds the wave sums in
// the same order, so all threads hold the same value.
template <int NT = BLOCK>
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) t += red[i];
  __syncthreads();
  return t;
}

template <int NT = BLOCK>
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < NT / WAVE; ++i) t = fmaxf(t, red[i]);
  __syncthreads();
  return t;
}

// ---- greedy argmax candidates ------------------------------------------------------------
// First-wins argmax: among values strictly above -inf (NaN never qualifies) the largest wins,
// ties go to the smaller index; no candidate at all means index 0.
struct ArgBest {
  float v;
  int i;  // -1: no candidate
};

__device__ __forceinline__ ArgBest arg_none() { return ArgBest{-INFINITY, -1}; }

__device__ __forceinline__ ArgBest arg_take(ArgBest a, float v, int i) {
  if (v > -INFINITY) {  // false for NaN and -inf
    if (a.i < 0 || v > a.v || (v == a.v && i < a.i)) return ArgBest{v, i};
  }
  return a;
}

__device__ __forceinline__ ArgBest arg_merge(ArgBest a, ArgBest b) {
  if (b.i < 0) return a;
  if (a.i < 0) return b;
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ __forceinline__ ArgBest wave_arg(ArgBest a) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    ArgBest o{__shfl_xor(a.v, m, WAVE), __shfl_xor(a.i, m, WAVE)};
    a = arg_merge(a, o);
  }
  return a;
}

// ---- 16-byte weight vectors -------------------------------------------------------------
template <typename WT> struct WVec;

template <> struct WVec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void cvt(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};

template <> struct WVec<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void cvt(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xFFFF0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xFFFF0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xFFFF0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xFFFF0000u);
  }
};

template <> struct WVec<int8_t> {
  static constexpr int N = 16;
  __device__ __forceinline__ static void cvt(const uint4 &u, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * j + b] = (float)(int32_t)(int8_t)((w[j] >> (8 * b)) & 0xFFu);
    }
  }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load with the non-temporal hint (weights are read once per frame).
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

// ---- weight streaming ------------------------------------------------------------------------
// A wave's share of a projection y = W . x: the rows [r0, r1) of W (row-major, K columns), walked
// in chunks of SCH 16-byte vectors per lane (8 KB per wave), always two chunks in flight.  Chunk c
// of a row covers the vectors c*SCH*64 + i*64 + lane (i < SCH) of the row.  Loads go through a
// buffer resource spanning exactly the row, so vectors past the row end read as zero without a
// memory access and every chunk is the same SCH unconditional loads: with no loads under a
// branch, the compiler can count the loads in flight and wait for one chunk at a time (loads
// complete in order; a branch around a load makes it wait for all of them).  The input vector is
// read from LDS.  begin() issues the first two chunks and returns, so a kernel can start its
// weight stream before its prologue; run() walks the rest and calls epi(row, value) once per row,
// in every lane, with the wave-reduced dot product times the row's scale (int8 rows).  Epilogues
// must not load from global memory, for the same reason.
constexpr int SCH = 8;
constexpr int BUF_DWORD3 = 0x00020000;  // raw 32-bit buffer resource word 3 for gfx9-family parts
constexpr int BUF_NT = 2;               // cache policy: nontemporal (streamed once)
constexpr int BUF_OOB = 0x7FFFFFF0;     // an offset past the end of every buffer resource used here

typedef unsigned int u32x4b __attribute__((ext_vector_type(4)));

template <typename WT>
struct RowStream {
  static constexpr int N = WVec<WT>::N;
  uint4 a[SCH], b[SCH];
  float sa, sb;  // scales of the rows whose last chunk is in a / b
  const WT *W;
  const float *S;
  int K, nv, nch, r0, T;
  int lq, lc;  // row (relative to r0) and chunk of the next load
  int cq, cc;  // row and chunk of the next chunk consumed

  // Load chunk (lq, lc) into buf and advance.
  __device__ __forceinline__ void load(uint4 (&buf)[SCH], float &sc) {
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + (size_t)(r0 + lq) * K), (short)0, nv * 16, BUF_DWORD3);
    const int soff = lc * (SCH * WAVE * 16);
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const u32x4b v = __builtin_amdgcn_raw_buffer_load_b128(rs, (i * WAVE + lane) * 16, soff, BUF_NT);
      buf[i] = uint4{v[0], v[1], v[2], v[3]};
    }
    if (S && lc == nch - 1) sc = S[r0 + lq];
    if (++lc == nch) {
      lc = 0;
      ++lq;
    }
  }

  __device__ __forceinline__ void begin(const WT *__restrict__ W_, const float *__restrict__ S_, int K_, int r0_,
                                        int r1_) {
    W = W_;
    S = S_;
    K = K_;
    nv = K_ / N;
    nch = (nv + SCH * WAVE - 1) / (SCH * WAVE);
    r0 = r0_;
    T = (r1_ > r0_ ? r1_ - r0_ : 0) * nch;
    lq = lc = 0;
    sa = sb = 1.f;
    if (T > 0) load(a, sa);
    if (T > 1) load(b, sb);
  }

  __device__ __forceinline__ float dot1(const uint4 &w, const float *__restrict__ xp, float acc) const {
    float xv[N], wf[N];
#pragma unroll
    for (int e = 0; e < N; e += 4) {
      const float4 q = *reinterpret_cast<const float4 *>(xp + e);
      xv[e] = q.x;
      xv[e + 1] = q.y;
      xv[e + 2] = q.z;
      xv[e + 3] = q.w;
    }
    WVec<WT>::cvt(w, wf);
#pragma unroll
    for (int e = 0; e < N; ++e) acc = fmaf(wf[e], xv[e], acc);
    return acc;
  }

  __device__ __forceinline__ float dot(const uint4 (&buf)[SCH], int c, const float *__restrict__ xs, float acc) const {
    const int lane = threadIdx.x & 63;
    const int left = nv - c * (SCH * WAVE);
    const float *xp = xs + (size_t)(c * (SCH * WAVE) + lane) * N;
    if (left >= SCH * WAVE) {
#pragma unroll
      for (int i = 0; i < SCH; ++i) acc = dot1(buf[i], xp + i * WAVE * N, acc);
    } else {
#pragma unroll
      for (int i = 0; i < SCH; ++i)
        if (i * WAVE + lane < left) acc = dot1(buf[i], xp + i * WAVE * N, acc);
    }
    return acc;
  }

  // Consume the chunk in buf (row cq, chunk cc); a finished row goes to the epilogue.
  template <typename Epi>
  __device__ __forceinline__ void consume(const uint4 (&buf)[SCH], float sc, const float *__restrict__ xs,
                                          float &acc, Epi &epi) {
    acc = dot(buf, cc, xs, acc);
    if (cc == nch - 1) {
      float v = wave_sum(acc);
      if (S) v *= sc;
      epi(r0 + cq, v);
      acc = 0.f;
      cc = 0;
      ++cq;
    } else {
      ++cc;
    }
  }

  // Steady state: every iteration consumes two chunks and loads the two after them, with no
  // condition on the loads; the last (up to three) chunks are peeled.
  template <typename Epi>
  __device__ __forceinline__ void run(const float *__restrict__ xs, Epi &&epi) {
    float acc = 0.f;
    cq = cc = 0;
    int t = 0;
    for (; t + 3 < T; t += 2) {
      consume(a, sa, xs, acc, epi);
      load(a, sa);
      consume(b, sb, xs, acc, epi);
      load(b, sb);
    }
    const int rem = T - t;
    if (rem >= 1) consume(a, sa, xs, acc, epi);
    if (rem == 3) load(a, sa);
    if (rem >= 2) consume(b, sb, xs, acc, epi);
    if (rem == 3) consume(a, sa, xs, acc, epi);
  }
};

// bf16 and int8 weights: rows are walked in pairs, so that each input fragment read from LDS
// (N floats per lane and 16-byte vector) feeds both rows' products; with one row at a time the
// LDS reads (4 bytes per weight byte for int8, 2 for bf16) and the widening share the CU with the
// stream.  A chunk is SCH_I8 vectors per lane of both rows of the pair; two pair-chunks are in
// flight (the same 16 KB per wave as the single-row stream).  A pair past the end of the wave's
// rows (odd count) reads zeros for its second row and emits only the first.  Rows are emitted in
// increasing order.
constexpr int SCH_I8 = 4;

template <typename WT>
struct PairStream {
  static constexpr int N = WVec<WT>::N;
  uint4 a0[SCH_I8], b0[SCH_I8], a1[SCH_I8], b1[SCH_I8];  // pair-chunk t (a: first row, b: second)
  float sa0, sb0, sa1, sb1;
  const WT *W;
  const float *S;
  int K, nv, nch, r0, r1, T;
  int lp, lc;  // pair and chunk of the next load
  int cp, cc;  // pair and chunk of the next chunk consumed

  __device__ __forceinline__ void load(uint4 (&A)[SCH_I8], uint4 (&B)[SCH_I8], float &sa, float &sb) {
    const int lane = threadIdx.x & 63;
    const int ra = r0 + 2 * lp, rb = ra + 1;
    const __amdgpu_buffer_rsrc_t rsa =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + (size_t)ra * K), (short)0, nv * 16, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rsb =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + (size_t)rb * K), (short)0, rb < r1 ? nv * 16 : 0, BUF_DWORD3);
    const int soff = lc * (SCH_I8 * WAVE * 16);
#pragma unroll
    for (int i = 0; i < SCH_I8; ++i) {
      const u32x4b va = __builtin_amdgcn_raw_buffer_load_b128(rsa, (i * WAVE + lane) * 16, soff, BUF_NT);
      const u32x4b vb = __builtin_amdgcn_raw_buffer_load_b128(rsb, (i * WAVE + lane) * 16, soff, BUF_NT);
      A[i] = uint4{va[0], va[1], va[2], va[3]};
      B[i] = uint4{vb[0], vb[1], vb[2], vb[3]};
    }
    if (S && lc == nch - 1) {
      sa = S[ra];
      sb = rb < r1 ? S[rb] : 0.f;
    }
    if (++lc == nch) {
      lc = 0;
      ++lp;
    }
  }

  __device__ __forceinline__ void begin(const WT *__restrict__ W_, const float *__restrict__ S_, int K_, int r0_,
                                        int r1_) {
    W = W_;
    S = S_;
    K = K_;
    nv = K_ / N;
    nch = (nv + SCH_I8 * WAVE - 1) / (SCH_I8 * WAVE);
    r0 = r0_;
    r1 = r1_ > r0_ ? r1_ : r0_;
    T = ((r1 - r0 + 1) / 2) * nch;
    lp = lc = 0;
    sa0 = sb0 = sa1 = sb1 = 1.f;
    if (T > 0) load(a0, b0, sa0, sb0);
    if (T > 1) load(a1, b1, sa1, sb1);
  }

  __device__ __forceinline__ static float cvt_dot(const uint4 &w, const float *xv, float acc) {
    float wf[N];
    WVec<WT>::cvt(w, wf);
#pragma unroll
    for (int e = 0; e < N; ++e) acc = fmaf(wf[e], xv[e], acc);
    return acc;
  }

  // Consume pair-chunk (A, B) (pair cp, chunk cc); finished rows go to the epilogue.
  template <typename Epi>
  __device__ __forceinline__ void consume(const uint4 (&A)[SCH_I8], const uint4 (&B)[SCH_I8], float sa, float sb,
                                          const float *__restrict__ xs, float &acca, float &accb, Epi &epi) {
    const int lane = threadIdx.x & 63;
    const int left = nv - cc * (SCH_I8 * WAVE);
    const float *xp = xs + (size_t)(cc * (SCH_I8 * WAVE) + lane) * N;
#pragma unroll
    for (int i = 0; i < SCH_I8; ++i) {
      if (left >= SCH_I8 * WAVE || i * WAVE + lane < left) {
        float xv[N];
#pragma unroll
        for (int e = 0; e < N; e += 4) {
          const float4 q = *reinterpret_cast<const float4 *>(xp + i * WAVE * N + e);
          xv[e] = q.x;
          xv[e + 1] = q.y;
          xv[e + 2] = q.z;
          xv[e + 3] = q.w;
        }
        acca = cvt_dot(A[i], xv, acca);
        accb = cvt_dot(B[i], xv, accb);
      }
    }
    if (cc == nch - 1) {
      const int ra = r0 + 2 * cp, rb = ra + 1;
      float va = wave_sum(acca), vb = wave_sum(accb);
      if (S) {
        va *= sa;
        vb *= sb;
      }
      epi(ra, va);
      if (rb < r1) epi(rb, vb);
      acca = accb = 0.f;
      cc = 0;
      ++cp;
    } else {
      ++cc;
    }
  }

  template <typename Epi>
  __device__ __forceinline__ void run(const float *__restrict__ xs, Epi &&epi) {
    float acca = 0.f, accb = 0.f;
    cp = cc = 0;
    int t = 0;
    for (; t + 3 < T; t += 2) {
      consume(a0, b0, sa0, sb0, xs, acca, accb, epi);
      load(a0, b0, sa0, sb0);
      consume(a1, b1, sa1, sb1, xs, acca, accb, epi);
      load(a1, b1, sa1, sb1);
    }
    const int rem = T - t;
    if (rem >= 1) consume(a0, b0, sa0, sb0, xs, acca, accb, epi);
    if (rem == 3) load(a0, b0, sa0, sb0);
    if (rem >= 2) consume(a1, b1, sa1, sb1, xs, acca, accb, epi);
    if (rem == 3) consume(a0, b0, sa0, sb0, xs, acca, accb, epi);
  }
};

template <> struct RowStream<int8_t> : PairStream<int8_t> {};
template <> struct RowStream<bf16_t> : PairStream<bf16_t> {};

// ---- block-scaled weights (the Q4_0 and q8_0 bands) --------------------------------------------
// A row of K weights is K / 32 blocks of 32 columns, each with one float32 scale; the scales of a
// matrix are [rows][K / 32].  Q4_0: 16 bytes per block, byte i holding the code of column i in its
// low nibble and of column i + 16 in its high nibble, each code stored + 8 (weight = (nibble - 8)
// x scale).  q8_0: 32 int8 codes per block (weight = code x scale).
struct q4_t {
  uint8_t bits;  // two 4-bit codes
};
struct q8_t {
  int8_t bits;  // one 8-bit code
};

template <typename QT> struct QVec;
template <> struct QVec<q4_t> {
  static constexpr int N = 32;    // weights per 16-byte vector: one whole block
  static constexpr int VPB = 1;   // vectors per block
  static constexpr int BPW2 = 1;  // bytes per two weights
  // weights 16 h .. 16 h + 15 of the vector: the low nibbles (h = 0) or the high ones (h = 1)
  __device__ __forceinline__ static void cvt16(const uint4 &u, int h, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (w[j] >> (8 * b)) & 0xFFu;
        f[4 * j + b] = (float)((int)(h ? (byte >> 4) : (byte & 15u)) - 8);
      }
    }
  }
};
template <> struct QVec<q8_t> {
  static constexpr int N = 16;
  static constexpr int VPB = 2;
  static constexpr int BPW2 = 2;
  __device__ __forceinline__ static void cvt16(const uint4 &u, int, float *f) { WVec<int8_t>::cvt(u, f); }
};

// The pair stream for block-scaled weights: rows walked in pairs as in PairStream (one input
// fragment from LDS feeds both rows), each 16-byte vector's products scaled by its block's scale
// before they join the row's sum.  Scales are loaded with the vectors (4 bytes per lane and
// vector, past the row's end zero).  A pair-chunk holds SCH_B vectors per lane of each row: the
// rows are short in vectors (Q4_0 packs 32 weights in one), and the converted weights of a vector
// are what fill the registers.
constexpr int SCH_B = 2;

template <typename QT>
struct BlockPairStream {
  static constexpr int N = QVec<QT>::N;
  static constexpr int VPB = QVec<QT>::VPB;
  uint4 a0[SCH_B], b0[SCH_B], a1[SCH_B], b1[SCH_B];
  float da0[SCH_B], db0[SCH_B], da1[SCH_B], db1[SCH_B];
  const uint8_t *W;
  const float *S;
  int K, nv, nsc, rowb, nch, r0, r1, T;
  int lp, lc;
  int cp, cc;

  __device__ __forceinline__ void load(uint4 (&A)[SCH_B], uint4 (&B)[SCH_B], float (&dA)[SCH_B], float (&dB)[SCH_B]) {
    const int lane = threadIdx.x & 63;
    const int ra = r0 + 2 * lp, rb = ra + 1;
    const bool hasb = rb < r1;
    const __amdgpu_buffer_rsrc_t rsa =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + (size_t)ra * rowb), (short)0, rowb, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rsb =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + (size_t)rb * rowb), (short)0, hasb ? rowb : 0, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t ssa =
        __builtin_amdgcn_make_buffer_rsrc((void *)(S + (size_t)ra * nsc), (short)0, nsc * 4, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t ssb =
        __builtin_amdgcn_make_buffer_rsrc((void *)(S + (size_t)rb * nsc), (short)0, hasb ? nsc * 4 : 0, BUF_DWORD3);
    const int soff = lc * (SCH_B * WAVE * 16);
#pragma unroll
    for (int i = 0; i < SCH_B; ++i) {
      const u32x4b va = __builtin_amdgcn_raw_buffer_load_b128(rsa, (i * WAVE + lane) * 16, soff, BUF_NT);
      const u32x4b vb = __builtin_amdgcn_raw_buffer_load_b128(rsb, (i * WAVE + lane) * 16, soff, BUF_NT);
      A[i] = uint4{va[0], va[1], va[2], va[3]};
      B[i] = uint4{vb[0], vb[1], vb[2], vb[3]};
      const int v = lc * (SCH_B * WAVE) + i * WAVE + lane;
      dA[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ssa, (v / VPB) * 4, 0, BUF_NT));
      dB[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ssb, (v / VPB) * 4, 0, BUF_NT));
    }
    if (++lc == nch) {
      lc = 0;
      ++lp;
    }
  }

  __device__ __forceinline__ void begin(const QT *__restrict__ W_, const float *__restrict__ S_, int K_, int r0_,
                                        int r1_) {
    W = reinterpret_cast<const uint8_t *>(W_);
    S = S_;
    K = K_;
    nv = K_ / N;
    nsc = K_ / 32;
    rowb = K_ * QVec<QT>::BPW2 / 2;
    nch = (nv + SCH_B * WAVE - 1) / (SCH_B * WAVE);
    r0 = r0_;
    r1 = r1_ > r0_ ? r1_ : r0_;
    T = ((r1 - r0 + 1) / 2) * nch;
    lp = lc = 0;
    if (T > 0) load(a0, b0, da0, db0);
    if (T > 1) load(a1, b1, da1, db1);
  }

  template <typename Epi>
  __device__ __forceinline__ void consume(const uint4 (&A)[SCH_B], const uint4 (&B)[SCH_B], const float (&dA)[SCH_B],
                                          const float (&dB)[SCH_B], const float *__restrict__ xs, float &acca,
                                          float &accb, Epi &epi) {
    const int lane = threadIdx.x & 63;
    const int left = nv - cc * (SCH_B * WAVE);
    const float *xp = xs + (size_t)(cc * (SCH_B * WAVE) + lane) * N;
#pragma unroll
    for (int i = 0; i < SCH_B; ++i) {
      if (left >= SCH_B * WAVE || i * WAVE + lane < left) {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int h = 0; h < N / 16; ++h) {  // 16 weights of both rows per pass
          float xv[16], wa[16], wb[16];
#pragma unroll
          for (int e = 0; e < 16; e += 4) {
            const float4 q = *reinterpret_cast<const float4 *>(xp + i * WAVE * N + 16 * h + e);
            xv[e] = q.x;
            xv[e + 1] = q.y;
            xv[e + 2] = q.z;
            xv[e + 3] = q.w;
          }
          QVec<QT>::cvt16(A[i], h, wa);
          QVec<QT>::cvt16(B[i], h, wb);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            sa = fmaf(wa[e], xv[e], sa);
            sb = fmaf(wb[e], xv[e], sb);
          }
        }
        acca = fmaf(dA[i], sa, acca);
        accb = fmaf(dB[i], sb, accb);
      }
    }
    if (cc == nch - 1) {
      const int ra = r0 + 2 * cp, rb = ra + 1;
      const float va = wave_sum(acca), vb = wave_sum(accb);
      epi(ra, va);
      if (rb < r1) epi(rb, vb);
      acca = accb = 0.f;
      cc = 0;
      ++cp;
    } else {
      ++cc;
    }
  }

  template <typename Epi>
  __device__ __forceinline__ void run(const float *__restrict__ xs, Epi &&epi) {
    float acca = 0.f, accb = 0.f;
    cp = cc = 0;
    int t = 0;
    for (; t + 3 < T; t += 2) {
      consume(a0, b0, da0, db0, xs, acca, accb, epi);
      load(a0, b0, da0, db0);
      consume(a1, b1, da1, db1, xs, acca, accb, epi);
      load(a1, b1, da1, db1);
    }
    const int rem = T - t;
    if (rem >= 1) consume(a0, b0, da0, db0, xs, acca, accb, epi);
    if (rem == 3) load(a0, b0, da0, db0);
    if (rem >= 2) consume(a1, b1, da1, db1, xs, acca, accb, epi);
    if (rem == 3) consume(a0, b0, da0, db0, xs, acca, accb, epi);
  }
};

template <> struct RowStream<q4_t> : BlockPairStream<q4_t> {};
template <> struct RowStream<q8_t> : BlockPairStream<q8_t> {};

template <typename WT> struct IsBlockBand : std::false_type {};
template <> struct IsBlockBand<q4_t> : std::true_type {};
template <> struct IsBlockBand<q8_t> : std::true_type {};

// Index of the calling wave in its block, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Balanced contiguous share of `units` units of P rows for wave w of TW: rows [lo, hi).
__device__ __forceinline__ void wave_rows(int w, int TW, int units, int P, int &lo, int &hi) {
  lo = (int)(((int64_t)w * units) / TW) * P;
  hi = (int)(((int64_t)(w + 1) * units) / TW) * P;
}

// ---- cross-block exchange inside one kernel -------------------------------------------------
// Data another block of the same kernel reads is written with system-scope stores (write-through
// past the per-XCD L2) and read with system-scope loads; the writer waits for its stores to
// complete (s_waitcnt vmcnt(0)) before it signals with an atomic.
__device__ __forceinline__ void st_sys(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
__device__ __forceinline__ float ld_sys(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// 16 bytes at byte offset `off` of an activation buffer written by another block of the same
// kernel, with the cache policy of a system-scope load (sc0 sc1: past both cache levels), through
// a buffer resource so that four floats move in one instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t act_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ float4 ld_sys4(__amdgpu_buffer_rsrc_t r, int off) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 17);
  return float4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
}
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Staging of a block's input vector into LDS.  Every thread issues STAGE_UNR float4 loads before
// it stores any of them (one memory round trip per STAGE_UNR * BLOCK * 4 floats instead of one
// per BLOCK floats).  K is a multiple of 4 and src is 16-byte aligned.
constexpr int STAGE_UNR = 8;

// xs[k] = src[k] for k < K; returns this thread's partial sum of squares.  No barrier.  With SYS
// the source is read with system-coherent 16-byte loads (data another block of the same kernel
// wrote), U loads per thread in flight per pass.
template <int NT = BLOCK, bool SYS = false, int U = 2 * STAGE_UNR>
__device__ __forceinline__ float stage_copy(const float *__restrict__ src, int K, float *xs) {
  float ss = 0.f;
  if (!SYS) {
    const int K4 = K >> 2;
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
    float4 *x4 = reinterpret_cast<float4 *>(xs);
    for (int base = 0; base < K4; base += STAGE_UNR * NT) {
      float4 v[STAGE_UNR];
#pragma unroll
      for (int u = 0; u < STAGE_UNR; ++u) {
        const int i = base + u * NT + threadIdx.x;
        v[u] = i < K4 ? s4[i] : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < STAGE_UNR; ++u) {
        const int i = base + u * NT + threadIdx.x;
        if (i < K4) {
          x4[i] = v[u];
          ss = fmaf(v[u].x, v[u].x, ss);
          ss = fmaf(v[u].y, v[u].y, ss);
          ss = fmaf(v[u].z, v[u].z, ss);
          ss = fmaf(v[u].w, v[u].w, ss);
        }
      }
    }
  } else {
    const int K4 = K >> 2;
    const __amdgpu_buffer_rsrc_t r = act_rsrc(src);
    float4 *x4 = reinterpret_cast<float4 *>(xs);
    for (int base = 0; base < K4; base += U * NT) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * NT + threadIdx.x;
        v[u] = i < K4 ? ld_sys4(r, i * 16) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * NT + threadIdx.x;
        if (i < K4) {
          x4[i] = v[u];
          ss = fmaf(v[u].x, v[u].x, ss);
          ss = fmaf(v[u].y, v[u].y, ss);
          ss = fmaf(v[u].z, v[u].z, ss);
          ss = fmaf(v[u].w, v[u].w, ss);
        }
      }
    }
  }
  return ss;
}

// xs[k] = src[k] for k < K, then a barrier.
template <int NT = BLOCK, bool SYS = false, int U = 2 * STAGE_UNR>
__device__ __forceinline__ void stage_vec(const float *__restrict__ src, int K, float *xs) {
  (void)stage_copy<NT, SYS, U>(src, K, xs);
  __syncthreads();
}

// xs = rms_norm(src; alpha): y = x * alpha * 1/sqrt(eps + mean(x^2)) (eps inside the mean).
template <int NT = BLOCK, bool SYS = false, int U = 2 * STAGE_UNR>
__device__ __forceinline__ void stage_rms(const float *__restrict__ src, const float *__restrict__ alpha, int K,
                                          float eps, float *xs, float *red) {
  const float tot = block_sum<NT>(stage_copy<NT, SYS, U>(src, K, xs), red);  // block_sum's barriers publish xs
  const float inv = 1.0f / sqrtf(eps + tot / (float)K);
  for (int k = threadIdx.x; k < K; k += NT) xs[k] = (xs[k] * alpha[k]) * inv;
  __syncthreads();
}

// In-place rms_norm of xs[0..K) already staged in LDS.
template <int NT = BLOCK>
__device__ __forceinline__ void rms_in_place(float *xs, const float *__restrict__ alpha, int K, float eps, float *red) {
  float ss = 0.f;
  for (int k = threadIdx.x; k < K; k += NT) ss = fmaf(xs[k], xs[k], ss);
  const float tot = block_sum<NT>(ss, red);
  const float inv = 1.0f / sqrtf(eps + tot / (float)K);
  for (int k = threadIdx.x; k < K; k += NT) xs[k] = (xs[k] * alpha[k]) * inv;
  __syncthreads();
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Delay of stream s for dep_q codebooks: text 0 | generated cb0 0, cb1.. 1 | user cb0 0, cb1.. 1.
__device__ __forceinline__ int stream_delay(int s, int Q) {
  if (s == 0) return 0;
  const int k = (s - 1) % Q;
  return k == 0 ? 0 : 1;
}

}  // namespace mk
