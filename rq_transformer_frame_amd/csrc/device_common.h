// Device-side primitives shared by the frame-step kernels (gfx950, wave64).
#pragma once
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

// Sum over the 64 lanes; the result is taken from lane 0 by callers that need one value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

// Sum over 64 lanes, lane 0's value broadcast so every lane holds identical bits.
__device__ __forceinline__ float wave_sum_bcast(float v) { return __shfl(wave_sum(v), 0, WAVE); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, WAVE));
  return v;
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

// One wave computes the dot products of R weight rows (row r starts at W + rowoff[r]) with the
// vector xs[0..K) held in LDS, for any K (multiple of the vector width): lane l handles the
// 16-byte vectors l, l + 64, l + 128, ... of each row, U vectors per row in flight at a time.
// acc[r] is the lane's partial sum.
template <typename WT, int R, int U>
__device__ __forceinline__ void wave_rows_dot(const WT *__restrict__ W, int K, const int64_t *rowoff,
                                              const float *__restrict__ xs, float *acc) {
  constexpr int N = WVec<WT>::N;
  const int lane = threadIdx.x & 63;
  const int nv = K / N;
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  int v0 = 0;
  for (; v0 + U * WAVE <= nv; v0 += U * WAVE) {
    uint4 w[R][U];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) w[r][u] = ld_stream(reinterpret_cast<const uint4 *>(W + rowoff[r]) + v0 + u * WAVE + lane);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float *xp = xs + (size_t)(v0 + u * WAVE + lane) * N;
      float xv[N];
#pragma unroll
      for (int i = 0; i < N; ++i) xv[i] = xp[i];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float wf[N];
        WVec<WT>::cvt(w[r][u], wf);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[r] = fmaf(wf[i], xv[i], acc[r]);
      }
    }
  }
  for (int v = v0 + lane; v < nv; v += WAVE) {
    const float *xp = xs + (size_t)v * N;
    float xv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) xv[i] = xp[i];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4 wv = ld_stream(reinterpret_cast<const uint4 *>(W + rowoff[r]) + v);
      float wf[N];
      WVec<WT>::cvt(wv, wf);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[r] = fmaf(wf[i], xv[i], acc[r]);
    }
  }
}

// Register tile of one wave: R whole weight rows, VPL 16-byte vectors per lane per row (vector v
// = lane + 64 i; vectors past the row end read as zero).  load() issues every load of the tile at
// once and returns; dot() consumes the tile against xs in LDS.  Splitting the two lets a kernel
// issue its weight loads before its prologue and prefetch the next rows while it reduces.
// VPL == 0 is the generic form for any K: load() only records the rows and dot() streams them.
template <typename WT, int R, int VPL>
struct RowTile {
  static constexpr int N = WVec<WT>::N;
  uint4 w[R][VPL];
  __device__ __forceinline__ void load(const WT *__restrict__ W, int K, const int *rows) {
    const int lane = threadIdx.x & 63;
    const int nv = K / N;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4 *p = reinterpret_cast<const uint4 *>(W + (size_t)rows[r] * K);
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int v = lane + WAVE * i;
        w[r][i] = v < nv ? ld_stream(p + v) : uint4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void dot(const WT *__restrict__, int K, const float *__restrict__ xs, float *acc) const {
    const int lane = threadIdx.x & 63;
    const int nv = K / N;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int v = lane + WAVE * i;
      if (v < nv) {
        const float *xp = xs + (size_t)v * N;
        float xv[N];
#pragma unroll
        for (int e = 0; e < N; ++e) xv[e] = xp[e];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float wf[N];
          WVec<WT>::cvt(w[r][i], wf);
#pragma unroll
          for (int e = 0; e < N; ++e) acc[r] = fmaf(wf[e], xv[e], acc[r]);
        }
      }
    }
  }
};

template <typename WT, int R>
struct RowTile<WT, R, 0> {
  int64_t ro[R];
  __device__ __forceinline__ void load(const WT *__restrict__, int K, const int *rows) {
#pragma unroll
    for (int r = 0; r < R; ++r) ro[r] = (int64_t)rows[r] * K;
  }
  __device__ __forceinline__ void dot(const WT *__restrict__ W, int K, const float *__restrict__ xs, float *acc) const {
    wave_rows_dot<WT, R, 8>(W, K, ro, xs, acc);
  }
};

// ---- cross-block exchange inside one kernel -------------------------------------------------
// Data another block of the same kernel reads is written with system-scope stores (write-through
// past the per-XCD L2) and read with system-scope loads; the writer waits for its stores to
// complete (s_waitcnt vmcnt(0)) before it signals with an atomic.
__device__ __forceinline__ void st_sys(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
__device__ __forceinline__ float ld_sys(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Staging of a block's input vector into LDS.  Every thread issues STAGE_UNR float4 loads before
// it stores any of them (one memory round trip per STAGE_UNR * BLOCK * 4 floats instead of one
// per BLOCK floats).  K is a multiple of 4 and src is 16-byte aligned.
constexpr int STAGE_UNR = 8;

// xs[k] = src[k] for k < K; returns this thread's partial sum of squares.  No barrier.  With SYS
// the source is read with system-scope 8-byte loads (data another block of the same kernel wrote),
// U loads per thread in flight per pass.
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
    const int K2 = K >> 1;
    const uint64_t *s2 = reinterpret_cast<const uint64_t *>(src);
    for (int base = 0; base < K2; base += U * NT) {
      uint64_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * NT + threadIdx.x;
        v[u] = i < K2 ? __hip_atomic_load(const_cast<uint64_t *>(s2 + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                      : 0ull;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * NT + threadIdx.x;
        if (i < K2) {
          const float a = __uint_as_float((uint32_t)v[u]), b = __uint_as_float((uint32_t)(v[u] >> 32));
          xs[2 * i] = a;
          xs[2 * i + 1] = b;
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
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
