// Batched projections on the matrix cores (gfx950 MFMA) for the frame of several conversations
// and for the teacher-forced prefill: Y[m][n] = sum_k X[m][k] * W[n][k] (times the row scale of an
// int8 W), stored or added to Y.  This is the same product the single-conversation kernels form
// one row at a time ([LM] temporal_step / depformer_cycle linears); with M conversations (or M
// prefill positions) the weights are streamed once for all of them.
//
// Operands: bf16 and int8 weights multiply the activations split into bf16 hi and lo parts
// (v_mfma_f32_32x32x16_bf16 twice, fp32 accumulation; int8 values convert to bf16 exactly); f32
// weights multiply f32 activations (v_mfma_f32_32x32x2_f32).
//
// Tiling: a block owns 32 weight rows and 64 activation rows; its 4 waves split K and their
// accumulators are summed in LDS in wave order.  Per 64-wide K block, lane l (n = l % 32,
// half g = l / 32) loads the contiguous 32 columns [kb + 32 g, kb + 32 g + 32) of weight row n
// and of activation rows m and m + 32.  The matrix core pairs equal (lane half, element) slots
// of its two operands, so handing both operands the same column permutation leaves every dot
// product intact.  Loads go through buffer resources: rows past N or M and 16-byte pieces past
// K read as zero (K a multiple of 16).
#pragma once
#include "device_common.h"

namespace mk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GM = 64;       // activation rows per block
constexpr int GN = 32;       // weight rows per block
constexpr int GKB = 64;      // K block
constexpr int GWAVES = 4;    // waves per block (split K)
constexpr int GBLOCK = GWAVES * WAVE;

// Activation element type paired with a weight type.
template <typename WT> struct GemmX { typedef bf16_t type; };
template <> struct GemmX<float> { typedef float type; };

// A projection input row holds K values.  With bf16 operands each value v is stored as the pair
// hi = bf16(v), lo = bf16(v - hi) (row = [hi of K columns | lo of K columns], so the row stride is
// at least 2 K): the products hi . w + lo . w carry v to about 16 significant bits, and the
// matrix-core result matches float32 activations far below the bf16 weights' own rounding.
// float32 operands store v once.
template <typename XT> struct XPut;
template <> struct XPut<float> {
  static constexpr int PLANES = 1;
  __device__ __forceinline__ static void put(float *row, int K, int k, float v) { row[k] = v; }
};
template <> struct XPut<bf16_t> {
  static constexpr int PLANES = 2;
  __device__ __forceinline__ static void put(bf16_t *row, int K, int k, float v) {
    const bf16_t hi = f2bf(v);
    row[k] = hi;
    row[K + k] = f2bf(v - bf2f(hi));
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

// 16 bytes at byte offset off of a buffer resource (zero when out of range).
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return uint4{v[0], v[1], v[2], v[3]};
}

// Eight int8 weights (low or high 8 bytes of u) as bf16 bit patterns.
__device__ __forceinline__ uint4 i8_to_bf16x8(uint32_t lo, uint32_t hi) {
  uint32_t w[2] = {lo, hi}, o[4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float a = (float)(int32_t)(int8_t)((w[j] >> (16 * p)) & 0xFFu);
      const float b = (float)(int32_t)(int8_t)((w[j] >> (16 * p + 8)) & 0xFFu);
      o[2 * j + p] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
    }
  return uint4{o[0], o[1], o[2], o[3]};
}

// One K block of one wave: the 4 (bf16) MFMA steps of 16 columns for both 32-row halves of the
// activation tile.
template <typename WT>
struct GemmCore;

template <>
struct GemmCore<bf16_t> {
  // w: 32 bf16 of weight row n (4 x 16 B); x0, x1: 32 bf16 (hi) of activation rows m, m + 32;
  // l0, l1: their lo parts (xlo bytes further on)
  uint4 w[4], x0[4], x1[4], l0[4], l1[4];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx, int woff, int xoff0,
                                       int xoff1, int kleft, int xlo) {
#pragma unroll
    for (int s = 0; s < 4; ++s) w[s] = buf_ld16(rw, (woff < 0 || 8 * s >= kleft) ? BUF_OOB : woff + 16 * s);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok0 = xoff0 >= 0 && 8 * s < kleft, ok1 = xoff1 >= 0 && 8 * s < kleft;
      x0[s] = buf_ld16(rx, ok0 ? xoff0 + 16 * s : BUF_OOB);
      l0[s] = buf_ld16(rx, ok0 ? xoff0 + xlo + 16 * s : BUF_OOB);
      x1[s] = buf_ld16(rx, ok1 ? xoff1 + 16 * s : BUF_OOB);
      l1[s] = buf_ld16(rx, ok1 ? xoff1 + xlo + 16 * s : BUF_OOB);
    }
  }
  __device__ __forceinline__ void mma(f32x16 &c0, f32x16 &c1) const {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x0[s]), as_bf16x8(w[s]), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x1[s]), as_bf16x8(w[s]), c1, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(l0[s]), as_bf16x8(w[s]), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(l1[s]), as_bf16x8(w[s]), c1, 0, 0, 0);
    }
  }
  static constexpr int WELT = 2;
};

template <>
struct GemmCore<int8_t> {
  uint4 wq[2], x0[4], x1[4], l0[4], l1[4];  // 32 int8 weights; activations as for bf16
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx, int woff, int xoff0,
                                       int xoff1, int kleft, int xlo) {
#pragma unroll
    for (int s = 0; s < 2; ++s) wq[s] = buf_ld16(rw, (woff < 0 || 16 * s >= kleft) ? BUF_OOB : woff + 16 * s);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok0 = xoff0 >= 0 && 8 * s < kleft, ok1 = xoff1 >= 0 && 8 * s < kleft;
      x0[s] = buf_ld16(rx, ok0 ? xoff0 + 16 * s : BUF_OOB);
      l0[s] = buf_ld16(rx, ok0 ? xoff0 + xlo + 16 * s : BUF_OOB);
      x1[s] = buf_ld16(rx, ok1 ? xoff1 + 16 * s : BUF_OOB);
      l1[s] = buf_ld16(rx, ok1 ? xoff1 + xlo + 16 * s : BUF_OOB);
    }
  }
  __device__ __forceinline__ void mma(f32x16 &c0, f32x16 &c1) const {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 &q = wq[s >> 1];
      const uint4 wb = (s & 1) ? i8_to_bf16x8(q.z, q.w) : i8_to_bf16x8(q.x, q.y);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x0[s]), as_bf16x8(wb), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x1[s]), as_bf16x8(wb), c1, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(l0[s]), as_bf16x8(wb), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(l1[s]), as_bf16x8(wb), c1, 0, 0, 0);
    }
  }
  static constexpr int WELT = 1;
};

template <>
struct GemmCore<float> {
  uint4 w[8], x0[8], x1[8];  // 32 floats each
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx, int woff, int xoff0,
                                       int xoff1, int kleft, int) {
#pragma unroll
    for (int s = 0; s < 8; ++s) w[s] = buf_ld16(rw, (woff < 0 || 4 * s >= kleft) ? BUF_OOB : woff + 16 * s);
#pragma unroll
    for (int s = 0; s < 8; ++s) x0[s] = buf_ld16(rx, (xoff0 < 0 || 4 * s >= kleft) ? BUF_OOB : xoff0 + 16 * s);
#pragma unroll
    for (int s = 0; s < 8; ++s) x1[s] = buf_ld16(rx, (xoff1 < 0 || 4 * s >= kleft) ? BUF_OOB : xoff1 + 16 * s);
  }
  __device__ __forceinline__ void mma(f32x16 &c0, f32x16 &c1) const {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t wv[4] = {w[s].x, w[s].y, w[s].z, w[s].w};
      const uint32_t a0[4] = {x0[s].x, x0[s].y, x0[s].z, x0[s].w};
      const uint32_t a1[4] = {x1[s].x, x1[s].y, x1[s].z, x1[s].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a0[e]), __uint_as_float(wv[e]), c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a1[e]), __uint_as_float(wv[e]), c1, 0, 0, 0);
      }
    }
  }
  static constexpr int WELT = 4;
};

// Y[m][n] (ADD: +=) sum_k X[m][k] W[n][k] (* wscale[n]) for m < M, n < N.  Grid (ceil(N / 32),
// ceil(M / 64)), GBLOCK threads.  X: [M][ldx] elements of GemmX<WT>::type in the XPut layout
// (bf16: hi and lo planes of K columns each); Y: [M][ldy] floats.  The byte sizes of W and of X
// must stay below 2^31.
template <typename WT, bool ADD, int TAG>
__global__ __launch_bounds__(GBLOCK) void k_gemm(const WT *__restrict__ W, const float *__restrict__ wscale, int N,
                                                 int K, const typename GemmX<WT>::type *__restrict__ X, int ldx,
                                                 int M, float *__restrict__ Y, int ldy) {
  typedef typename GemmX<WT>::type XT;
  constexpr int XE = (int)sizeof(XT);
  constexpr int WE = GemmCore<WT>::WELT;
  __shared__ float red[GWAVES][GM * GN];  // 32 KB: each wave's partial tile
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n0 = blockIdx.x * GN, m0 = blockIdx.y * GM;
  const int ln = lane & 31, g = lane >> 5;
  const int n = n0 + ln, ma = m0 + ln, mb = m0 + 32 + ln;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void *)W, (short)0, (int)((size_t)N * K * WE), BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void *)X, (short)0, (int)((size_t)M * ldx * XE), BUF_DWORD3);
  // this wave's K blocks: a balanced share of the ceil(K / 64) blocks
  const int nkb = (K + GKB - 1) / GKB;
  const int kb0 = (wave * nkb) / GWAVES, kb1 = ((wave + 1) * nkb) / GWAVES;
  f32x16 c0 = {}, c1 = {};
  GemmCore<WT> pa, pb;  // K blocks kb (pa) and kb + 1 (pb) in flight
  auto fetch = [&](GemmCore<WT> &c, int kb) {
    const int k = kb * GKB + 32 * g;  // first of this lane's 32 columns; 16-byte pieces past K read zero
    const bool kin = kb < kb1 && k < K;
    const int wo = (kin && n < N) ? (int)(((size_t)n * K + k) * WE) : -1;
    const int xa = (kin && ma < M) ? (int)(((size_t)ma * ldx + k) * XE) : -1;
    const int xb = (kin && mb < M) ? (int)(((size_t)mb * ldx + k) * XE) : -1;
    c.load(rw, rx, wo, xa, xb, K - k, K * XE);
  };
  // Both buffers are refilled unconditionally (past kb1 with out-of-range loads that read zero
  // and move no data), so no load sits under a branch and the waits stay per buffer.
  fetch(pa, kb0);
  fetch(pb, kb0 + 1);
  // The scheduling barriers keep each refill ahead of the next buffer's wait: without them the
  // compiler sinks the refill below that wait and only one buffer is ever in flight.
  for (int kb = kb0; kb < kb1; kb += 2) {
    pa.mma(c0, c1);
    fetch(pa, kb + 2);
    __builtin_amdgcn_sched_barrier(0);
    pb.mma(c0, c1);
    fetch(pb, kb + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  // partial tiles to LDS: element i of lane l is row (i / 4) * 8 + g * 4 + (i % 4), column ln
  float *rp = red[wave];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = (i >> 2) * 8 + g * 4 + (i & 3);
    rp[r * GN + ln] = c0[i];
    rp[(32 + r) * GN + ln] = c1[i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < GM * GN; e += GBLOCK) {
    const int r = e / GN, cidx = e % GN;
    const int m = m0 + r, nn = n0 + cidx;
    if (m >= M || nn >= N) continue;
    float v = red[0][e];
#pragma unroll
    for (int w2 = 1; w2 < GWAVES; ++w2) v += red[w2][e];
    if (wscale) v *= wscale[nn];
    float *yp = Y + (size_t)m * ldy + nn;
    if (ADD)
      *yp += v;
    else
      *yp = v;
  }
}

}  // namespace mk
