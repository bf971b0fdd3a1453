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


// ---- wide tiles, both operands streamed through an LDS ring -------------------------------------
// For bf16 and int8 weights.  A block owns 128 NT weight rows (32 NT per wave, NT = 1 or 2) and
// XM = 64 activation rows; its waves do not split K.  Every K block (64 columns) of both operands goes
// straight from memory into one stage of a ring of LDS stages with LDS-direct loads (no
// registers), as many K blocks ahead of the multiply as the LDS holds stages, minus one.  The
// activation tile (hi and lo planes) is loaded once per block and read by all four waves (tiles
// that split K over waves reload it per wave), and every activation fragment a wave reads from LDS
// feeds the products of its NT 32-row weight tiles (two tiles halve the LDS reads per product but
// halve the number of blocks: the host takes them for wide projections).  Each 1 KB load fills whole 128-byte row segments (8 rows of a 64-column bf16 block, or
// 16 rows of int8), so every cache line is fetched by one instruction; within a row the 16-byte
// pieces are stored XOR-swizzled by the row (xswz), so the matrix-core fragment reads (lane l:
// row l % 32, pieces of columns 32 (l / 32) ..) hit distinct banks.
// A grid z dimension splits K: every split writes its partial tile to `part` ([split][M][N]
// floats) and k_gemm_reduce adds the splits in order, so the result does not depend on timing.
constexpr int XNMAX = 2;                // most 32-row weight tiles per wave
constexpr int XM = 64;                  // activation rows per block
constexpr int XKB = 64;                 // K block
constexpr int XLDS = 160 * 1024;        // the LDS of a CU: the ring takes as many stages as fit

// Weight chunks per 32 weight rows and K block: bf16 4 (8 bf16 per lane), int8 2 (16 int8 per
// lane); PER elements per 16-byte piece, PPR pieces per 64-column row, RPC rows per 1 KB chunk.
template <typename WT> struct XWC;
template <> struct XWC<bf16_t> { static constexpr int N = 4, ELT = 2, PER = 8, PPR = 8, RPC = 8; };
template <> struct XWC<int8_t> { static constexpr int N = 2, ELT = 1, PER = 16, PPR = 4, RPC = 16; };

// The LDS serves a 16-byte read of 16 lanes per cycle from 64 banks (256 bytes), so the 16 rows a
// fragment read touches must land on 16 distinct 16-byte slots of the 256-byte bank window.  A row
// of PPR pieces spans 16 PPR bytes: 16 / PPR rows share a window position, and piece p of row r is
// stored at slot p ^ ((r / (16 / PPR)) % PPR).
template <int PPR> __device__ __forceinline__ int xswz(int r) { return (r / (16 / PPR)) % PPR; }

// s_waitcnt immediate that waits until at most n vector memory operations are outstanding
// (expcnt and lgkmcnt left at their maxima: no wait on them).
constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw 32-bit buffer descriptor of `bytes` bytes at base (loads past the end read zero).
__device__ __forceinline__ i32x4 raw_desc(const void *base, int bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)(a >> 32) & 0xFFFF),
               __builtin_amdgcn_readfirstlane(bytes), BUF_DWORD3};
}

// LDS-direct load: lane l's 16 bytes at byte offset voff of the buffer go to the LDS byte address
// lds + 16 l (lds wave-uniform, a scalar).  Issued from inline assembly so that the compiler does
// not track it: it would otherwise wait for every such load before the next LDS read.  The caller
// waits for it with an explicit s_waitcnt (a wave's vector memory operations complete in issue
// order).
__device__ __forceinline__ void lds_load16_at(i32x4 desc, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(desc)
               : "memory", "m0");
}

// Y[m][n] (ADD: +=) sum_k X[m][k] W[n][k] (* wscale[n]), or with gridDim.z > 1 the partial sums of
// K blocks [z * kbs, (z + 1) * kbs) into part[z][m][n].  Grid (ceil(N / (128 NT)), ceil(M / XM), splits),
// GBLOCK threads.  X: [M][ldx] bf16 in the hi | lo layout (planes K apart); K a multiple of 16.
template <typename WT, bool ADD, int TAG, int XNT>
__global__ __launch_bounds__(GBLOCK) void k_gemm_x(const WT *__restrict__ W, const float *__restrict__ wscale, int N,
                                                   int K, const bf16_t *__restrict__ X, int ldx, int M,
                                                   float *__restrict__ Y, int ldy, float *__restrict__ part, int kbs) {
  constexpr int WC = XWC<WT>::N * XNT, WE = XWC<WT>::ELT;  // weight chunks per wave
  constexpr int XCH = 16;                      // activation chunks per stage: [plane][8-row group]
  constexpr int NCH = XCH + GWAVES * WC;       // chunks per stage
  constexpr int NL = XCH / GWAVES + WC;        // loads each wave issues per K block
  constexpr int XST = XLDS / (NCH * WAVE * 16);  // stages (bf16: 3 x 48 KB, int8: 5 x 32 KB)
  static_assert(XST >= 3, "the ring needs at least three stages");
  __shared__ __align__(16) uint4 ring[XST][NCH * WAVE];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n0 = blockIdx.x * (GWAVES * 32 * XNT), m0 = blockIdx.y * XM;
  const int ln = lane & 31, g = lane >> 5;
  const int nw = n0 + wave * 32 * XNT;  // the wave's first weight row
  const i32x4 rw = raw_desc(W, (int)((size_t)N * K * WE));
  const i32x4 rx = raw_desc(X, (int)((size_t)M * ldx * 2));
  const int nkb = (K + XKB - 1) / XKB;
  const int kb0 = blockIdx.z * kbs, kb1 = min(nkb, kb0 + kbs);
  constexpr int PER = XWC<WT>::PER, PPR = XWC<WT>::PPR, RPC = XWC<WT>::RPC;
  // this wave's activation chunks c = 4 wave + i: plane c / 8, rows 8 (c % 8) .. + 8 of the tile;
  // lane l fills slot l % 8 of row 8 (c % 8) + l / 8 with piece (l % 8) ^ (row % 8)
  int xo[XCH / GWAVES], xcol[XCH / GWAVES];
#pragma unroll
  for (int i = 0; i < XCH / GWAVES; ++i) {
    const int c = GWAVES * wave + i;
    const int pl = c >> 3, r = 8 * (c & 7) + (lane >> 3);
    const int m = m0 + r;
    xcol[i] = 8 * ((lane & 7) ^ xswz<8>(r));
    xo[i] = m < M ? (int)(((size_t)m * ldx + (size_t)pl * K + xcol[i]) * 2) : -1;
  }
  // this wave's weight chunks c: rows RPC c .. + RPC of its 32 XNT; lane l fills slot l % PPR of
  // row RPC c + l / PPR with piece (l % PPR) ^ (row % PPR)
  int wo[WC], wcol[WC];
#pragma unroll
  for (int c = 0; c < WC; ++c) {
    const int rr = RPC * c + lane / PPR;
    const int nr = nw + rr;
    wcol[c] = PER * ((lane % PPR) ^ xswz<PPR>(rr));
    wo[c] = nr < N ? (int)(((size_t)nr * K + wcol[c]) * WE) : -1;
  }
  // K block kb into a stage (past kb1 or K: out-of-range loads, which read zero and move no data,
  // so every wave issues the same count and the waits below stay exact)
  // LDS byte address of the ring: stage s, chunk c at ring0 + ((s NCH + c) WAVE) 16
  const uint32_t ring0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)&ring[0][0]);
  auto issue = [&](int stage, int kb) {
    const int k = kb * XKB;
    const bool in = kb < kb1;
    const uint32_t sb = ring0 + (uint32_t)(stage * NCH * WAVE * 16);
#pragma unroll
    for (int i = 0; i < XCH / GWAVES; ++i) {
      const int off = (in && xo[i] >= 0 && k + xcol[i] < K) ? xo[i] + k * 2 : BUF_OOB;
      lds_load16_at(rx, sb + (uint32_t)((GWAVES * wave + i) * WAVE * 16), off);
    }
#pragma unroll
    for (int c = 0; c < WC; ++c) {
      const int off = (in && wo[c] >= 0 && k + wcol[c] < K) ? wo[c] + k * WE : BUF_OOB;
      lds_load16_at(rw, sb + (uint32_t)((XCH + wave * WC + c) * WAVE * 16), off);
    }
  };
  f32x16 acc[XNT][2] = {};  // [weight tile][activation tile]
  auto compute = [&](const uint4 *stg) {
    // all of this K block's fragments first (one wave per SIMD: nothing else hides LDS latency)
    // weight pieces 4 g + s (bf16) or 2 g + t (int8) of row 32 t + l % 32; activation piece
    // 4 g + s of row 32 tile + l % 32 in plane 0 (hi) and 1 (lo)
    constexpr int WCT = XWC<WT>::N;  // weight chunks per 32 rows
    uint4 wq[XNT][WCT], xf[16];
    const uint4 *wst = stg + (XCH + wave * WC) * WAVE;
#pragma unroll
    for (int t = 0; t < XNT; ++t)
#pragma unroll
      for (int c = 0; c < WCT; ++c) {
        const int pi = WCT * g + c, r = 32 * t + ln;
        wq[t][c] = wst[(r / RPC) * WAVE + (r % RPC) * PPR + (pi ^ xswz<PPR>(r))];
      }
#pragma unroll
    for (int stp = 0; stp < 4; ++stp)
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // j: (plane, m tile) = (j / 2, j % 2)
        const int pl = j >> 1, r = 32 * (j & 1) + ln;
        xf[4 * stp + j] = stg[(pl * 8 + (r >> 3)) * WAVE + (r & 7) * 8 + ((4 * g + stp) ^ xswz<8>(r))];
      }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the multiplies
#pragma unroll
    for (int stp = 0; stp < 4; ++stp)
#pragma unroll
      for (int t = 0; t < XNT; ++t) {
        uint4 wv;
        if constexpr (WCT == 4) {
          wv = wq[t][stp];
        } else {
          const uint4 &q = wq[t][stp >> 1];
          wv = (stp & 1) ? i8_to_bf16x8(q.z, q.w) : i8_to_bf16x8(q.x, q.y);
        }
        const bf16x8 wb = as_bf16x8(wv);
        f32x16 &a0 = acc[t][0], &a1 = acc[t][1];
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xf[4 * stp + 0]), wb, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xf[4 * stp + 1]), wb, a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xf[4 * stp + 2]), wb, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xf[4 * stp + 3]), wb, a1, 0, 0, 0);
      }
  };
  // Barrier without a memory fence: a fenced barrier would wait for every LDS-direct load in
  // flight.  Each wave first waits for its own loads of the stage about to be read (the oldest
  // NL of the (XST - 1) NL it has in flight); after the barrier every wave's copies of it are in
  // LDS, and every wave is done reading the stage the next issue overwrites.
  auto sync = [&] {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm((XST - 2) * NL));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
#pragma unroll
  for (int i = 0; i < XST - 1; ++i) issue(i, kb0 + i);
  int cur = 0;  // stage of K block kb
  for (int kb = kb0; kb < kb1; ++kb) {
    sync();
    issue(cur == 0 ? XST - 1 : cur - 1, kb + XST - 1);
    compute(ring[cur]);
    cur = cur == XST - 1 ? 0 : cur + 1;
  }
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));  // no copy may still be writing LDS at exit
  // element i of lane l in acc[t][h]: activation row (i / 4) * 8 + g * 4 + (i % 4) + 32 h,
  // weight row nw + 32 t + l % 32
#pragma unroll
  for (int t = 0; t < XNT; ++t) {
    const int n = nw + 32 * t + ln;
    if (n >= N) continue;
    const float sc = (wscale && gridDim.z == 1) ? wscale[n] : 1.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = (i >> 2) * 8 + g * 4 + (i & 3);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = m0 + r + 32 * h;
        if (m >= M) continue;
        const float v = acc[t][h][i];
        if (gridDim.z > 1) {
          part[((size_t)blockIdx.z * M + m) * N + n] = v;
        } else {
          float *yp = Y + (size_t)m * ldy + n;
          if (ADD)
            *yp += v * sc;
          else
            *yp = v * sc;
        }
      }
    }
  }
}

// ---- many activation rows (the prefill's chunks): 128 x 256 tiles ------------------------------
// The same product for M > XM.  With 64-row activation tiles every weight tile is read once per
// 64 rows, and the re-reads bound the projection (at M = 1024 gate_in moves 4.4 GB for 189 GFLOP).
// Here a block owns BM = 128 activation rows and 256 weight rows and its four waves split both
// (2 x 2: 64 rows x 128 weight rows each, 8 accumulator tiles); a K block is 32 columns, so that a
// stage (the activation tile's hi and lo planes, 16 KB, and the weight tile, 16 KB for bf16 or 8 KB
// for int8) leaves room for 5 (6) stages in LDS.  (A block of 256 rows halves the weight re-reads
// but leaves 3 stages and 1.4 rounds of blocks over the CUs at 1024 rows: slower.)  Loads, the LDS-direct ring and the waits are those of
// k_gemm_x.  A row segment of a stage is 64 bytes (bf16: 4 pieces of 8 columns; int8 weights: 32
// bytes, 2 pieces of 16) and its pieces are swizzled with xswz.  MFMA step s of a K block takes, in
// lane half g, columns 16 g + 8 s .. + 7 of both operands.  The grid walks the activation tiles
// fastest, so the blocks that read one weight tile run together.
constexpr int XLM = 128;  // activation rows per block
constexpr int XLN = 256;  // weight rows per block
constexpr int XLK = 32;   // K block

template <typename WT> struct XLW;
template <> struct XLW<bf16_t> { static constexpr int ELT = 2, PPR = 4, RPC = 16, PER = 8, CH = 16; };
template <> struct XLW<int8_t> { static constexpr int ELT = 1, PPR = 2, RPC = 32, PER = 16, CH = 8; };

// The dispatcher hands workgroups to the 8 XCDs in turn (linear block b to XCD b % 8), and each XCD
// has its own L2.  Renumbered so that each XCD runs one contiguous range of tiles, M fastest, the
// blocks that run together on an XCD share weight and activation tiles in its L2 instead of each
// fetching its own weight tile through the fabric.
constexpr int XCDS = 8;
__device__ __forceinline__ void xcd_tile(int &bx, int &by, int &bz) {
  const int nx = gridDim.x, ny = gridDim.y, n = nx * ny * gridDim.z;
  const int b = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int per = n / XCDS, rem = n % XCDS, x = b % XCDS, i = b / XCDS;
  const int l = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
  bx = l % nx;
  by = (l / nx) % ny;
  bz = l / (nx * ny);
}

// GATE (the gated unit's first product, one split): the epilogue writes
// gx[m][j] = silu(y[m][2j]) * y[m][2j + 1] in the XPut layout (row stride ldg, F = N / 2 columns)
// in place of Y.  The block's product tile goes through the LDS of the ring (free once the K loop
// is done), so the pairs are read as float2 and the outputs stored row by row.
template <typename WT, bool ADD, int TAG, bool GATE = false>
__global__ __launch_bounds__(GBLOCK) void k_gemm_xl(const WT *__restrict__ W, const float *__restrict__ wscale, int N,
                                                    int K, const bf16_t *__restrict__ X, int ldx, int M,
                                                    float *__restrict__ Y, int ldy, float *__restrict__ part, int kbs,
                                                    bf16_t *__restrict__ gx = nullptr, int ldg = 0) {
  constexpr int WE = XLW<WT>::ELT, PPR = XLW<WT>::PPR, RPC = XLW<WT>::RPC, PER = XLW<WT>::PER;
  constexpr int WCH = XLW<WT>::CH;   // weight chunks per stage
  constexpr int BM = XLM;
  constexpr int XG = BM / 16;        // 16-row groups of the activation tile
  constexpr int XCH = 2 * XG;        // activation chunks per stage: [plane][16-row group]
  constexpr int MT = BM / 64;        // 32-row activation tiles per wave
  constexpr int NCH = XCH + WCH;
  constexpr int NL = NCH / GWAVES;   // loads each wave issues per K block
  constexpr int XST = XLDS / (NCH * WAVE * 16);
  static_assert(NCH % GWAVES == 0 && XST >= 3, "stage shape");
  __shared__ __align__(16) uint4 ring[XST][NCH * WAVE];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave & 1, wn = wave >> 1;
  int bx, by, bz;
  xcd_tile(bx, by, bz);
  const int m0 = bx * BM, n0 = by * XLN;
  const int ln = lane & 31, g = lane >> 5;
  const i32x4 rw = raw_desc(W, (int)((size_t)N * K * WE));
  const i32x4 rx = raw_desc(X, (int)((size_t)M * ldx * 2));
  const int nkb = (K + XLK - 1) / XLK;
  const int kb0 = bz * kbs, kb1 = min(nkb, kb0 + kbs);
  // the NL chunks this wave loads: chunk c = wave + GWAVES i (activations first, then weights)
  int off0[NL], col0[NL];
  bool isx[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int c = wave + GWAVES * i;
    if (c < XCH) {  // activations: plane c / XG, rows 16 (c % XG) + lane / 4, 4 pieces of 8 columns
      const int pl = c / XG, r = 16 * (c % XG) + (lane >> 2);
      const int m = m0 + r;
      col0[i] = 8 * ((lane & 3) ^ xswz<4>(r));
      off0[i] = m < M ? (int)(((size_t)m * ldx + (size_t)pl * K + col0[i]) * 2) : -1;
      isx[i] = true;
    } else {  // weights: rows RPC (c - XCH) + lane / PPR
      const int r = RPC * (c - XCH) + lane / PPR;
      const int n = n0 + r;
      col0[i] = PER * ((lane % PPR) ^ xswz<PPR>(r));
      off0[i] = n < N ? (int)(((size_t)n * K + col0[i]) * WE) : -1;
      isx[i] = false;
    }
  }
  // A K block is two MFMA steps of 16 columns, and the loop is pipelined by steps: a step's
  // fragments are read from LDS while the previous step's products run, and the barrier that
  // publishes the next stage sits between the two steps, where the step-1 fragments are already in
  // registers.  Each phase interleaves its memory instructions one by one with the products.
  f32x16 acc[MT][4] = {};  // [m tile][n tile] of this wave
  constexpr int NRD = 2 * MT + 4;  // fragment reads per step
  uint4 fr[2][NRD];                // [step][activation (m tile, plane) ..., weights (n tile) ...]
  auto rd = [&](const uint4 *stg, int st, int j) {  // fragment read j of step st
    if (j < 2 * MT) {
      const int mt = j >> 1, pl = j & 1;
      const int r = (BM / 2) * wm + 32 * mt + ln;  // block row
      fr[st][j] = stg[(pl * XG + (r >> 4)) * WAVE + (r & 15) * 4 + ((2 * g + st) ^ xswz<4>(r))];
    } else {
      const int t = j - 2 * MT;
      const int r = 128 * wn + 32 * t + ln;  // block weight row
      const uint4 *wst = stg + XCH * WAVE;
      // int8: one piece holds the 32 weights of both steps; each step reads it for itself
      const int pc = PPR == 4 ? 2 * g + st : g;
      fr[st][j] = wst[(r / RPC) * WAVE + (r % RPC) * PPR + (pc ^ xswz<PPR>(r))];
    }
  };
  // product j of a step: plane j / (4 MT) (hi products first, then lo), n tile (j / MT) % 4, m tile j % MT
  auto mma = [&](int st, int j) {
    const int pl = j / (4 * MT), t = (j / MT) % 4, mt = j % MT;
    uint4 wv = fr[st][2 * MT + t];
    if constexpr (PPR != 4) wv = st ? i8_to_bf16x8(wv.z, wv.w) : i8_to_bf16x8(wv.x, wv.y);
    acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[st][2 * mt + pl]), as_bf16x8(wv), acc[mt][t], 0, 0, 0);
  };
  constexpr int NMM = 8 * MT;  // products per step
  static_assert(NMM >= NRD && NMM >= NRD + NL, "a phase spreads its memory instructions over its products");
  // LDS byte address of the ring; stage s, chunk c sits at ring0 + ((s NCH + c) WAVE) 16
  const uint32_t ring0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)&ring[0][0]);
  auto issue1 = [&](int stage, int kb, int i) {
    const int c = wave + GWAVES * i;
    const int k = kb * XLK;
    const int off = (kb < kb1 && off0[i] >= 0 && k + col0[i] < K) ? off0[i] + k * (isx[i] ? 2 : WE) : BUF_OOB;
    lds_load16_at(isx[i] ? rx : rw, ring0 + (uint32_t)((stage * NCH + c) * WAVE * 16), off);
  };
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // prologue: stages for the first XST - 1 K blocks in flight, then the first block's step-0 reads
#pragma unroll
  for (int i = 0; i < XST - 1; ++i)
#pragma unroll
    for (int l = 0; l < NL; ++l) issue1(i, kb0 + i, l);
  __builtin_amdgcn_s_waitcnt(vm_wait_imm((XST - 2) * NL));
  barrier();
#pragma unroll
  for (int j = 0; j < NRD; ++j) rd(ring[0], 0, j);
  int cur = 0;
  for (int kb = kb0; kb < kb1; ++kb) {
    const int nxt = cur == XST - 1 ? 0 : cur + 1, prv = cur == 0 ? XST - 1 : cur - 1;
    // phase A: step-0 products, step-1 reads of this block
#pragma unroll
    for (int j = 0; j < NMM; ++j) {
      mma(0, j);
      if (j < NRD) rd(ring[cur], 1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next block's stage has landed (the loads of the XST - 3 blocks after it may still be in
    // flight), and every wave is done with the previous block's stage, which the loads below refill
    __builtin_amdgcn_s_waitcnt(vm_wait_imm((XST - 3) * NL));
    barrier();
    // phase B: step-1 products; the loads of block kb + XST - 1 and the next block's step-0 reads
#pragma unroll
    for (int j = 0; j < NMM; ++j) {
      mma(1, j);
      if (j < NL) issue1(prv, kb + XST - 1, j);
      else if (j < NL + NRD) rd(ring[nxt], 0, j - NL);
      __builtin_amdgcn_sched_barrier(0);
    }
    cur = nxt;
  }
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));  // no copy may still be writing LDS at exit
  static_assert(!GATE || sizeof(ring) >= (size_t)BM * XLN * 4, "the product tile fits the ring");
  float *gtile = reinterpret_cast<float *>(&ring[0][0]);  // GATE: [BM][XLN] products
  if (GATE) __syncthreads();  // every wave's fragment reads of the last stage are done
  // element i of lane l in acc[mt][t]: activation row (BM / 2) wm + 32 mt + (i / 4) * 8 + g * 4 +
  // (i % 4), weight row 128 wn + 32 t + l % 32
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n0 + 128 * wn + 32 * t + ln;
    if (n >= N) continue;
    const float sc = (wscale && gridDim.z == 1) ? wscale[n] : 1.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + (BM / 2) * wm + 32 * mt + (i >> 2) * 8 + g * 4 + (i & 3);
        if (m >= M) continue;
        const float v = acc[mt][t][i];
        if (GATE) {
          gtile[(m - m0) * XLN + (n - n0)] = v * sc;
        } else if (gridDim.z > 1) {
          part[((size_t)bz * M + m) * N + n] = v;
        } else {
          float *yp = Y + (size_t)m * ldy + n;
          if (ADD)
            *yp += v * sc;
          else
            *yp = v * sc;
        }
      }
  }
  if (GATE) {
    __syncthreads();
    const float2 *t2 = reinterpret_cast<const float2 *>(gtile);
    for (int e = threadIdx.x; e < BM * (XLN / 2); e += GBLOCK) {
      const int r = e / (XLN / 2), jj = e - r * (XLN / 2);
      const int m = m0 + r, n = n0 + 2 * jj;
      if (m < M && n < N) {
        const float2 gm = t2[e];
        XPut<bf16_t>::put(gx + (size_t)m * ldg, N >> 1, n >> 1, silu(gm.x) * gm.y);
      }
    }
  }
}

// Sum over the splits, in order, of part[s][m][c .. c + 4) (the loads of up to 8 splits in flight).
__device__ __forceinline__ float4 split_sum4(const float *__restrict__ part, int S, int M, int N, int m, int c) {
  float4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    float4 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      p[u] = s0 + u < S ? *reinterpret_cast<const float4 *>(part + ((size_t)(s0 + u) * M + m) * N + c)
                        : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v.x += p[u].x;
      v.y += p[u].y;
      v.z += p[u].z;
      v.w += p[u].w;
    }
  }
  return v;
}

// Y[m][n] (ADD: +=) (sum over the splits in order of part[s][m][n]) * wscale[n], four columns per
// thread (when N is a multiple of 4 the partial rows are 16-byte aligned and read as float4;
// otherwise one column at a time).  Grid (ceil(N / (4 BLOCK)), M).
template <bool ADD>
__global__ __launch_bounds__(BLOCK) void k_gemm_reduce(const float *__restrict__ part, int S, int M, int N,
                                                       const float *__restrict__ wscale, float *__restrict__ Y,
                                                       int ldy) {
  const int c = 4 * (blockIdx.x * BLOCK + threadIdx.x), m = blockIdx.y;
  if (c >= N) return;
  float r[4] = {0.f, 0.f, 0.f, 0.f};
  const int ne = min(4, N - c);
  if ((N & 3) == 0) {
    const float4 v = split_sum4(part, S, M, N, m, c);
    r[0] = v.x;
    r[1] = v.y;
    r[2] = v.z;
    r[3] = v.w;
  } else {
    for (int s = 0; s < S; ++s)
      for (int e = 0; e < ne; ++e) r[e] += part[((size_t)s * M + m) * N + c + e];
  }
  float *yp = Y + (size_t)m * ldy + c;
  for (int e = 0; e < ne; ++e) {
    if (wscale) r[e] *= wscale[c + e];
    if (ADD)
      yp[e] += r[e];
    else
      yp[e] = r[e];
  }
}

}  // namespace mk
