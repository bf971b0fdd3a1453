// Row-batched frame path: the frame of several conversations (one activation row per
// conversation) and the teacher-forced prefill of one conversation (one row per position) run
// their projections on the matrix cores (gemm.h).  The kernels here are the steps around those
// products, one block per activation row unless stated: the norm and bf16 rounding of a
// projection's input, rope and the KV append, the gated-unit product, the argmax of a head, the
// depformer entry and attention ([LM]: the docs.rs page "inferencelayer 0.2.4 src/moshi_lm.rs").
#pragma once
#include "gemm.h"
#include "kernels.h"

namespace mk {

// Which conversation and absolute position an activation row stands for.  In a frame, row m is
// conversation b0 + m at its own offset; in a prefill every row belongs to conversation `conv`,
// at consecutive positions pos0 + m.
struct RowMap {
  int conv;  // < 0: frame
  int b0;
  int64_t pos0;
  __device__ __forceinline__ int conv_of(int m) const { return conv < 0 ? b0 + m : conv; }
  __device__ __forceinline__ int64_t pos_of(const Bufs &s, int m) const {
    return conv < 0 ? s.offset[b0 + m] : pos0 + m;
  }
};

// X[m] = rms_norm(src[m]; alpha) (or src[m] when alpha is null) in the XPut layout; with `copy` set
// the float32 result also goes to copy[m] (the post-out_norm hidden).  Dynamic LDS: K floats.
template <typename XT>
__global__ __launch_bounds__(BLOCK) void k_rows_cvt(const float *__restrict__ src, int lds,
                                                    const float *__restrict__ alpha, float eps, int K,
                                                    XT *__restrict__ X, int ldx, float *__restrict__ copy, int ldc) {
  extern __shared__ float xs[];
  __shared__ float red[NWAVES];
  const int m = blockIdx.x;
  if (alpha)
    stage_rms(src + (size_t)m * lds, alpha, K, eps, xs, red);
  else
    stage_vec(src + (size_t)m * lds, K, xs);
  for (int k = threadIdx.x; k < K; k += BLOCK) {
    XPut<XT>::put(X + (size_t)m * ldx, K, k, xs[k]);
    if (copy) copy[(size_t)m * ldc + k] = xs[k];
  }
}

// Residual projection epilogue fused with the next input conversion: Y[m] += (sum over the splits,
// in order, of part[s][m]) * wscale, then X[m] = rms_norm(Y[m]; alpha) (or Y[m] when alpha is null)
// in the XPut layout -- the split reduction of k_gemm_x and k_rows_cvt in one launch.  One block
// of ADD_BLOCK threads per row, four columns per thread and pass (N a multiple of 4), the loads of
// up to 8 splits in flight at once.  Grid (M), dynamic LDS: N floats.
constexpr int ADD_BLOCK = 1024;
template <typename XT>
__global__ __launch_bounds__(ADD_BLOCK) void k_add_rows_cvt(const float *__restrict__ part, int S, int M, int N,
                                                            const float *__restrict__ wscale, float *__restrict__ Y,
                                                            int ldy, const float *__restrict__ alpha, float eps,
                                                            XT *__restrict__ X, int ldx) {
  extern __shared__ float xs[];
  __shared__ float red[ADD_BLOCK / WAVE];
  const int m = blockIdx.x;
  float ss = 0.f;
  for (int c = 4 * threadIdx.x; c < N; c += 4 * ADD_BLOCK) {
    float *yp = Y + (size_t)m * ldy + c;
    const float4 y = *reinterpret_cast<const float4 *>(yp);  // in flight with the partials below
    float4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 8) {
      float4 p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        p[u] = s0 + u < S ? *reinterpret_cast<const float4 *>(part + ((size_t)(s0 + u) * M + m) * N + c)
                          : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // in split order
        v.x += p[u].x;
        v.y += p[u].y;
        v.z += p[u].z;
        v.w += p[u].w;
      }
    }
    float xn[4] = {v.x, v.y, v.z, v.w};
    const float yv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (wscale) xn[e] *= wscale[c + e];
      xn[e] = yv[e] + xn[e];
      xs[c + e] = xn[e];
      ss = fmaf(xn[e], xn[e], ss);
    }
    *reinterpret_cast<float4 *>(yp) = float4{xn[0], xn[1], xn[2], xn[3]};
  }
  float inv = 1.f;
  if (alpha) {
    const float tot = block_sum<ADD_BLOCK>(ss, red);
    inv = 1.0f / sqrtf(eps + tot / (float)N);
  }
  for (int c = 4 * threadIdx.x; c < N; c += 4 * ADD_BLOCK)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      XPut<XT>::put(X + (size_t)m * ldx, N, c + e, alpha ? (xs[c + e] * alpha[c + e]) * inv : xs[c + e]);
}

// a4.1 after the fused q|k|v product, one block per (head h, row m).  The head's q, k and v
// columns (c = part * D + h * hd + e) are the sum over the S splits, in order, of
// part[s][m][c] (row length 3 D), times the int8 row scales when wscale is set; with S = 1 and no
// scales `part` is the product itself.  Then interleaved rope on q and k at the row's position
// (angle f_i * pos in float32, sin / cos in double), q to q_out[m], k and v to the row's
// conversation's KV slot pos % cap of `layer` ([LM] temporal_step, rope_row).  Four columns (two
// rope pairs) per thread.  Grid (H, rows).
constexpr int QKV_BLOCK = 128;
template <typename KT>
__global__ __launch_bounds__(QKV_BLOCK) void k_qkv_post(Dims d, Bufs s, KV<KT> kv, const float *__restrict__ part,
                                                        int S, int M, const float *__restrict__ wscale,
                                                        float *__restrict__ q_out, int layer, RowMap rm) {
  __shared__ float rcs[256];  // cos, sin of pair i at [2i], [2i + 1] (head dim <= 256)
  const int h = blockIdx.x, m = blockIdx.y;
  const int conv = rm.conv_of(m);
  const int64_t pos = rm.pos_of(s, m);
  const int slot = (int)(pos % d.cap);
  for (int i = threadIdx.x; i < d.hd / 2; i += QKV_BLOCK) {
    const float ang = s.rope_freq[i] * (float)pos;
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    rcs[2 * i] = (float)cd;
    rcs[2 * i + 1] = (float)sd;
  }
  __syncthreads();
  const int N = 3 * d.D, per = d.hd / 4;
  for (int t = threadIdx.x; t < 3 * per; t += QKV_BLOCK) {
    const int pt = t / per, e = 4 * (t - pt * per);  // 0 q, 1 k, 2 v; element of the head
    const int c = pt * d.D + h * d.hd + e;
    const float4 v4 = split_sum4(part, S, M, N, m, c);
    float r[4] = {v4.x, v4.y, v4.z, v4.w};
    if (wscale) {
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] *= wscale[c + k];
    }
    if (pt < 2) {
#pragma unroll
      for (int k = 0; k < 4; k += 2) {
        const float cs = rcs[e + k], sn = rcs[e + k + 1];
        const float a0 = r[k] * cs - r[k + 1] * sn;
        const float a1 = r[k] * sn + r[k + 1] * cs;
        r[k] = a0;
        r[k + 1] = a1;
      }
    }
    if (pt == 0) {
      *reinterpret_cast<float4 *>(q_out + (size_t)m * d.D + h * d.hd + e) = float4{r[0], r[1], r[2], r[3]};
    } else {
      KT *cache = pt == 1 ? kv.k : kv.v;
      const size_t idx = kv_index(d, conv, layer, slot, h, e);
#pragma unroll
      for (int k = 0; k < 4; ++k) cache[idx + k] = from_f<KT>(r[k]);
    }
  }
}

// a5 between the two gated-unit products: X[m][j] = silu(Y[m][2j]) * Y[m][2j + 1] (the device
// copy of linear_in has gate row j and mult row j interleaved), in the XPut layout.  Grid
// (rows, ceil(F / BLOCK)).
template <typename XT>
__global__ __launch_bounds__(BLOCK) void k_gate_post(const float *__restrict__ Y, int ldy, int F, XT *__restrict__ X,
                                                     int ldx) {
  const int m = blockIdx.x;
  const int j = blockIdx.y * BLOCK + threadIdx.x;
  if (j >= F) return;
  const float2 gm = *reinterpret_cast<const float2 *>(Y + (size_t)m * ldy + 2 * j);
  XPut<XT>::put(X + (size_t)m * ldx, F, j, silu(gm.x) * gm.y);
}

// The gated unit's split reduction fused with its epilogue: the sum over the splits of the
// interleaved gate / mult columns 2j, 2j + 1 (times their int8 row scales), then
// X[m][j] = silu(gate) * mult in the XPut layout.  Two outputs per thread.  Grid
// (ceil(F / (2 BLOCK)), M); F even.
template <typename XT>
__global__ __launch_bounds__(BLOCK) void k_reduce_gate(const float *__restrict__ part, int S, int M, int F,
                                                       const float *__restrict__ wscale, XT *__restrict__ X, int ldx) {
  const int j = 2 * (blockIdx.x * BLOCK + threadIdx.x), m = blockIdx.y;
  if (j >= F) return;
  const float4 v = split_sum4(part, S, M, 2 * F, m, 2 * j);  // gate j, mult j, gate j + 1, mult j + 1
  float g[4] = {v.x, v.y, v.z, v.w};
  if (wscale) {
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] *= wscale[2 * j + e];
  }
  XPut<XT>::put(X + (size_t)m * ldx, F, j, silu(g[0]) * g[1]);
  XPut<XT>::put(X + (size_t)m * ldx, F, j + 1, silu(g[2]) * g[3]);
}

// a7 / a8 greedy head: the first-wins argmax of logits row m (N values), stored as the single
// partial part[m * stride] that the consumers of a head's token merge.
static __global__ __launch_bounds__(BLOCK) void k_argmax_rows(const float *__restrict__ L, int ld, int N,
                                                       ArgBest *__restrict__ part, int stride) {
  __shared__ ArgBest wb[NWAVES];
  const int m = blockIdx.x;
  const float *l = L + (size_t)m * ld;
  ArgBest best = arg_none();
  for (int i = threadIdx.x; i < N; i += BLOCK) best = arg_take(best, l[i], i);
  best = wave_arg(best);
  if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgBest t = wb[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) t = arg_merge(t, wb[w]);
    part[(size_t)m * stride] = t;
  }
}

// a8 entry of depformer step cb for conversation b0 + m: prev = the previous head's token,
// y = depformer_in[cb] . hidden + table[prev], X[m] = rms_norm(y; norm1 of layer 0) (XPut layout).
// Dynamic LDS: Dd floats.
template <typename ET, typename XT>
__global__ __launch_bounds__(BLOCK) void k_dep_entry(Dims d, Bufs s, const ET *__restrict__ table, int cb,
                                                     const float *__restrict__ norm, XT *__restrict__ X, int ldx,
                                                     int b0) {
  extern __shared__ float xs[];
  __shared__ float red[NWAVES];
  const int m = blockIdx.x, b = b0 + m;
  const int Dd = d.Dd;
  const int prev = reduce_head_partials(s.am_part + ((size_t)b * (1 + d.Q) + cb) * AM_MAX_BLOCKS, 1);
  if (threadIdx.x == 0) s.tokens[(size_t)b * (1 + d.Q) + cb] = prev;
  const float *dinp = s.din + ((size_t)b * d.Q + cb) * Dd;
  float *y = s.y + (size_t)b * Dd;
  for (int k = threadIdx.x; k < Dd; k += BLOCK) {
    const float v = dinp[k] + to_f(table[(size_t)prev * Dd + k]);  // argmax tokens are >= 0
    xs[k] = v;
    y[k] = v;
  }
  __syncthreads();
  rms_in_place(xs, norm, Dd, d.eps, red);
  for (int k = threadIdx.x; k < Dd; k += BLOCK) XPut<XT>::put(X + (size_t)m * ldx, Dd, k, xs[k]);
}

// a8 after the depformer q|k|v product Y[m] (3 Dd columns, no rope): q to dq, k and v to the
// per-frame cache entry (layer, cb) of conversation b0 + m.
static __global__ __launch_bounds__(BLOCK) void k_dep_qkv_post(Dims d, Bufs s, const float *__restrict__ Y, int ldy,
                                                        int layer, int cb, int b0) {
  const int m = blockIdx.x, b = b0 + m;
  const int Dd = d.Dd;
  const float *y = Y + (size_t)m * ldy;
  float *kvbase = s.dkv + ((((size_t)b * d.Ld + layer) * d.Q + cb) * 2) * Dd;
  for (int r = threadIdx.x; r < 3 * Dd; r += BLOCK) {
    if (r < Dd)
      s.dq[(size_t)b * Dd + r] = y[r];
    else
      kvbase[r - Dd] = y[r];
  }
}

// a8 depformer attention of conversation b0 + m: dq over the cb + 1 cache entries of `layer`
// ([LM] attend; weights e_p / den), 16 lanes per head, EPL dims per lane; o goes to X[m] (XPut
// layout).
template <typename XT, int EPL>
__global__ __launch_bounds__(BLOCK) void k_dep_attn(Dims d, Bufs s, int layer, int cb, XT *__restrict__ X, int ldx,
                                                    int b0) {
  const int m = blockIdx.x, b = b0 + m;
  const int Dd = d.Dd, hdd = d.hdd;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, sub = lane & 15;
  const float *q = s.dq + (size_t)b * Dd;
  const float *kv0 = s.dkv + ((((size_t)b * d.Ld + layer) * d.Q) * 2) * Dd;
  const float scale = 1.0f / sqrtf((float)hdd);
  const int npos = cb + 1;
  for (int hh = wave * 4 + g; hh < d.Hd; hh += NWAVES * 4) {
    const int e0 = hh * hdd + sub * EPL;
    float qv[EPL], kk[DEP_MAX_POS][EPL], vv[DEP_MAX_POS][EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) qv[i] = q[e0 + i];
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p)
      if (p < npos) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          kk[p][i] = kv0[(size_t)p * 2 * Dd + e0 + i];
          vv[p][i] = kv0[(size_t)p * 2 * Dd + Dd + e0 + i];
        }
      }
    float sc[DEP_MAX_POS];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p) {
      float dot = 0.f;
      if (p < npos) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) dot = fmaf(qv[i], kk[p][i], dot);
      }
      dot = row16_sum(dot);
      dot = __shfl(dot, lane & 48, WAVE);
      sc[p] = dot * scale;
      if (p < npos) mx = fmaxf(mx, sc[p]);
    }
    float den = 0.f;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p)
      if (p < npos) {
        sc[p] = expf(sc[p] - mx);
        den += sc[p];
      }
    float o[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = 0.f;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p)
      if (p < npos) {
        const float wgt = sc[p] / den;
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[i] = fmaf(wgt, vv[p][i], o[i]);
      }
#pragma unroll
    for (int i = 0; i < EPL; ++i) XPut<XT>::put(X + (size_t)m * ldx, Dd, e0 + i, o[i]);
  }
}

// a8 depformer step of conversation b0 + m after its q|k|v product, in one launch: the q, k and v
// columns of each head are the sum over the S splits, in order, of part[s][m][c] (row length
// 3 Dd), times the int8 row scales when wscale is set (S = 1 and no scales: `part` is the product
// itself); k and v become the per-frame cache entry (layer, cb); then the attention of q over the
// cb + 1 entries exactly as k_dep_attn, this step's entry taken from registers; o goes to X[m]
// (XPut layout).  EPL (head dims per lane) a multiple of 4.  Grid (rows, ceil(Hd / 4)) of one wave:
// each 16-lane group takes one head, and the earlier entries' loads are issued with the split
// partials', one memory round trip.
template <typename XT, int EPL>
__global__ __launch_bounds__(WAVE) void k_dep_qkv_attn(Dims d, Bufs s, const float *__restrict__ part, int S, int M,
                                                        const float *__restrict__ wscale, int layer, int cb,
                                                        XT *__restrict__ X, int ldx, int b0) {
  static_assert(EPL % 4 == 0, "columns are summed four at a time");
  const int m = blockIdx.x, b = b0 + m;
  const int Dd = d.Dd, hdd = d.hdd, N = 3 * Dd;
  const int lane = threadIdx.x & 63, g = lane >> 4, sub = lane & 15;
  float *kv0 = s.dkv + ((((size_t)b * d.Ld + layer) * d.Q) * 2) * Dd;
  float *kvc = kv0 + (size_t)cb * 2 * Dd;
  const float scale = 1.0f / sqrtf((float)hdd);
  const int npos = cb + 1;
  const int hh = blockIdx.y * 4 + g;
  if (hh < d.Hd) {  // a whole 16-lane group (the lanes its row sums read) or none
    const int e0 = hh * hdd + sub * EPL;
    float qv[EPL], kk[DEP_MAX_POS][EPL], vv[DEP_MAX_POS][EPL], kc[EPL], vc[EPL];
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p) {  // the earlier entries first: they do not wait for the sums
      if (p < cb) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          kk[p][i] = kv0[(size_t)p * 2 * Dd + e0 + i];
          vv[p][i] = kv0[(size_t)p * 2 * Dd + Dd + e0 + i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; i += 4) {
      const float4 a4 = split_sum4(part, S, M, N, m, e0 + i);
      const float4 k4 = split_sum4(part, S, M, N, m, Dd + e0 + i);
      const float4 v4 = split_sum4(part, S, M, N, m, 2 * Dd + e0 + i);
      const float qa[4] = {a4.x, a4.y, a4.z, a4.w}, ka[4] = {k4.x, k4.y, k4.z, k4.w}, va[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        qv[i + t] = wscale ? qa[t] * wscale[e0 + i + t] : qa[t];
        kc[i + t] = wscale ? ka[t] * wscale[Dd + e0 + i + t] : ka[t];
        vc[i + t] = wscale ? va[t] * wscale[2 * Dd + e0 + i + t] : va[t];
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      kvc[e0 + i] = kc[i];
      kvc[Dd + e0 + i] = vc[i];
    }
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p) {
      if (p == cb) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          kk[p][i] = kc[i];
          vv[p][i] = vc[i];
        }
      }
    }
    float sc[DEP_MAX_POS];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p) {
      float dot = 0.f;
      if (p < npos) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) dot = fmaf(qv[i], kk[p][i], dot);
      }
      dot = row16_sum(dot);  // identical bits in the group's 16 lanes
      sc[p] = dot * scale;
      if (p < npos) mx = fmaxf(mx, sc[p]);
    }
    float den = 0.f;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p)
      if (p < npos) {
        sc[p] = expf(sc[p] - mx);
        den += sc[p];
      }
    float o[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = 0.f;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p)
      if (p < npos) {
        const float wgt = sc[p] / den;
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[i] = fmaf(wgt, vv[p][i], o[i]);
      }
#pragma unroll
    for (int i = 0; i < EPL; ++i) XPut<XT>::put(X + (size_t)m * ldx, Dd, e0 + i, o[i]);
  }
}

// a11 bookkeeping of a teacher-forced prefill of T frames of conversation `conv`: for each frame,
// the user write and the gather of the 17 model inputs (into rows[t]), then the forced ring write
// and the offset step, exactly as the frame kernels do them one frame at a time.  Every step
// touches only its own stream's three ring slots, so thread st carries stream st through all T
// frames with its slots in registers, reading its forced tokens 32 frames at a time.  One block of
// 64 threads.
static __global__ __launch_bounds__(64) void k_prefill_ring(Dims d, Bufs s, int conv, int T,
                                                            const int32_t *__restrict__ text,
                                                            const int32_t *__restrict__ agent,
                                                            const int32_t *__restrict__ user,
                                                            int32_t *__restrict__ rows) {
  constexpr int U = 32;
  const int st = threadIdx.x;
  const bool on = blockIdx.x == 0 && st < d.NS;
  const int64_t off0 = s.offset[conv];
  if (on) {
    int32_t *rg = s.ring + ((size_t)conv * d.NS + st) * 3;
    int r0 = rg[0], r1 = rg[1], r2 = rg[2];
    const int delay = stream_delay(st, d.Q);
    const bool ust = st >= d.Q + 1;  // a user stream: written from the user tokens
    // this stream's forced token of frame t: text, agent codebook st - 1, or user codebook
    const int32_t *src = st == 0 ? text : ust ? user + (st - d.Q - 1) : agent + (st - 1);
    const int stride = st == 0 ? 1 : d.Q;
    for (int t0 = 0; t0 < T; t0 += U) {
      int tk[U];
#pragma unroll
      for (int i = 0; i < U; ++i) tk[i] = t0 + i < T ? src[(size_t)(t0 + i) * stride] : 0;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (t0 + i >= T) break;
        const int64_t off = off0 + t0 + i;
        const int slot = (int)(off % 3);
        int v;
        if (off <= delay)
          v = st == 0 ? d.Vt : d.Va;
        else if (ust && delay == 0)
          v = tk[i];
        else
          v = slot == 0 ? r0 : slot == 1 ? r1 : r2;
        rows[(size_t)(t0 + i) * d.NS + st] = v;
        // user streams: this frame's user token at (off + delay) % 3; generated streams: the
        // forced token at the next offset's slot
        const int w = ust ? (int)((off + delay) % 3) : (int)((off + 1) % 3);
        if (w == 0) r0 = tk[i];
        if (w == 1) r1 = tk[i];
        if (w == 2) r2 = tk[i];
      }
    }
    rg[0] = r0;
    rg[1] = r1;
    rg[2] = r2;
  }
  __syncthreads();  // every thread has read the offset before it moves
  if (blockIdx.x == 0 && st == 0) s.offset[conv] = off0 + T;
}

// a3 for prefill rows: x[t] = the 17-row embedding sum of rows[t] (audio tables in stream order,
// then text; -1 adds nothing, < -1 reads row 0).  Grid (ceil(D / BLOCK), T).
template <typename ET>
__global__ __launch_bounds__(BLOCK) void k_embed_rows(Dims d, const int32_t *__restrict__ rows,
                                                      const ET *__restrict__ emb_audio,
                                                      const ET *__restrict__ emb_text, float *__restrict__ x) {
  __shared__ int tok[MAX_STREAMS];
  const int t = blockIdx.y;
  if (threadIdx.x < d.NS) tok[threadIdx.x] = rows[(size_t)t * d.NS + threadIdx.x];
  __syncthreads();
  for (int c = blockIdx.x * BLOCK + threadIdx.x; c < d.D; c += gridDim.x * BLOCK) {
    float v[MAX_STREAMS];
#pragma unroll
    for (int k = 0; k < MAX_STREAMS; ++k) {
      if (k < d.NS) {
        const int tk = tok[k];
        const int row = tk < 0 ? 0 : tk;
        v[k] = tk == -1 ? 0.f
                        : to_f(k == 0 ? emb_text[(size_t)row * d.D + c]
                                      : emb_audio[((size_t)(k - 1) * (d.Va + 1) + row) * d.D + c]);
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int k = 1; k < MAX_STREAMS; ++k)
      if (k < d.NS && tok[k] != -1) acc += v[k];
    if (tok[0] != -1) acc += v[0];
    x[(size_t)t * d.D + c] = acc;
  }
}

// NW consecutive 32-bit words through a buffer resource from byte offset `off` (16-byte aligned
// for NW >= 4, else 8-byte); an offset past the resource's extent reads zeros and makes no request.
template <int NW>
__device__ __forceinline__ void ld_words_rsrc(__amdgpu_buffer_rsrc_t r, int off, uint32_t (&w)[NW]) {
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * c, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[4 * c + i] = v[i];
    }
  } else {
    static_assert(NW == 2, "8 bytes or a multiple of 16");
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v[0];
    w[1] = v[1];
  }
}

// a4.2 for many conversation rows at once (one decode step each): one block per (head h, row z)
// and no split of the positions.  A single pass over the n cached positions loads each step's
// keys and values together (two batches of KU steps in flight per wave, through buffer resources
// over the head's cache region: positions past n read zeros without a memory request), and every
// 16-lane group keeps an online softmax over the positions it takes (jw + g + 16 t, jw = 4 wave),
// rescaling its running sum and output when the running max grows.  The 4 groups of a wave then
// merge through the lane swaps (each swap returns the even-row or lower-half value and the
// odd-row or upper-half value in fixed slots, so both lanes of a pair compute identical bits),
// and the 4 waves through LDS in wave order: m = max, weights exp(m_w - m), out = sum w o_w /
// sum w l_w ([LM] attend: softmax(q k^T / sqrt(hd)) v over the cached positions).
template <typename KT, int HD>
__global__ __launch_bounds__(BLOCK) void k_attn_dec(Dims d, Bufs s, KV<KT> kv, int layer, int b0, AttnQ aq) {
  constexpr int EPL = HD / 16;  // elements per lane; 16 lanes cover one position's head slice
  constexpr int KU = 2;         // steps per batch
  constexpr int STEP = KU * NWAVES * 4;
  __shared__ float wm[NWAVES], wl[NWAVES];
  __shared__ float wo[NWAVES][HD];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, sub = lane & 15;
  // rows in order of decreasing cached length (ties by row): block y takes the y-th longest, so
  // the longest conversations are dispatched first and none is left streaming alone at the end.
  // With up to 64 rows every wave ranks them itself (lane l holds row l); more rows keep the
  // grid's order.
  int z = blockIdx.y;
  if (gridDim.y <= WAVE) {
    const int rows = gridDim.y;
    const int nl = lane < rows ? (int)min(s.offset[b0 + lane] + 1, (int64_t)d.C) : -1;
    int rank = 0;
    for (int k = 0; k < rows; ++k) {
      const int nk = __builtin_amdgcn_readlane(nl, k);
      rank += (nk > nl || (nk == nl && k < lane)) ? 1 : 0;
    }
    const unsigned long long hit = __ballot(lane < rows && rank == (int)blockIdx.y);
    z = __builtin_ctzll(hit);
  }
  const int b = b0 + z;
  const int64_t pos = s.offset[b];
  const int n = (int)(pos + 1 < (int64_t)d.C ? pos + 1 : (int64_t)d.C);
  float qv[EPL];
  const float *qp = s.q + (size_t)b * d.D + h * HD + sub * EPL;
#pragma unroll
  for (int i = 0; i < EPL; ++i) qv[i] = qp[i];
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t base = kv_index(d, b, layer, 0, h, 0);
  const int region = d.cap * HD * (int)sizeof(KT);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)(kv.k + base), (short)0, region, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)(kv.v + base), (short)0, region, BUF_DWORD3);
  // loaded rows stay in their storage words until used (bf16: half the registers of floats)
  constexpr int NW = EPL * (int)sizeof(KT) / 4;
  auto load = [&](int jb, uint32_t(&kr)[KU][NW], uint32_t(&vr)[KU][NW]) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int j = jb + g + u * NWAVES * 4;
      const int off = j < n ? (j * HD + sub * EPL) * (int)sizeof(KT) : BUF_OOB;
      ld_words_rsrc<NW>(rk, off, kr[u]);
      ld_words_rsrc<NW>(rv, off, vr[u]);
    }
  };
  auto elt = [](const uint32_t(&w)[NW], int i) {
    if constexpr (sizeof(KT) == 4)
      return __uint_as_float(w[i]);
    else
      return __uint_as_float((i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16));
  };
  float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) o[i] = 0.f;
  auto consume = [&](int jb, const uint32_t(&kr)[KU][NW], const uint32_t(&vr)[KU][NW]) {
    float sc[KU];
    float mx = m;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) dot = fmaf(qv[i], elt(kr[u], i), dot);
      dot = row16_sum(dot) * scale;
      sc[u] = jb + g + u * NWAVES * 4 < n ? dot : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    if (mx == -INFINITY) return;  // no position of this group yet
    const float corr = expf(m - mx);  // 0 while m is -inf
    l *= corr;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] *= corr;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const float p = expf(sc[u] - mx);  // 0 for a position past n
      l += p;
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i] = fmaf(p, elt(vr[u], i), o[i]);
    }
    m = mx;
  };
  {
    const int jw = wave * 4;
    uint32_t ka[KU][NW], va[KU][NW], kb2[KU][NW], vb2[KU][NW];
    load(jw, ka, va);
    for (int jb = jw; jb < n; jb += 2 * STEP) {
      load(jb + STEP, kb2, vb2);
      consume(jb, ka, va);
      load(jb + 2 * STEP, ka, va);
      consume(jb + STEP, kb2, vb2);
    }
  }
  // merge two (m, l, o) states; a and b are the same two states in both lanes of a pair
  auto merge = [&](float ma, float la, const float *oa, float mb, float lb, const float *ob) {
    const float mm = fmaxf(ma, mb);
    const float wa = ma == -INFINITY ? 0.f : expf(ma - mm), wb = mb == -INFINITY ? 0.f : expf(mb - mm);
    m = mm;
    l = la * wa + lb * wb;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = oa[i] * wa + ob[i] * wb;
  };
  {
    float oa[EPL], ob[EPL];
    const auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const auto rl = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(o[i]), __float_as_uint(o[i]), false, false);
      oa[i] = __uint_as_float(r[0]);
      ob[i] = __uint_as_float(r[1]);
    }
    merge(__uint_as_float(rm[0]), __uint_as_float(rl[0]), oa, __uint_as_float(rm[1]), __uint_as_float(rl[1]), ob);
  }
  {
    float oa[EPL], ob[EPL];
    const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const auto rl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[i]), __float_as_uint(o[i]), false, false);
      oa[i] = __uint_as_float(r[0]);
      ob[i] = __uint_as_float(r[1]);
    }
    merge(__uint_as_float(rm[0]), __uint_as_float(rl[0]), oa, __uint_as_float(rm[1]), __uint_as_float(rl[1]), ob);
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) wo[wave][sub * EPL + i] = o[i];
    if (sub == 0) {
      wm[wave] = m;
      wl[wave] = l;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < HD; t += BLOCK) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) mm = fmaxf(mm, wm[w]);
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      const float ww = wm[w] == -INFINITY ? 0.f : expf(wm[w] - mm);
      lsum += wl[w] * ww;
      acc += wo[w][t] * ww;
    }
    const float v = acc / lsum;
    if (aq.xo) {
      bf16_t *row = aq.xo + (size_t)z * aq.ldxo + h * HD;
      const bf16_t hi = f2bf(v);
      row[t] = hi;
      row[d.D + t] = f2bf(v - bf2f(hi));
    } else {
      s.o[(size_t)b * d.D + h * HD + t] = v;
    }
  }
}

}  // namespace mk
