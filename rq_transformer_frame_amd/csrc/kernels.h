// Frame-step kernels for gfx950.  Each kernel is one stage of the Moshi RQ-Transformer frame as
// the docs.rs page "inferencelayer 0.2.4 src/moshi_lm.rs" defines it (cited as [LM]).
//
// Weight-streaming projections share one pattern (RowStream): every wave owns a balanced,
// contiguous range of output rows, starts streaming them (two 8 KB chunks in flight) BEFORE the
// block's prologue (norm, attention, ...), and keeps two chunks in flight until its range ends.  Kernels used by several stages take the stage id as a template
// tag so that each stage is its own symbol in profiler traces.
#pragma once
#include "device_common.h"

namespace mk {

// Shapes of one session (all ints are element counts).
struct Dims {
  int B;                       // conversations
  int L, D, H, hd, F;          // temporal: layers, width, heads, head dim, FFN hidden
  int C, cap;                  // context window, KV slots held per conversation
  int Vt, Va;                  // text / audio head widths (tables have one more row)
  int Ld, Dd, Hd, hdd, Fd, Q;  // depformer
  int NS;                      // 2 * Q + 1 token streams
  int S;                       // temporal attention: most splits over positions
  float eps;
};

constexpr int AM_MAX_BLOCKS = 1024;  // argmax partials per head
constexpr int ATTN_MAX_S = 32;       // temporal attention splits
constexpr int ATTN_MIN_CHUNK = 64;   // positions per split before another split is used
constexpr int DEP_MAX_POS = 16;      // depformer steps (dep_q) per frame

// Token pick of a conversation ([LM] Sampling / MoshiLm::pick): greedy argmax, top-k temperature
// sampling or full-vocabulary Gumbel-max, with the text stream's own temperature and k.
enum { PICK_GREEDY = 0, PICK_TOPK = 1, PICK_GUMBEL = 2 };
struct SampleCfg {
  int32_t mode;
  float temp, temp_text;
  int32_t top_k, top_k_text, pad;
};

// Device-resident session state and activations.
struct Bufs {
  int32_t *ring;        // [B][NS][3]  token ring ([LM] MoshiState cache)
  int64_t *offset;      // [B]         absolute position of the next step
  int32_t *user;        // [B][Q]      this step's user tokens
  int32_t *inputs;      // [B][NS]     gathered model inputs (trace)
  float *x;             // [B][D]      temporal residual stream
  float *emb_sum;       // [B][D]      summed embedding (trace)
  float *hidden;        // [B][D]      post-out_norm hidden
  float *q;             // [B][D]      roped query
  float *o;             // [B][D]      attention output
  float *a;             // [B][F]      silu(gate) * mult
  float *text_logits;   // [B][Vt]
  int32_t *tokens;      // [B][1+Q]    text, audio cb0..Q-1 of this step
  float *din;           // [B][Q][Dd]  depformer_in[cb] . hidden
  float *y;             // [B][Dd]     depformer residual stream
  float *dq;            // [B][Dd]
  float *dkv;           // [B][Ld][Q][2][Dd] per-frame depformer KV
  float *da;            // [B][Fd]
  float *audio_logits;  // [B][Q][Va]
  int32_t *outpack;     // [B][1+Q] realigned output, then [B] has_out
  float *attn_part;     // [B][H][ATTN_MAX_S][hd+2] (max, sum, o[hd]) per split
  uint32_t *attn_cnt;   // [B][H]
  ArgBest *am_part;     // [B][1+Q][AM_MAX_BLOCKS] best row of each head block
  float *rope_freq;     // [hd/2]
  SampleCfg *samp;      // [B]         token pick of each conversation
  uint64_t *rng;        // [B]         xorshift state of each conversation's sampler
  const uint64_t *jump; // [32][64]    columns of the xorshift step's 2^i-th power over GF(2)
};

// Element e of head h at cache slot `slot` of conversation b's layer: [B][L][H][cap][hd], head-major,
// so that the positions one head's attention reads are one contiguous run of hd-element rows (an
// attention block streams whole DRAM pages instead of one 2 * hd-byte piece of every position's
// row of all heads).
__device__ __forceinline__ size_t kv_index(const Dims &d, int b, int layer, int slot, int h, int e) {
  return ((((size_t)b * d.L + layer) * d.H + h) * d.cap + slot) * d.hd + e;
}

template <typename KT>
struct KV {
  KT *k, *v;  // [B][L][H][cap][hd]
};

// ---- argmax partials --------------------------------------------------------------------------
// Each head block stores the best (value, row) of its rows; the next kernel that needs the
// token merges them (first-wins; no candidate gives 0).
__device__ __forceinline__ int reduce_head_partials(const ArgBest *__restrict__ part, int n) {
  __shared__ ArgBest wb[NWAVES];
  ArgBest bb = arg_none();
  for (int i = threadIdx.x; i < n; i += BLOCK) bb = arg_merge(bb, part[i]);
  bb = wave_arg(bb);
  if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = bb;
  __syncthreads();
  ArgBest t = wb[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) t = arg_merge(t, wb[i]);
  __syncthreads();
  return t.i < 0 ? 0 : t.i;
}

// --------------------------------------------------------------------------------------------
// a1-a3: user write, gather with INITIAL substitution, 17-row embedding sum ([LM] step_ext
// steps 1-3, MoshiLm::embed).  Grid (ceil(D / BLOCK), nb); conversation b = b0 + blockIdx.y.
// `user` holds nb rows of Q tokens.
// --------------------------------------------------------------------------------------------
template <typename ET>
__global__ __launch_bounds__(BLOCK) void k_embed_begin(Dims d, Bufs s, const ET *__restrict__ emb_audio,
                                                       const ET *__restrict__ emb_text,
                                                       const int32_t *__restrict__ user, int b0) {
  __shared__ int tok[MAX_STREAMS];
  const int b = b0 + blockIdx.y;
  const int64_t off = s.offset[b];
  const int32_t *urow = user + (size_t)blockIdx.y * d.Q;
  if (threadIdx.x < d.NS) {
    const int st = threadIdx.x;
    const int delay = stream_delay(st, d.Q);
    int v;
    if (off <= delay)
      v = (st == 0) ? d.Vt : d.Va;  // INITIAL token
    else if (st >= d.Q + 1 && delay == 0)
      v = urow[st - d.Q - 1];  // written this step at slot off % 3 and read back at once
    else
      v = s.ring[((size_t)b * d.NS + st) * 3 + (int)(off % 3)];
    tok[st] = v;
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x < d.NS) {
    const int st = threadIdx.x;
    s.inputs[(size_t)b * d.NS + st] = tok[st];
    if (st >= d.Q + 1)
      s.ring[((size_t)b * d.NS + st) * 3 + (int)((off + stream_delay(st, d.Q)) % 3)] = urow[st - d.Q - 1];
  }
  // every row value of a column is loaded before the sum, which then runs in the stream order
  for (int c = blockIdx.x * BLOCK + threadIdx.x; c < d.D; c += gridDim.x * BLOCK) {
    float v[MAX_STREAMS];
#pragma unroll
    for (int k = 0; k < MAX_STREAMS; ++k) {
      if (k < d.NS) {
        const int t = tok[k];
        const int row = t < 0 ? 0 : t;
        v[k] = t == -1 ? 0.f
                       : to_f(k == 0 ? emb_text[(size_t)row * d.D + c]
                                     : emb_audio[((size_t)(k - 1) * (d.Va + 1) + row) * d.D + c]);
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int k = 1; k < MAX_STREAMS; ++k)
      if (k < d.NS && tok[k] != -1) acc += v[k];
    if (tok[0] != -1) acc += v[0];
    s.x[(size_t)b * d.D + c] = acc;
    s.emb_sum[(size_t)b * d.D + c] = acc;
  }
}

// --------------------------------------------------------------------------------------------
// a4.1: x -> rms_norm(norm1) -> fused q|k|v rows -> interleaved rope on q, k at pos = offset ->
// q to s.q, k and v to KV slot offset % cap ([LM] temporal_step, rope_row).  Waves own balanced
// ranges of row pairs (2i, 2i+1), i.e. whole rope pairs.  Dynamic LDS: D + hd floats.
// --------------------------------------------------------------------------------------------
template <typename WT, typename KT>
__global__ __launch_bounds__(BLOCK) void k_qkv_rope(Dims d, Bufs s, KV<KT> kv, const WT *__restrict__ w,
                                                    const float *__restrict__ wscale,
                                                    const float *__restrict__ norm, int layer, int b0) {
  extern __shared__ float xs[];  // D floats, then the rope table: cos, sin of pair i at [2i], [2i+1]
  __shared__ float red[NWAVES];
  const int b = b0 + blockIdx.y;
  const int lane = threadIdx.x & 63;
  int lo, hi;
  wave_rows(blockIdx.x * NWAVES + wave_id(), gridDim.x * NWAVES, 3 * d.D / 2, 2, lo, hi);
  RowStream<WT> st;
  st.begin(w, wscale, d.D, lo, hi);
  const int64_t pos = s.offset[b];
  const int slot = (int)(pos % d.cap);
  float *rcs = xs + d.D;
  for (int i = threadIdx.x; i < d.hd / 2; i += BLOCK) {  // angle f_i * pos in float32, sin/cos in double
    const float ang = s.rope_freq[i] * (float)pos;
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    rcs[2 * i] = (float)cd;
    rcs[2 * i + 1] = (float)sd;
  }
  stage_rms(s.x + (size_t)b * d.D, norm, d.D, d.eps, xs, red);  // its barriers publish rcs
  float pend = 0.f;
  st.run(xs, [&](int row, float v) {
    if (lane != 0) return;
    if ((row & 1) == 0) {
      pend = v;
      return;
    }
    const int r0 = row - 1;
    float v0 = pend, v1 = v;
    const int part = r0 / d.D;  // 0 q, 1 k, 2 v
    const int rr = r0 - part * d.D;
    const int h = rr / d.hd, e = rr - h * d.hd;
    if (part < 2) {
      const float cs = rcs[e], sn = rcs[e + 1];
      const float a0 = v0 * cs - v1 * sn;
      const float a1 = v0 * sn + v1 * cs;
      v0 = a0;
      v1 = a1;
    }
    if (part == 0) {
      s.q[(size_t)b * d.D + rr] = v0;
      s.q[(size_t)b * d.D + rr + 1] = v1;
    } else {
      KT *cache = part == 1 ? kv.k : kv.v;
      const size_t idx = kv_index(d, b, layer, slot, h, e);
      cache[idx] = from_f<KT>(v0);
      cache[idx + 1] = from_f<KT>(v1);
    }
  });
}

// --------------------------------------------------------------------------------------------
// a4.2: single-query attention of head h over the n = min(offset + 1, context) cached positions
// ([LM] attend: scale 1/sqrt(hd) after the dot, max-subtracted softmax).  Grid (H, S, nb); only
// S_eff = min(S, ceil(n / 64)) splits take part.  Split sp takes a contiguous slice of the slots
// [0, n) (the softmax is order-free) and computes its local (max, sum, sum e*v); with one split it
// writes o directly, otherwise the last split to finish merges the partials in split order.
// Dynamic LDS: ceil(cap / S) floats.
// --------------------------------------------------------------------------------------------
// Query rows of the attention: in a frame (conv < 0) block z serves conversation b0 + z with its q
// row, its offset and its cache; in a prefill block z serves query row z of q / o, at position
// pos0 + z of conversation `conv` (launched with one split: every query attends to its own
// window [max(0, pos + 1 - C), pos], all of which is in the cache before the launch).
struct AttnQ {
  const float *q;
  float *o;
  int conv;
  int64_t pos0;
  bf16_t *xo;  // set: o goes straight to the next projection's input row z of xo (bf16 hi plane,
               // then lo plane, row stride ldxo) instead of float32
  int ldxo;
};

// N consecutive cache elements as floats (N a multiple of 4; float rows 16-byte aligned, bf16
// rows 8-byte aligned).
template <int N> __device__ __forceinline__ void ld_row(const float *p, float *o) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const float4 t = *reinterpret_cast<const float4 *>(p + i);
    o[i] = t.x;
    o[i + 1] = t.y;
    o[i + 2] = t.z;
    o[i + 3] = t.w;
  }
}
template <int N> __device__ __forceinline__ void ld_row(const bf16_t *p, float *o) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const uint2 t = *reinterpret_cast<const uint2 *>(p + i);
    o[i] = __uint_as_float(t.x << 16);
    o[i + 1] = __uint_as_float(t.x & 0xffff0000u);
    o[i + 2] = __uint_as_float(t.y << 16);
    o[i + 3] = __uint_as_float(t.y & 0xffff0000u);
  }
}

// N consecutive cache elements as floats through a buffer resource, from byte offset `off` (16-byte
// aligned for N * sizeof(KT) >= 16, else 8-byte); an offset past the resource's extent reads zeros
// and makes no memory request.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <typename KT, int N>
__device__ __forceinline__ void ld_row_rsrc(__amdgpu_buffer_rsrc_t r, int off, float *o) {
  constexpr int BYTES = N * (int)sizeof(KT);
  uint32_t w[BYTES / 4];
  if constexpr (BYTES % 16 == 0) {
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * c, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[4 * c + i] = v[i];
    }
  } else {
    static_assert(BYTES == 8, "8 or a multiple of 16 bytes");
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v[0];
    w[1] = v[1];
  }
  if constexpr (sizeof(KT) == 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// k_attn: a wave takes positions jb + g with jb stepping by NWAVES * 4 and issues the cache loads
// of ATTN_KU steps at once (one split of ATTN_MIN_CHUNK positions is one batch of loads).
constexpr int ATTN_KU = ATTN_MIN_CHUNK / (NWAVES * 4);

template <typename KT, int HD>
__global__ __launch_bounds__(BLOCK) void k_attn(Dims d, Bufs s, KV<KT> kv, int layer, int b0, AttnQ aq) {
  extern __shared__ float sc[];
  __shared__ float red[NWAVES];
  __shared__ float ored[NWAVES][HD];
  __shared__ float pbuf[ATTN_MAX_S * (HD + 2)];
  __shared__ float pws[ATTN_MAX_S];
  __shared__ int s_last;
  constexpr int EPL = HD / 16;  // elements per lane; 16 lanes cover one position's head slice
  const int h = blockIdx.x, sp = blockIdx.y;
  const bool pf = aq.conv >= 0;
  const int b = pf ? aq.conv : b0 + blockIdx.z;  // conversation whose cache is read
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, sub = lane & 15;
  const int64_t pos = pf ? aq.pos0 + blockIdx.z : s.offset[b];
  const int n = (int)(pos + 1 < (int64_t)d.C ? pos + 1 : (int64_t)d.C);
  const int S = min((int)gridDim.y, max(1, (n + ATTN_MIN_CHUNK - 1) / ATTN_MIN_CHUNK));
  if (sp >= S) return;
  const int chunk = (n + S - 1) / S;
  const int j0 = sp * chunk;
  const int j1 = min(n, j0 + chunk);
  const int len = j1 > j0 ? j1 - j0 : 0;

  float qv[EPL];
  const float *qp = (pf ? aq.q + (size_t)blockIdx.z * d.D : s.q + (size_t)b * d.D) + h * HD + sub * EPL;
#pragma unroll
  for (int i = 0; i < EPL; ++i) qv[i] = qp[i];
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t base = kv_index(d, b, layer, 0, h, 0);
  constexpr int PS = HD;  // elements from one cached position of the head to the next
  const KT *kb = kv.k + base, *vb = kv.v + base;

  // the next batch's loads are issued before the current batch is used (two batches in flight per
  // wave), through buffer resources over the head's cache region: a step wholly past the split
  // takes an offset past the region, which reads zeros without a memory request (results
  // discarded), so the prefetch past the end costs no traffic and the loads carry no branch;
  // within a step that starts inside the split, indexes past its end clamp to its last position.
  constexpr int STEP = ATTN_KU * NWAVES * 4;
  const int jl = j1 > j0 ? j1 - 1 : 0;
  const int jf = j0 + wave * 4;
  const int region = d.cap * HD * (int)sizeof(KT);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, region, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, region, BUF_DWORD3);
  auto load_batch = [&](__amdgpu_buffer_rsrc_t src, int jb0, float(&r)[ATTN_KU][EPL]) {
#pragma unroll
    for (int u = 0; u < ATTN_KU; ++u) {
      const int off = jb0 + u * NWAVES * 4 < j1
                          ? (min(jb0 + u * NWAVES * 4 + g, jl) * PS + sub * EPL) * (int)sizeof(KT)
                          : BUF_OOB;
      ld_row_rsrc<KT, EPL>(src, off, r[u]);
    }
  };
  auto scores = [&](int jb0, const float(&kr)[ATTN_KU][EPL]) {
#pragma unroll
    for (int u = 0; u < ATTN_KU; ++u) {
      const int j = jb0 + u * NWAVES * 4 + g;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) dot = fmaf(qv[i], kr[u][i], dot);
      dot = row16_sum(dot);
      if (j < j1 && sub == 0) sc[j - j0] = dot * scale;
    }
  };
  {
    float ka[ATTN_KU][EPL], kb2[ATTN_KU][EPL];
    load_batch(rk, jf, ka);
    for (int jb0 = jf; jb0 < j1; jb0 += 2 * STEP) {
      load_batch(rk, jb0 + STEP, kb2);
      scores(jb0, ka);
      load_batch(rk, jb0 + 2 * STEP, ka);
      scores(jb0 + STEP, kb2);
    }
  }
  __syncthreads();
  float m = -INFINITY;
  for (int t = threadIdx.x; t < len; t += BLOCK) m = fmaxf(m, sc[t]);
  m = block_max(m, red);
  float l = 0.f;
  for (int t = threadIdx.x; t < len; t += BLOCK) {
    const float e = expf(sc[t] - m);
    sc[t] = e;
    l += e;
  }
  l = block_sum(l, red);  // ends with a barrier, so sc[] is complete

  float op[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) op[i] = 0.f;
  auto accum = [&](int jb0, const float(&vr)[ATTN_KU][EPL]) {
#pragma unroll
    for (int u = 0; u < ATTN_KU; ++u) {
      const int j = jb0 + u * NWAVES * 4 + g;
      const float e = j < j1 ? sc[j - j0] : 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) op[i] = fmaf(e, vr[u][i], op[i]);
    }
  };
  {
    float va[ATTN_KU][EPL], vb2[ATTN_KU][EPL];
    load_batch(rv, jf, va);
    for (int jb0 = jf; jb0 < j1; jb0 += 2 * STEP) {
      load_batch(rv, jb0 + STEP, vb2);
      accum(jb0, va);
      load_batch(rv, jb0 + 2 * STEP, va);
      accum(jb0 + STEP, vb2);
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    op[i] = xor32_sum(xor16_sum(op[i]));
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) ored[wave][sub * EPL + i] = op[i];
  }
  __syncthreads();
  float *out = (pf ? aq.o + (size_t)blockIdx.z * d.D : s.o + (size_t)b * d.D) + h * HD;
  auto put_o = [&](int t, float v) {
    if (aq.xo) {
      bf16_t *row = aq.xo + (size_t)blockIdx.z * aq.ldxo + h * HD;
      const bf16_t hi = f2bf(v);
      row[t] = hi;
      row[d.D + t] = f2bf(v - bf2f(hi));
    } else {
      out[t] = v;
    }
  };
  if (S == 1) {
    for (int t = threadIdx.x; t < HD; t += BLOCK) {
      float acc = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NWAVES; ++w2) acc += ored[w2][t];
      put_o(t, acc / l);
    }
    return;
  }
  float *part = s.attn_part + (((size_t)b * d.H + h) * ATTN_MAX_S + sp) * (HD + 2);
  for (int t = threadIdx.x; t < HD; t += BLOCK) {
    float acc = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NWAVES; ++w2) acc += ored[w2][t];
    st_sys(part + 2 + t, acc);
  }
  if (threadIdx.x == 0) {
    st_sys(part, m);
    st_sys(part + 1, l);
  }
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&s.attn_cnt[(size_t)b * d.H + h], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (uint32_t)(S - 1));
  }
  __syncthreads();
  if (!s_last) return;
  // last split: stage every partial in LDS with one parallel pass, then merge in split order
  const float *p0 = s.attn_part + ((size_t)b * d.H + h) * ATTN_MAX_S * (HD + 2);
  for (int i = threadIdx.x; i < S * (HD + 2); i += BLOCK) pbuf[i] = ld_sys(p0 + i);
  __syncthreads();
  float M = -INFINITY;
  for (int k = 0; k < S; ++k) M = fmaxf(M, pbuf[k * (HD + 2)]);
  if (threadIdx.x < S) {
    const float mk = pbuf[threadIdx.x * (HD + 2)];
    pws[threadIdx.x] = mk > -INFINITY ? expf(mk - M) : 0.f;
  }
  __syncthreads();
  float Lsum = 0.f;
  for (int k = 0; k < S; ++k) Lsum += pws[k] * pbuf[k * (HD + 2) + 1];
  for (int t = threadIdx.x; t < HD; t += BLOCK) {
    float acc = 0.f;
    for (int k = 0; k < S; ++k) acc += pws[k] * pbuf[k * (HD + 2) + 2 + t];
    put_o(t, acc / Lsum);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&s.attn_cnt[(size_t)b * d.H + h], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------------------------------------------
// Projection of `in` into `out`: out[r] = (W . in)[r] (STORE) or out[r] += (W . in)[r] (residual
// add: [LM] out_proj / gate_out followed by the residual).  Dynamic LDS: K floats, plus (ADD) one
// float per row of the block's share.
// --------------------------------------------------------------------------------------------
template <typename WT, bool ADD, int TAG>
__global__ __launch_bounds__(BLOCK) void k_gemv(const WT *__restrict__ w, const float *__restrict__ wscale, int N,
                                                int K, const float *__restrict__ in, int in_ld,
                                                float *__restrict__ out, int out_ld, int b0) {
  extern __shared__ float xs[];  // K floats, then (ADD) this block's row results
  const int b = b0 + blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w0 = blockIdx.x * NWAVES, TW = gridDim.x * NWAVES;
  int lo, hi, blo, bhi;
  wave_rows(w0 + wave_id(), TW, N, 1, lo, hi);
  RowStream<WT> st;
  st.begin(w, wscale, K, lo, hi);
  stage_vec(in + (size_t)b * in_ld, K, xs);
  float *o = out + (size_t)b * out_ld;
  if (!ADD) {
    st.run(xs, [&](int row, float v) {
      if (lane == 0) o[row] = v;
    });
    return;
  }
  // residual add after the stream: a load of o inside the loop would drain the chunks in flight
  int t0, t1;
  wave_rows(w0, TW, N, 1, blo, t1);
  wave_rows(w0 + NWAVES - 1, TW, N, 1, t0, bhi);
  float *ys = xs + K;
  st.run(xs, [&](int row, float v) {
    if (lane == 0) ys[row - blo] = v;
  });
  __syncthreads();
  for (int r = blo + threadIdx.x; r < bhi; r += BLOCK) o[r] += ys[r - blo];
}

// --------------------------------------------------------------------------------------------
// a5 (first half): h = rms_norm(x; norm2), g = linear_in . h, a[j] = silu(g_gate[j]) * g_mult[j]
// ([LM] temporal_step / depformer_cycle gating).  The device copy of linear_in has its rows
// interleaved at load time (row 2j = gate row j, row 2j+1 = mult row j), so a wave's balanced range
// of row pairs yields whole outputs.  Dynamic LDS: K floats.
// --------------------------------------------------------------------------------------------
template <typename WT, int TAG>
__global__ __launch_bounds__(BLOCK) void k_gate(const WT *__restrict__ w, const float *__restrict__ wscale, int F,
                                                int K, const float *__restrict__ x, int x_ld,
                                                const float *__restrict__ norm, float eps,
                                                float *__restrict__ a, int a_ld, int b0) {
  extern __shared__ float xs[];
  __shared__ float red[NWAVES];
  const int b = b0 + blockIdx.y;
  const int lane = threadIdx.x & 63;
  int lo, hi;
  wave_rows(blockIdx.x * NWAVES + wave_id(), gridDim.x * NWAVES, F, 2, lo, hi);
  RowStream<WT> st;
  st.begin(w, wscale, K, lo, hi);
  stage_rms(x + (size_t)b * x_ld, norm, K, eps, xs, red);
  float gv = 0.f;
  st.run(xs, [&](int row, float v) {
    if ((row & 1) == 0) {
      gv = v;
      return;
    }
    if (lane == 0) a[(size_t)b * a_ld + (row >> 1)] = silu(gv) * v;
  });
}

// --------------------------------------------------------------------------------------------
// a6-a8 heads: logits = W . v with v = rms_norm(src; norm) (text head after out_norm) or v = src
// (depformer heads read y with no norm).  Each block stores the best (value, row) of its rows in
// am_part[blockIdx.x]; the kernel that needs the token merges them.  With hid_out set, block 0
// also stores the normalised vector (the post-out_norm hidden).  Dynamic LDS: K floats.
// --------------------------------------------------------------------------------------------
template <typename WT, int TAG>
__global__ __launch_bounds__(BLOCK) void k_head(const WT *__restrict__ w, const float *__restrict__ wscale, int N,
                                                int K, const float *__restrict__ src, int src_ld,
                                                const float *__restrict__ norm, float eps,
                                                float *__restrict__ hid_out, float *__restrict__ logits,
                                                int logits_ld, ArgBest *__restrict__ am_part, int am_ld, int b0) {
  extern __shared__ float xs[];
  __shared__ float red[NWAVES];
  __shared__ ArgBest wbest[NWAVES];
  const int b = b0 + blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int lo, hi;
  wave_rows(blockIdx.x * NWAVES + wave_id(), gridDim.x * NWAVES, N, 1, lo, hi);
  RowStream<WT> st;
  st.begin(w, wscale, K, lo, hi);
  if (norm)
    stage_rms(src + (size_t)b * src_ld, norm, K, eps, xs, red);
  else
    stage_vec(src + (size_t)b * src_ld, K, xs);
  if (hid_out && blockIdx.x == 0)
    for (int k = threadIdx.x; k < K; k += BLOCK) hid_out[(size_t)b * src_ld + k] = xs[k];
  ArgBest best = arg_none();
  float *lg = logits + (size_t)b * logits_ld;
  st.run(xs, [&](int row, float v) {
    if (lane != 0) return;
    lg[row] = v;
    best = arg_take(best, v, row);
  });
  if (lane == 0) wbest[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgBest bb = wbest[0];
    for (int i = 1; i < NWAVES; ++i) bb = arg_merge(bb, wbest[i]);
    am_part[(size_t)b * am_ld + blockIdx.x] = bb;
  }
}

// --------------------------------------------------------------------------------------------
// a8 depformer step cb, layer j, first half: y (layer 0: depformer_in[cb] . hidden + emb(prev),
// prev = the previous head's token, merged here from its block partials) -> rms_norm(norm1_j) ->
// q|k|v rows of in_projs[j][cb] (no rope) -> q to dq, k and v to the per-frame cache entry
// (j, cb) ([LM] depformer_cycle).  Dynamic LDS: Dd floats.
// --------------------------------------------------------------------------------------------
template <typename WT, typename ET>
__global__ __launch_bounds__(BLOCK) void k_dep_qkv(Dims d, Bufs s, const WT *__restrict__ w,
                                                   const float *__restrict__ wscale, const float *__restrict__ norm,
                                                   const ET *__restrict__ table, int layer, int cb, int prev_parts,
                                                   int b0) {
  extern __shared__ float xs[];
  __shared__ float red[NWAVES];
  const int b = b0 + blockIdx.y;
  const int Dd = d.Dd;
  const int lane = threadIdx.x & 63;
  int lo, hi;
  wave_rows(blockIdx.x * NWAVES + wave_id(), gridDim.x * NWAVES, 3 * Dd, 1, lo, hi);
  RowStream<WT> st;
  st.begin(w, wscale, Dd, lo, hi);
  float *y = s.y + (size_t)b * Dd;
  if (layer == 0) {
    const int prev =
        reduce_head_partials(s.am_part + ((size_t)b * (1 + d.Q) + cb) * AM_MAX_BLOCKS, prev_parts);
    if (blockIdx.x == 0 && threadIdx.x == 0) s.tokens[(size_t)b * (1 + d.Q) + cb] = prev;
    const float *dinp = s.din + ((size_t)b * d.Q + cb) * Dd;
    for (int k = threadIdx.x; k < Dd; k += BLOCK) {
      const float v = dinp[k] + to_f(table[(size_t)prev * Dd + k]);  // argmax tokens are >= 0
      xs[k] = v;
      if (blockIdx.x == 0) y[k] = v;
    }
    __syncthreads();
    rms_in_place(xs, norm, Dd, d.eps, red);
  } else {
    stage_rms(y, norm, Dd, d.eps, xs, red);
  }
  float *kvbase = s.dkv + ((((size_t)b * d.Ld + layer) * d.Q + cb) * 2) * Dd;
  st.run(xs, [&](int row, float v) {
    if (lane != 0) return;
    if (row < Dd)
      s.dq[(size_t)b * Dd + row] = v;
    else
      kvbase[row - Dd] = v;  // k at [0, Dd), v at [Dd, 2 Dd)
  });
}

// --------------------------------------------------------------------------------------------
// a8 depformer step cb, layer j, attention + out_proj: every block recomputes the attention of
// dq over the cb + 1 cache entries of layer j ([LM] attend; weights e_p / den) into LDS -- 16
// lanes per head, EPL dims per lane, all loads issued at once -- then y[r] += out_projs[j][cb] . o.
// Dynamic LDS: Dd floats plus one float per row of the block's share.
// --------------------------------------------------------------------------------------------
template <typename WT, int EPL>
__global__ __launch_bounds__(BLOCK) void k_dep_out(Dims d, Bufs s, const WT *__restrict__ w,
                                                   const float *__restrict__ wscale, int layer, int cb, int b0) {
  extern __shared__ float xs[];
  const int b = b0 + blockIdx.y;
  const int Dd = d.Dd, hdd = d.hdd;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, sub = lane & 15;
  int lo, hi;
  wave_rows(blockIdx.x * NWAVES + wave_id(), gridDim.x * NWAVES, Dd, 1, lo, hi);
  RowStream<WT> st;
  st.begin(w, wscale, Dd, lo, hi);

  const float *q = s.dq + (size_t)b * Dd;
  const float *kv0 = s.dkv + ((((size_t)b * d.Ld + layer) * d.Q) * 2) * Dd;
  const float scale = 1.0f / sqrtf((float)hdd);
  const int npos = cb + 1;
  for (int hh = wave * 4 + g; hh < d.Hd; hh += NWAVES * 4) {  // 16 lanes per head
    const int e0 = hh * hdd + sub * EPL;
    float qv[EPL], kk[DEP_MAX_POS][EPL], vv[DEP_MAX_POS][EPL];
    if constexpr (EPL % 4 == 0) {  // 16-byte loads
#pragma unroll
      for (int i = 0; i < EPL; i += 4) {
        const float4 t4 = *reinterpret_cast<const float4 *>(q + e0 + i);
        qv[i] = t4.x;
        qv[i + 1] = t4.y;
        qv[i + 2] = t4.z;
        qv[i + 3] = t4.w;
      }
#pragma unroll
      for (int p = 0; p < DEP_MAX_POS; ++p)
        if (p < npos) {
#pragma unroll
          for (int i = 0; i < EPL; i += 4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(kv0 + (size_t)p * 2 * Dd + e0 + i);
            const float4 v4 = *reinterpret_cast<const float4 *>(kv0 + (size_t)p * 2 * Dd + Dd + e0 + i);
            kk[p][i] = k4.x;
            kk[p][i + 1] = k4.y;
            kk[p][i + 2] = k4.z;
            kk[p][i + 3] = k4.w;
            vv[p][i] = v4.x;
            vv[p][i + 1] = v4.y;
            vv[p][i + 2] = v4.z;
            vv[p][i + 3] = v4.w;
          }
        }
    } else {
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
    }
    float sc[DEP_MAX_POS];
    float m = -INFINITY;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p) {
      float dot = 0.f;
      if (p < npos) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) dot = fmaf(qv[i], kk[p][i], dot);
      }
      dot = row16_sum(dot);
      dot = __shfl(dot, lane & 48, WAVE);  // the group's first lane: identical bits in the group
      sc[p] = dot * scale;
      if (p < npos) m = fmaxf(m, sc[p]);
    }
    float den = 0.f;
#pragma unroll
    for (int p = 0; p < DEP_MAX_POS; ++p)
      if (p < npos) {
        sc[p] = expf(sc[p] - m);
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
    for (int i = 0; i < EPL; ++i) xs[e0 + i] = o[i];
  }
  __syncthreads();
  int blo, bhi, t0, t1;
  wave_rows(blockIdx.x * NWAVES, gridDim.x * NWAVES, Dd, 1, blo, t1);
  wave_rows(blockIdx.x * NWAVES + NWAVES - 1, gridDim.x * NWAVES, Dd, 1, t0, bhi);
  float *ys = xs + Dd;  // this block's row results; the residual add follows the stream
  st.run(xs, [&](int row, float v) {
    if (lane == 0) ys[row - blo] = v;
  });
  __syncthreads();
  float *yb = s.y + (size_t)b * Dd;
  for (int r = blo + threadIdx.x; r < bhi; r += BLOCK) yb[r] += ys[r - blo];
}

// --------------------------------------------------------------------------------------------
// a9: merge the last head's argmax partials into its token, then offset += 1, ring slot
// offset % 3 <- this step's text and audio tokens, and the delay-realigned output read at
// (offset - 1 + delay) % 3 once offset > 1 ([LM] step_ext steps 7-8).  With `forced` set
// (teacher-forced prefill, [LM] step_forced) the ring gets forced[0..Q] instead and no output is
// produced.  Grid (nb), BLOCK threads.
// --------------------------------------------------------------------------------------------
struct Forced {
  int32_t t[17];
};

static __global__ __launch_bounds__(BLOCK) void k_frame_end(Dims d, Bufs s, int b0, int use_forced, Forced forced,
                                                     int last_parts) {
  const int b = b0 + blockIdx.x;
  int32_t *tk = s.tokens + (size_t)b * (1 + d.Q);
  if (!use_forced) {
    const int last = reduce_head_partials(s.am_part + ((size_t)b * (1 + d.Q) + d.Q) * AM_MAX_BLOCKS, last_parts);
    if (threadIdx.x == 0) tk[d.Q] = last;
  }
  if (threadIdx.x != 0) return;
  const int64_t off = s.offset[b] + 1;
  s.offset[b] = off;
  const int p = (int)(off % 3);
  int32_t *rg = s.ring + (size_t)b * d.NS * 3;
  for (int st = 0; st <= d.Q; ++st) rg[st * 3 + p] = use_forced ? forced.t[st] : tk[st];
  int32_t *out = s.outpack + (size_t)b * (1 + d.Q);
  int32_t *has = s.outpack + (size_t)d.B * (1 + d.Q) + b;
  if (!use_forced && off > 1) {
    for (int st = 0; st <= d.Q; ++st) out[st] = rg[st * 3 + (int)((off - 1 + stream_delay(st, d.Q)) % 3)];
    *has = 1;
  } else {
    *has = 0;
  }
}

// [LM] state(): ring <- -2, offset <- 0 for conversations [b0, b0 + gridDim.x).  The temporal
// attention's per-head split counters are cleared too: a frame that was abandoned part-way (a
// timed-out wait of the persistent kernel) can leave them raised, and a raised counter would make
// a later frame merge a head's splits before all of them are written.
static __global__ void k_reset(Dims d, Bufs s, int b0) {
  const int b = b0 + blockIdx.x;
  for (int i = threadIdx.x; i < d.NS * 3; i += blockDim.x) s.ring[(size_t)b * d.NS * 3 + i] = -2;
  for (int h = threadIdx.x; h < d.H; h += blockDim.x) s.attn_cnt[(size_t)b * d.H + h] = 0u;
  if (threadIdx.x == 0) s.offset[b] = 0;
}

// [LM] force_generated: ring slot offset % 3 of the text and generated streams <- forced tokens.
static __global__ void k_force(Dims d, Bufs s, int b, Forced forced) {
  if (threadIdx.x != 0) return;
  const int p = (int)(s.offset[b] % 3);
  for (int st = 0; st <= d.Q; ++st) s.ring[((size_t)b * d.NS + st) * 3 + p] = forced.t[st];
}

// Block quantisation at load time (the Q4_0 band with BITS = 4, q8_0 with BITS = 8), per row and
// 32-column block: d = (the block's value of largest magnitude, the first on ties) / -2^(BITS-1),
// code = clamp(round-half-away(x * (1 / d)), -2^(BITS-1), 2^(BITS-1) - 1), code 0 where d = 0; the
// float32 operations are IEEE round-to-nearest (no contraction).  Q4_0 stores code + 8 as a nibble,
// column i in the low and i + 16 in the high nibble of byte i of the block's 16; q8_0 stores the
// int8 codes.  One block of threads per row, one thread per 32-column block.
template <int BITS>
static __global__ __launch_bounds__(BLOCK) void k_quant_blocks(const float *__restrict__ w, int K,
                                                            uint8_t *__restrict__ codes, float *__restrict__ scale,
                                                            int64_t row0) {
  const int64_t r = row0 + blockIdx.x;
  const float *wr = w + (size_t)blockIdx.x * K;
  const int nb = K / 32;
  const int qmin = -(1 << (BITS - 1)), qmax = (1 << (BITS - 1)) - 1;
  for (int bk = threadIdx.x; bk < nb; bk += BLOCK) {
    const float *x = wr + bk * 32;
    float amax = 0.f, mx = 0.f;
    for (int j = 0; j < 32; ++j)
      if (fabsf(x[j]) > amax) {
        amax = fabsf(x[j]);
        mx = x[j];
      }
    const float d = __fdiv_rn(mx, (float)qmin);
    const float id = d != 0.f ? __fdiv_rn(1.0f, d) : 0.f;
    int q[32];
    for (int j = 0; j < 32; ++j) {
      const float v = roundf(__fmul_rn(x[j], id));
      q[j] = (int)fminf(fmaxf(v, (float)qmin), (float)qmax);
    }
    scale[(size_t)r * nb + bk] = d;
    if (BITS == 4) {
      uint8_t *o = codes + (size_t)r * (K / 2) + bk * 16;
      for (int i = 0; i < 16; ++i) o[i] = (uint8_t)((q[i] + 8) | ((q[i + 16] + 8) << 4));
    } else {
      int8_t *o = reinterpret_cast<int8_t *>(codes) + (size_t)r * K + bk * 32;
      for (int j = 0; j < 32; ++j) o[j] = (int8_t)q[j];
    }
  }
}

// Session snapshot ([LM] MoshiState::snapshot): copy the n cached positions p0 .. p0 + n - 1 of
// conversation b's temporal KV (position p at slot p % cap) to (to_buf = 1) or from (0) a
// position-ordered buffer [2][L][n][D] (keys, then values).  Grid (n, L).
template <typename KT>
__global__ __launch_bounds__(BLOCK) void k_kv_snapshot(Dims d, KV<KT> kv, KT *__restrict__ buf, int b, int64_t p0,
                                                    int n, int to_buf) {
  const int j = blockIdx.x, l = blockIdx.y;
  const int slot = (int)((p0 + j) % d.cap);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    KT *c = which ? kv.v : kv.k;
    KT *o = buf + (((size_t)which * d.L + l) * n + j) * d.D;
    for (int e = threadIdx.x; e < d.D; e += BLOCK) {
      const size_t ci = kv_index(d, b, l, slot, e / d.hd, e % d.hd);
      if (to_buf)
        o[e] = c[ci];
      else
        c[ci] = o[e];
    }
  }
}

// Streaming-read probe (measurement): block b of NT threads reads its contiguous share of n16 16-byte vectors
// with nontemporal buffer loads, 8 per lane in flight and no load under a branch (past the share's
// end the buffer resource returns zeros), and folds them into one word; the word is stored only if
// it equals a value no input here produces, which keeps the loads without a real store.
template <int NT>
__global__ __launch_bounds__(NT) void k_read_probe(const uint4 *__restrict__ p, int64_t n16, uint32_t *__restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  if (lo >= hi) return;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)(p + lo), (short)0, (int)((hi - lo) * 16), BUF_DWORD3);
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; i < hi - lo; i += 8 * NT) {
    u32x4b v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((i + u * NT) * 16), 0, BUF_NT);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// Per-row symmetric int8 quantisation (load time): s_r = max|w_r| / 127, q = round half away
// from zero of w / s_r, clamped to [-127, 127]; q = 0 when s_r = 0.  One block per row.
static __global__ __launch_bounds__(BLOCK) void k_quant_rows(const float *__restrict__ w, int64_t K, int8_t *__restrict__ q,
                                                      float *__restrict__ scale, int64_t row0) {
  __shared__ float red[NWAVES];
  const int64_t r = row0 + blockIdx.x;
  const float *wr = w + (size_t)blockIdx.x * K;
  float am = 0.f;
  for (int64_t k = threadIdx.x; k < K; k += BLOCK) am = fmaxf(am, fabsf(wr[k]));
  am = block_max(am, red);
  const float s_r = am / 127.0f;
  for (int64_t k = threadIdx.x; k < K; k += BLOCK) {
    float v = 0.f;
    if (s_r > 0.f) {
      v = roundf(wr[k] / s_r);
      v = fminf(fmaxf(v, -127.f), 127.f);
    }
    q[(size_t)r * K + k] = (int8_t)(int)v;
  }
  if (threadIdx.x == 0) scale[r] = s_r;
}

}  // namespace mk
