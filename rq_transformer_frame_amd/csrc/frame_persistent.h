// Persistent frame kernel: one cooperative launch runs a whole B=1 frame of the Moshi
// RQ-Transformer ([LM]: the docs.rs page "inferencelayer 0.2.4 src/moshi_lm.rs", MoshiLm::step_ext)
// as a chain of phases, one block per CU.
//
// Every phase is a weight-streaming projection (or the temporal attention) spread over all waves
// of the grid.  Phase p+1's first weight tile is loaded into registers BEFORE the block waits for
// phase p to complete, so HBM keeps streaming across phase boundaries and the wait is hidden
// behind the fetch.  Completion of a phase is signalled by per-block flags that carry a tag
// growing with the frame serial number and the phase; a waiter reads all flags.  Activations that other blocks read (x, q, o, a, y, dq, dkv, ...) are
// written with system-scope stores (write-through past the per-XCD L2) after which the writer
// waits for its stores (s_waitcnt) before it arrives, and are read with system-scope loads.  Inside
// a depformer step the phases skip the flags: their outputs travel as {value, tag} pairs that the
// readers poll (st_ll below).  Every wait is a bounded spin: on timeout the block raises the error
// flag and the whole grid exits.
#pragma once
#include "sample.h"

namespace mk {

constexpr int PBLOCK = 512;
constexpr int PWAVES = PBLOCK / WAVE;
constexpr int PQ = 8;                // most depformer steps (dep_q) the persistent kernel takes
constexpr int PSTREAMS = 2 * PQ + 1; // most token streams

struct LayerPtrs {
  const void *w_in, *w_out, *w_gin, *w_gout;
  const float *s_in, *s_out, *s_gin, *s_gout;
  const float *norm1, *norm2;
};

struct PArgs {
  Dims d;
  Bufs s;
  void *kc, *vc;
  const void *emb_audio, *emb_text;
  const LayerPtrs *tl;  // [L]
  const LayerPtrs *dl;  // [Ld][Q]
  const float *out_norm;
  const void *w_text;
  const float *s_text;
  const void *w_din;  // [Q * Dd][D]
  const float *s_din;
  const void *dep_table[PQ];  // cb 0: depformer text table, cb > 0: depformer_emb[cb - 1]
  const void *w_lin[PQ];
  const float *s_lin[PQ];
  uint32_t *sync;  // [gridDim.x] per-block phase flags
  uint64_t *ll;    // depformer exchange pairs {value, tag} (layout at st_ll)
  int *err;        // error flag (also copied back to the host with the outputs)
  int spin_limit;
  uint64_t *phase_ts;  // optional [phases][2]: block 0's arrival and the phase's completion time
  uint64_t *block_ts;  // optional [phases][gridDim.x]: every block's arrival time
};

// Four consecutive table values as one load (8 bytes of bf16 or 16 bytes of float), widened to
// float32 only when summed.
template <typename ET> struct Packed4;
template <> struct Packed4<bf16_t> {
  typedef uint2 type;
  __device__ __forceinline__ static void unpack(const uint2 &u, float *f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xFFFF0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
};
template <> struct Packed4<float> {
  typedef float4 type;
  __device__ __forceinline__ static void unpack(const float4 &u, float *f) {
    f[0] = u.x;
    f[1] = u.y;
    f[2] = u.z;
    f[3] = u.w;
  }
};

__device__ __forceinline__ void st_sys_u32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys_u64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t ld_sys_u64(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <typename KT> __device__ __forceinline__ void st_sys_pair(KT *p, float a, float b);
template <> __device__ __forceinline__ void st_sys_pair<float>(float *p, float a, float b) {
  st_sys_u64(reinterpret_cast<uint64_t *>(p), (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32));
}
template <> __device__ __forceinline__ void st_sys_pair<bf16_t>(bf16_t *p, float a, float b) {
  st_sys_u32(reinterpret_cast<uint32_t *>(p), (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16));
}

__device__ __forceinline__ void st_sys_arg(ArgBest *p, ArgBest v) {
  st_sys_u64(reinterpret_cast<uint64_t *>(p), (uint64_t)__float_as_uint(v.v) | ((uint64_t)(uint32_t)v.i << 32));
}
__device__ __forceinline__ ArgBest ld_sys_arg(const ArgBest *p) {
  const uint64_t u = ld_sys_u64(reinterpret_cast<const uint64_t *>(p));
  return ArgBest{__uint_as_float((uint32_t)u), (int)(uint32_t)(u >> 32)};
}

// Stage two vectors written by other blocks (system-coherent 16-byte loads; per pass U1 and U2
// loads per thread are issued before any LDS store): dst1[0..K1) = src1, dst2[0..K2) = src2
// (K1, K2 multiples of 4).
template <int U1, int U2>
__device__ __forceinline__ void stage2_sys(const float *src1, int K1, float *dst1, const float *src2, int K2,
                                           float *dst2) {
  const __amdgpu_buffer_rsrc_t r1 = act_rsrc(src1), r2 = act_rsrc(src2);
  float4 *d1 = reinterpret_cast<float4 *>(dst1);
  float4 *d2 = reinterpret_cast<float4 *>(dst2);
  const int n1 = K1 >> 2, n2 = K2 >> 2;
  for (int b1 = 0, b2 = 0; b1 < n1 || b2 < n2; b1 += U1 * PBLOCK, b2 += U2 * PBLOCK) {
    float4 v1[U1], v2[U2];
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      const int i = b1 + u * PBLOCK + threadIdx.x;
      v1[u] = i < n1 ? ld_sys4(r1, i * 16) : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int i = b2 + u * PBLOCK + threadIdx.x;
      v2[u] = i < n2 ? ld_sys4(r2, i * 16) : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      const int i = b1 + u * PBLOCK + threadIdx.x;
      if (i < n1) d1[i] = v1[u];
    }
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int i = b2 + u * PBLOCK + threadIdx.x;
      if (i < n2) d2[i] = v2[u];
    }
  }
  __syncthreads();
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Temporal attention: a block (one head, one position split) walks its positions in steps of
// PWAVES * 4 and issues the cache loads of ATTN_U steps at once; a split takes P_ATTN_CHUNK
// positions (one batch of loads per wave) before another block is used.
constexpr int ATTN_U = 2;
constexpr int P_ATTN_CHUNK = ATTN_U * PWAVES * 4;

// ---- phase completion ------------------------------------------------------------------------
// Every block owns one 32-bit flag (packed, so a waiting wave reads them all with a few loads in
// one round trip).  Arriving at phase p of the frame with serial number `serial` stores the tag
// serial * nph + p + 1 into the block's flag (a system-scope store: no read-modify-write, no
// contention); waiting for phase p means every flag has reached that tag.  Tags only grow (modulo
// 2^32, compared by signed difference), so flags are never cleared between frames.
__device__ __forceinline__ uint32_t p_tag(uint32_t serial, int nph, int p) { return serial * (uint32_t)nph + (uint32_t)p + 1u; }

// All of this block's stores of the phase are complete (s_waitcnt in every thread, then the
// barrier); then the block's flag is raised.
__device__ __forceinline__ void p_arrive(const PArgs &a, uint32_t tag, int p) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    st_sys_u32(a.sync + blockIdx.x, tag);
    if (a.phase_ts && blockIdx.x == 0) a.phase_ts[2 * p] = wall_clock64();
    if (a.block_ts) a.block_ts[(size_t)p * gridDim.x + blockIdx.x] = wall_clock64();
  }
}

__device__ __forceinline__ uint32_t ld_sys_u32(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Wait until every block's flag has reached `tag`.  Returns false (and raises the error flag) if
// the error flag is up or the spin limit is reached: the caller then leaves the kernel.
__device__ __forceinline__ bool p_wait(const PArgs &a, uint32_t tag, int p, int *s_ok) {
  if (threadIdx.x < WAVE) {
    const int lane = threadIdx.x;
    const int nb = gridDim.x;
    int ok = 1;
    for (int spins = 0;; ++spins) {
      uint32_t f[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) f[u] = lane + u * WAVE < nb ? ld_sys_u32(a.sync + lane + u * WAVE) : tag;
      bool done = true;
#pragma unroll
      for (int u = 0; u < 4; ++u) done = done && (int32_t)(f[u] - tag) >= 0;
      for (int i = lane + 4 * WAVE; i < nb; i += WAVE) done = done && (int32_t)(ld_sys_u32(a.sync + i) - tag) >= 0;
      if (__all(done)) break;
      int e = lane == 0 ? __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      e = __shfl(e, 0, WAVE);
      if (e != 0 || spins >= a.spin_limit) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) {
      if (!ok) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_ok = ok;
      if (a.phase_ts && blockIdx.x == 0) a.phase_ts[2 * p + 1] = wall_clock64();
    }
  }
  __syncthreads();
  return *s_ok != 0;
}

// ---- flag-in-data exchange (depformer) ---------------------------------------------------------
// Inside the depformer every value another block reads travels with a tag of the frame in the
// same 8-byte system-scope store {value, tag}, and a reader polls the values themselves until each
// carries the frame's tag.  Every location is written at most once per frame, so no grid-wide wait
// separates these phases: a reader goes on one memory round trip after the producer's store lands,
// where a phase flag costs the stores' completion, the flag store, the flag poll and a separate
// load of the data.  Layout (pairs): y0 [Q][Dd], then per (layer j, step cb) a unit
// [k: Dd][v: Dd][q: Dd][y1: Dd][a: Fd][y2: Dd].  Tags of an earlier frame never match.
__device__ __forceinline__ void st_ll(uint64_t *p, float v, uint32_t tag) {
  st_sys_u64(p, (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32));
}

__device__ __forceinline__ size_t ll_unit(const Dims &d, int j, int cb) {
  return (size_t)d.Q * d.Dd + (size_t)(j * d.Q + cb) * (5 * d.Dd + d.Fd);
}

// Poll the 16 bytes (two pairs) at byte offset `off` until both carry `tag`.  Sets `bad` on the
// spin limit or a raised error flag; the values are then meaningless and the caller exits.
__device__ __forceinline__ void ll_settle(float4 &v, __amdgpu_buffer_rsrc_t r, int off, uint32_t tag, const PArgs &a,
                                          int &bad) {
  for (int spins = 0; !bad && (__float_as_uint(v.y) != tag || __float_as_uint(v.w) != tag); ++spins) {
    if (spins >= a.spin_limit ||
        ((spins & 255) == 255 && __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)) {
      bad = 1;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = ld_sys4(r, off);
  }
}

// dst[k] = value of pair k of src for k < K (K even), U 16-byte loads per thread in flight per
// pass; returns this thread's sum of squares.  No barrier.
template <int U>
__device__ __forceinline__ float ll_copy(const uint64_t *src, int K, uint32_t tag, float *dst, const PArgs &a,
                                         int &bad) {
  const __amdgpu_buffer_rsrc_t r = act_rsrc(src);
  const int K2 = K >> 1;
  float ss = 0.f;
  for (int base = 0; base < K2; base += U * PBLOCK) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * PBLOCK + threadIdx.x;
      if (i < K2) v[u] = ld_sys4(r, i * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * PBLOCK + threadIdx.x;
      if (i < K2) {
        ll_settle(v[u], r, i * 16, tag, a, bad);
        dst[2 * i] = v[u].x;
        dst[2 * i + 1] = v[u].z;
        ss = fmaf(v[u].x, v[u].x, ss);
        ss = fmaf(v[u].z, v[u].z, ss);
      }
    }
  }
  return ss;
}

// Block-wide verdict after a polled copy (a barrier): true if any thread gave up, with the error
// flag raised so that the rest of the grid leaves too.
__device__ __forceinline__ bool ll_fail(const PArgs &a, int bad) {
  if (!__syncthreads_or(bad)) return false;
  if (threadIdx.x == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// xs = rms_norm(src; alpha) from a polled copy; false if the block must leave.
template <int U>
__device__ __forceinline__ bool ll_stage_rms(const uint64_t *src, const float *__restrict__ alpha, int K, float eps,
                                             float *xs, float *red, uint32_t tag, const PArgs &a) {
  int bad = 0;
  const float ss = ll_copy<U>(src, K, tag, xs, a, bad);
  if (ll_fail(a, bad)) return false;
  const float tot = block_sum<PBLOCK>(ss, red);
  const float inv = 1.0f / sqrtf(eps + tot / (float)K);
  for (int k = threadIdx.x; k < K; k += PBLOCK) xs[k] = (xs[k] * alpha[k]) * inv;
  __syncthreads();
  return true;
}

// End of this block's part of an exchange phase: every wave is done with the staged input (LDS is
// reused next); block 0's and every block's times are recorded as at a flag arrival.
__device__ __forceinline__ void ll_arrive(const PArgs &a, int p) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.phase_ts && blockIdx.x == 0) a.phase_ts[2 * p] = wall_clock64();
    if (a.block_ts) a.block_ts[(size_t)p * gridDim.x + blockIdx.x] = wall_clock64();
  }
}
// Block 0 holds every input of the phase after p.
__device__ __forceinline__ void ll_done(const PArgs &a, int p) {
  if (a.phase_ts && blockIdx.x == 0 && threadIdx.x == 0) a.phase_ts[2 * p + 1] = wall_clock64();
}

// ---- row phases --------------------------------------------------------------------------------
// Global wave index and count of the persistent grid.
__device__ __forceinline__ int gwave() { return blockIdx.x * PWAVES + wave_id(); }
__device__ __forceinline__ int nwaves() { return gridDim.x * PWAVES; }

// Start this wave's balanced share of a projection phase (units of P rows over the whole grid).
// Called before the wait for the previous phase: the weight stream does not depend on it.
template <typename WT>
__device__ __forceinline__ void p_begin(RowStream<WT> &rs, const void *W, const float *S, int K, int units, int P) {
  int lo, hi;
  wave_rows(gwave(), nwaves(), units, P, lo, hi);
  rs.begin(reinterpret_cast<const WT *>(W), S, K, lo, hi);
}

// Block-wide first-wins merge of the waves' best rows (lane 0 of each wave holds its best).
__device__ __forceinline__ ArgBest block_arg(ArgBest best, ArgBest *wb) {
  if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = best;
  __syncthreads();
  ArgBest t = wb[0];
#pragma unroll
  for (int i = 1; i < PWAVES; ++i) t = arg_merge(t, wb[i]);
  __syncthreads();
  return t;
}

// Merge the per-block partials of one head (system-scope loads) into its token.
__device__ __forceinline__ int merge_head(const ArgBest *part, int n, ArgBest *wb) {
  ArgBest bb = arg_none();
  for (int i = threadIdx.x; i < n; i += PBLOCK) bb = arg_merge(bb, ld_sys_arg(part + i));
  bb = wave_arg(bb);
  const ArgBest t = block_arg(bb, wb);
  return t.i < 0 ? 0 : t.i;
}

// ---- the frame ---------------------------------------------------------------------------------
// Template: weight / embedding / KV storage types, temporal head dim, depformer dims per lane
// (head_dim / 16) and the staging loads per thread for inputs of width D, F, Dd and Fd.
// The arguments live in device memory (written once per session): reading them where they are
// used keeps the ~150 dwords of pointers and sizes out of the registers of every phase.
template <typename WT, typename ET, typename KT, int HD, int DEPL, int UD, int UF, int UDd, int UFd>
__global__ __launch_bounds__(PBLOCK) void k_frame_persistent(const PArgs *__restrict__ pa, uint32_t serial) {
  const PArgs &a = *pa;
  extern __shared__ float xs[];  // max(D, F, Dd, Fd) floats; the attention phase reuses it
  __shared__ float red[PWAVES];
  __shared__ ArgBest wb[PWAVES];
  __shared__ int tok[PSTREAMS];
  __shared__ float rcs[HD];  // rope cos, sin of this frame's position, pair i at [2i], [2i+1]
  __shared__ float ored[PWAVES][HD];
  __shared__ int s_ok, s_last;
  const Dims &d = a.d;
  const Bufs &s = a.s;
  KT *kc = reinterpret_cast<KT *>(a.kc);
  KT *vc = reinterpret_cast<KT *>(a.vc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t pos = s.offset[0];
  const int slot = (int)(pos % d.cap);
  const int NPT = 5 * d.L;  // temporal phases
  const int P_HEAD = NPT;
  const int NPH = P_HEAD + d.Q * (4 * d.Ld + 1) + 1;  // phases of the frame

  // ---- a1-a3: gather (every block), user ring write (block 0), embedding sum (every block) ----
  if (threadIdx.x < d.NS) {
    const int st = threadIdx.x;
    const int delay = stream_delay(st, d.Q);
    int v;
    if (pos <= delay)
      v = (st == 0) ? d.Vt : d.Va;
    else if (st >= d.Q + 1 && delay == 0)
      v = s.user[st - d.Q - 1];
    else
      v = s.ring[st * 3 + (int)(pos % 3)];
    tok[st] = v;
  }
  if (threadIdx.x < HD / 2) {  // rope angle f_i * pos formed in float32, sin/cos in double
    const float ang = s.rope_freq[threadIdx.x] * (float)pos;
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    rcs[2 * threadIdx.x] = (float)cd;
    rcs[2 * threadIdx.x + 1] = (float)sd;
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x < d.NS) {
    const int st = threadIdx.x;
    s.inputs[st] = tok[st];
    if (st >= d.Q + 1) s.ring[st * 3 + (int)((pos + stream_delay(st, d.Q)) % 3)] = s.user[st - d.Q - 1];
  }
  {
    // four consecutive columns per thread and load; all rows of a column group are loaded before
    // the sum, which runs in the stream order (audio tables, then text)
    const ET *ea = reinterpret_cast<const ET *>(a.emb_audio);
    const ET *et = reinterpret_cast<const ET *>(a.emb_text);
    for (int c = 4 * threadIdx.x; c < d.D; c += 4 * PBLOCK) {
      typename Packed4<ET>::type raw[PSTREAMS];
#pragma unroll
      for (int k = 0; k < PSTREAMS; ++k)
        if (k < d.NS) {
          const int t = tok[k];
          const int row = t < 0 ? 0 : t;
          const ET *src = k == 0 ? et + (size_t)row * d.D + c : ea + ((size_t)(k - 1) * (d.Va + 1) + row) * d.D + c;
          raw[k] = *reinterpret_cast<const typename Packed4<ET>::type *>(src);
        }
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 1; k < PSTREAMS; ++k)
        if (k < d.NS && tok[k] != -1) {
          float f[4];
          Packed4<ET>::unpack(raw[k], f);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += f[e];
        }
      if (tok[0] != -1) {
        float f[4];
        Packed4<ET>::unpack(raw[0], f);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += f[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xs[c + e] = acc[e];
        if (blockIdx.x == 0) {
          st_sys(s.x + c + e, acc[e]);
          s.emb_sum[c + e] = acc[e];
        }
      }
    }
  }
  __syncthreads();

  // one weight stream for every phase; each phase's first chunks are requested before the wait
  // for the phase it depends on
  RowStream<WT> rs;
  p_begin(rs, a.tl[0].w_in, a.tl[0].s_in, d.D, 3 * d.D / 2, 2);

  // ---- a4-a5: temporal layers ----
  for (int l = 0; l < d.L; ++l) {
    const LayerPtrs lp = a.tl[l];
    const int P = 5 * l;
    // qkv + rope + KV append: row pairs (2i, 2i+1) are whole rope pairs
    if (l == 0)
      rms_in_place<PBLOCK>(xs, lp.norm1, d.D, d.eps, red);
    else
      stage_rms<PBLOCK, true, UD>(s.x, lp.norm1, d.D, d.eps, xs, red);
    {
      float pend = 0.f;
      rs.run(xs, [&](int row, float v) {
        if (lane != 0) return;
        if ((row & 1) == 0) {
          pend = v;
          return;
        }
        const int r0 = row - 1;
        float v0 = pend, v1 = v;
        const int part = r0 / d.D;
        const int rr = r0 - part * d.D;
        const int h = rr / HD, e = rr - h * HD;
        if (part < 2) {
          const float cs = rcs[e], sn = rcs[e + 1];
          const float a0 = v0 * cs - v1 * sn;
          const float a1 = v0 * sn + v1 * cs;
          v0 = a0;
          v1 = a1;
        }
        if (part == 0) {
          st_sys_u64(reinterpret_cast<uint64_t *>(s.q + rr),
                     (uint64_t)__float_as_uint(v0) | ((uint64_t)__float_as_uint(v1) << 32));
        } else {
          KT *cache = part == 1 ? kc : vc;
          st_sys_pair<KT>(cache + kv_index(d, 0, l, slot, h, e), v0, v1);
        }
      });
    }
    p_arrive(a, p_tag(serial, NPH, P), P);
    p_begin(rs, lp.w_out, lp.s_out, d.D, d.D, 1);  // out_proj, after attention
    if (!p_wait(a, p_tag(serial, NPH, P), P, &s_ok)) return;

    // attention: block bi < H * S takes head bi % H, split bi / H
    {
      const int n = (int)(pos + 1 < (int64_t)d.C ? pos + 1 : (int64_t)d.C);
      // splits: enough for P_ATTN_CHUNK positions each, at most ATTN_MAX_S, and every (head,
      // split) pair needs a block of its own (the grid holds at least H blocks)
      const int S = min(min(ATTN_MAX_S, (int)gridDim.x / d.H), max(1, (n + P_ATTN_CHUNK - 1) / P_ATTN_CHUNK));
      const int bi = blockIdx.x;
      if (bi < d.H * S) {
        constexpr int EPL = HD / 16;
        const int h = bi % d.H, sp = bi / d.H;
        const int g = lane >> 4, sub = lane & 15;
        const int chunk = (n + S - 1) / S;
        const int j0 = sp * chunk, j1 = min(n, j0 + chunk);
        const int len = j1 > j0 ? j1 - j0 : 0;
        float *sc = xs;  // scores
        float qv[EPL];
        {
          const __amdgpu_buffer_rsrc_t rq = act_rsrc(s.q);
#pragma unroll
          for (int i = 0; i < EPL; i += 4) {
            const float4 t4 = ld_sys4(rq, (h * HD + sub * EPL + i) * 4);
            qv[i] = t4.x;
            qv[i + 1] = t4.y;
            qv[i + 2] = t4.z;
            qv[i + 3] = t4.w;
          }
        }
        const float scale = 1.0f / sqrtf((float)HD);
        const size_t base = kv_index(d, 0, l, 0, h, 0);
        constexpr int PS = HD;  // elements from one cached position of the head to the next
        const KT *kb = kc + base, *vb = vc + base;
        // a wave takes positions jb + g, jb stepping by PWAVES * 4; the loads of ATTN_U steps are
        // issued together (indexes past the split clamp to its last position, results discarded)
        constexpr int STEP = ATTN_U * PWAVES * 4;
        const int jl = j1 > j0 ? j1 - 1 : 0;
        for (int jb0 = j0 + wave * 4; jb0 < j1; jb0 += STEP) {
          float kr[ATTN_U][EPL];
#pragma unroll
          for (int u = 0; u < ATTN_U; ++u)
            ld_row<EPL>(kb + (size_t)min(jb0 + u * PWAVES * 4 + g, jl) * PS + sub * EPL, kr[u]);
#pragma unroll
          for (int u = 0; u < ATTN_U; ++u) {
            const int j = jb0 + u * PWAVES * 4 + g;
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < EPL; ++i) dot = fmaf(qv[i], kr[u][i], dot);
            dot = row16_sum(dot);
            if (j < j1 && sub == 0) sc[j - j0] = dot * scale;
          }
        }
        __syncthreads();
        float m = -INFINITY;
        for (int t = threadIdx.x; t < len; t += PBLOCK) m = fmaxf(m, sc[t]);
        m = block_max<PBLOCK>(m, red);
        float lsum = 0.f;
        for (int t = threadIdx.x; t < len; t += PBLOCK) {
          const float e = expf(sc[t] - m);
          sc[t] = e;
          lsum += e;
        }
        lsum = block_sum<PBLOCK>(lsum, red);
        float op[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) op[i] = 0.f;
        for (int jb0 = j0 + wave * 4; jb0 < j1; jb0 += STEP) {
          float vr[ATTN_U][EPL];
#pragma unroll
          for (int u = 0; u < ATTN_U; ++u)
            ld_row<EPL>(vb + (size_t)min(jb0 + u * PWAVES * 4 + g, jl) * PS + sub * EPL, vr[u]);
#pragma unroll
          for (int u = 0; u < ATTN_U; ++u) {
            const int j = jb0 + u * PWAVES * 4 + g;
            const float e = j < j1 ? sc[j - j0] : 0.f;
#pragma unroll
            for (int i = 0; i < EPL; ++i) op[i] = fmaf(e, vr[u][i], op[i]);
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
        if (S == 1) {
          for (int t = threadIdx.x; t < HD; t += PBLOCK) {
            float acc = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < PWAVES; ++w2) acc += ored[w2][t];
            st_sys(s.o + h * HD + t, acc / lsum);
          }
        } else {
          float *part = s.attn_part + ((size_t)h * ATTN_MAX_S + sp) * (HD + 2);
          for (int t = threadIdx.x; t < HD; t += PBLOCK) {
            float acc = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < PWAVES; ++w2) acc += ored[w2][t];
            st_sys(part + 2 + t, acc);
          }
          if (threadIdx.x == 0) {
            st_sys(part, m);
            st_sys(part + 1, lsum);
          }
          wait_mem();
          __syncthreads();
          if (threadIdx.x == 0) {
            const uint32_t prev =
                __hip_atomic_fetch_add(&s.attn_cnt[h], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (uint32_t)(S - 1));
          }
          __syncthreads();
          if (s_last) {
            float *pbuf = xs;  // S * (HD + 2) floats
            const float *p0 = s.attn_part + (size_t)h * ATTN_MAX_S * (HD + 2);
            for (int i = threadIdx.x; i < S * (HD + 2); i += PBLOCK) pbuf[i] = ld_sys(p0 + i);
            __syncthreads();
            float M = -INFINITY;
            for (int k = 0; k < S; ++k) M = fmaxf(M, pbuf[k * (HD + 2)]);
            float *pws = xs + ATTN_MAX_S * (HD + 2);
            if (threadIdx.x < S) {
              const float mk = pbuf[threadIdx.x * (HD + 2)];
              pws[threadIdx.x] = mk > -INFINITY ? expf(mk - M) : 0.f;
            }
            __syncthreads();
            float Lsum = 0.f;
            for (int k = 0; k < S; ++k) Lsum += pws[k] * pbuf[k * (HD + 2) + 1];
            for (int t = threadIdx.x; t < HD; t += PBLOCK) {
              float acc = 0.f;
              for (int k = 0; k < S; ++k) acc += pws[k] * pbuf[k * (HD + 2) + 2 + t];
              st_sys(s.o + h * HD + t, acc / Lsum);
            }
            if (threadIdx.x == 0) __hip_atomic_store(&s.attn_cnt[h], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    p_arrive(a, p_tag(serial, NPH, P + 1), P + 1);
    if (!p_wait(a, p_tag(serial, NPH, P + 1), P + 1, &s_ok)) return;

    // out_proj + residual (x staged next to o)
    stage2_sys<UD, UD>(s.o, d.D, xs, s.x, d.D, xs + d.D);
    rs.run(xs, [&](int row, float v) {
      if (lane == 0) st_sys(s.x + row, xs[d.D + row] + v);
    });
    p_arrive(a, p_tag(serial, NPH, P + 2), P + 2);
    p_begin(rs, lp.w_gin, lp.s_gin, d.D, d.F, 2);
    if (!p_wait(a, p_tag(serial, NPH, P + 2), P + 2, &s_ok)) return;

    // norm2 + gate_in + silu * mult (rows interleaved: 2j gate, 2j + 1 mult)
    stage_rms<PBLOCK, true, UD>(s.x, lp.norm2, d.D, d.eps, xs, red);
    {
      float gv = 0.f;
      rs.run(xs, [&](int row, float v) {
        if (lane != 0) return;
        if ((row & 1) == 0)
          gv = v;
        else
          st_sys(s.a + (row >> 1), silu(gv) * v);
      });
    }
    p_arrive(a, p_tag(serial, NPH, P + 3), P + 3);
    p_begin(rs, lp.w_gout, lp.s_gout, d.F, d.D, 1);
    if (!p_wait(a, p_tag(serial, NPH, P + 3), P + 3, &s_ok)) return;

    // gate_out + residual (x staged next to a)
    stage2_sys<UF, UD>(s.a, d.F, xs, s.x, d.D, xs + d.F);
    rs.run(xs, [&](int row, float v) {
      if (lane == 0) st_sys(s.x + row, xs[d.F + row] + v);
    });
    p_arrive(a, p_tag(serial, NPH, P + 4), P + 4);
    if (l + 1 < d.L)
      p_begin(rs, a.tl[l + 1].w_in, a.tl[l + 1].s_in, d.D, 3 * d.D / 2, 2);
    else
      p_begin(rs, a.w_text, a.s_text, d.D, d.Vt, 1);
    if (!p_wait(a, p_tag(serial, NPH, P + 4), P + 4, &s_ok)) return;
  }

  // ---- a6-a7: out_norm, text head (argmax partials) and depformer_in for every codebook ----
  {
    stage_rms<PBLOCK, true, UD>(s.x, a.out_norm, d.D, d.eps, xs, red);
    if (blockIdx.x == 0)
      for (int k = threadIdx.x; k < d.D; k += PBLOCK) s.hidden[k] = xs[k];
    ArgBest best = arg_none();
    // full-vocabulary Gumbel-max sampling folded into the heads' argmax: each wave starts its
    // rows' draws at the frame's stream state advanced to its first row ([LM] gumbel_full_pick
    // draws one uniform per logit, text head first, then codebooks 0..Q-1); the sampler fields
    // are read where they are used, so that nothing stays live across the frame
    const bool gumbel = s.samp[0].mode == PICK_GUMBEL;
    uint64_t gx = 0;
    float gt = 1.f;
    if (gumbel) {
      int lo, hi;
      wave_rows(gwave(), nwaves(), d.Vt, 1, lo, hi);
      gx = wave_xs_jump(s.rng[0], (uint32_t)lo, s.jump);
      gt = s.samp[0].temp_text;
    }
    rs.run(xs, [&](int row, float v) {
      const float sc = gumbel ? gumbel_score(v, gt, gx) : v;
      if (lane != 0) return;
      s.text_logits[row] = v;
      best = arg_take(best, sc, row);
    });
    best = wave_arg(best);
    best = block_arg(best, wb);
    if (threadIdx.x == 0) st_sys_arg(s.am_part + blockIdx.x, best);
    p_begin(rs, a.w_din, a.s_din, d.D, d.Q * d.Dd, 1);
    rs.run(xs, [&](int row, float v) {
      if (lane == 0) st_sys(s.din + row, v);
    });
  }
  p_arrive(a, p_tag(serial, NPH, P_HEAD), P_HEAD);
  p_begin(rs, a.dl[0].w_in, a.dl[0].s_in, d.Dd, 3 * d.Dd, 1);
  if (!p_wait(a, p_tag(serial, NPH, P_HEAD), P_HEAD, &s_ok)) return;

  // ---- a8: depformer, 8 sequential codebook steps ----
  // Inside a step the phases exchange their outputs as tagged pairs (no grid-wide wait); the
  // codebook head still ends with one, since the next step merges every block's argmax partial.
  const uint32_t ft = p_tag(serial, NPH, NPH - 1);  // this frame's exchange tag
  const __amdgpu_buffer_rsrc_t rll = act_rsrc(a.ll);
  const ET *tbl;
  for (int cb = 0; cb < d.Q; ++cb) {
    const int PC = P_HEAD + 1 + cb * (4 * d.Ld + 1);
    for (int j = 0; j < d.Ld; ++j) {
      const LayerPtrs lp = a.dl[j * d.Q + cb];
      const int P = PC + 4 * j;
      uint64_t *u = a.ll + ll_unit(d, j, cb);  // this (layer, step)'s k | v | q | y1 | a | y2
      const size_t yin = j == 0 ? (size_t)cb * d.Dd : ll_unit(d, j - 1, cb) + 4 * d.Dd + d.Fd;
      // entry (layer 0): previous token, y = depformer_in[cb] . hidden + emb(prev)
      if (j == 0) {
        const int prev = merge_head(s.am_part + (size_t)cb * AM_MAX_BLOCKS, gridDim.x, wb);
        if (blockIdx.x == 0 && threadIdx.x == 0) s.tokens[cb] = prev;
        tbl = reinterpret_cast<const ET *>(a.dep_table[cb]);
        for (int k = threadIdx.x; k < d.Dd; k += PBLOCK) {
          const float v = ld_sys(s.din + (size_t)cb * d.Dd + k) + to_f(tbl[(size_t)prev * d.Dd + k]);
          xs[k] = v;
          if (blockIdx.x == 0) st_ll(a.ll + yin + k, v, ft);
        }
        __syncthreads();
        rms_in_place<PBLOCK>(xs, lp.norm1, d.Dd, d.eps, red);
      } else {
        if (!ll_stage_rms<2 * UDd>(a.ll + yin, lp.norm1, d.Dd, d.eps, xs, red, ft, a)) return;
        ll_done(a, P - 1);
      }
      // k, v also go to the plain per-frame KV: later steps read them after the codebook head's
      // grid-wide wait, which follows the completion of these stores
      float *kvbase = s.dkv + ((size_t)j * d.Q + cb) * 2 * d.Dd;
      rs.run(xs, [&](int row, float v) {
        if (lane != 0) return;
        if (row < d.Dd) {
          st_ll(u + 2 * d.Dd + row, v, ft);
        } else {
          st_ll(u + row - d.Dd, v, ft);
          st_sys(kvbase + row - d.Dd, v);
        }
      });
      ll_arrive(a, P);
      p_begin(rs, lp.w_out, lp.s_out, d.Dd, d.Dd, 1);

      // attention of q over the cb + 1 entries of layer j (every block), then out_proj + residual
      float *ys = xs + d.Dd;  // y, for the residual
      {
        int bad = 0;
        constexpr int UY = 2 * UDd;  // y pairs in UY 16-byte loads per thread (one pass when Dd <= 4 * UDd * PBLOCK)
        const int Y2 = d.Dd >> 1;
        float4 yv[UY];
#pragma unroll
        for (int uu = 0; uu < UY; ++uu) {
          const int i = uu * PBLOCK + threadIdx.x;
          if (i < Y2) yv[uu] = ld_sys4(rll, (int)((yin + 2 * i) * 8));
        }
        const int g = lane >> 4, sub = lane & 15;
        const float scale = 1.0f / sqrtf((float)d.hdd);
        const int npos = cb + 1;
        static_assert(DEPL % 2 == 0, "depformer dims per lane load as pairs of pairs");
        constexpr int DL2 = DEPL / 2;
        const float *kv0 = s.dkv + (size_t)j * d.Q * 2 * d.Dd;
        const __amdgpu_buffer_rsrc_t rkv = act_rsrc(kv0);
        for (int hh = wave * 4 + g; hh < d.Hd; hh += PWAVES * 4) {
          const int e0 = hh * d.hdd + sub * DEPL;
          // this step's q, k, v as tagged pairs; the earlier steps' k, v from the plain KV
          float4 qr[DL2], kr[DL2], vr[DL2];
          const int qoff = (int)((ll_unit(d, j, cb) + 2 * d.Dd + e0) * 8);
          const int koff = (int)((ll_unit(d, j, cb) + e0) * 8);
#pragma unroll
          for (int i = 0; i < DL2; ++i) {
            qr[i] = ld_sys4(rll, qoff + 16 * i);
            kr[i] = ld_sys4(rll, koff + 16 * i);
            vr[i] = ld_sys4(rll, koff + d.Dd * 8 + 16 * i);
          }
          float qv[DEPL], kk[PQ][DEPL], vv[PQ][DEPL];
          static_assert(DEPL % 4 == 0, "depformer dims per lane load as float4");
#pragma unroll
          for (int p = 0; p < PQ; ++p)
            if (p < cb) {
#pragma unroll
              for (int i = 0; i < DEPL; i += 4) {
                const float4 k4 = ld_sys4(rkv, (p * 2 * d.Dd + e0 + i) * 4);
                const float4 v4 = ld_sys4(rkv, (p * 2 * d.Dd + d.Dd + e0 + i) * 4);
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
#pragma unroll
          for (int i = 0; i < DL2; ++i) {
            ll_settle(qr[i], rll, qoff + 16 * i, ft, a, bad);
            ll_settle(kr[i], rll, koff + 16 * i, ft, a, bad);
            ll_settle(vr[i], rll, koff + d.Dd * 8 + 16 * i, ft, a, bad);
            qv[2 * i] = qr[i].x;
            qv[2 * i + 1] = qr[i].z;
          }
#pragma unroll
          for (int p = 0; p < PQ; ++p)
            if (p == cb) {
#pragma unroll
              for (int i = 0; i < DL2; ++i) {
                kk[p][2 * i] = kr[i].x;
                kk[p][2 * i + 1] = kr[i].z;
                vv[p][2 * i] = vr[i].x;
                vv[p][2 * i + 1] = vr[i].z;
              }
            }
          float sc[PQ];
          float m = -INFINITY;
#pragma unroll
          for (int p = 0; p < PQ; ++p) {
            float dot = 0.f;
            if (p < npos) {
#pragma unroll
              for (int i = 0; i < DEPL; ++i) dot = fmaf(qv[i], kk[p][i], dot);
            }
            dot = row16_sum(dot);
            dot = __shfl(dot, lane & 48, WAVE);
            sc[p] = dot * scale;
            if (p < npos) m = fmaxf(m, sc[p]);
          }
          float den = 0.f;
#pragma unroll
          for (int p = 0; p < PQ; ++p)
            if (p < npos) {
              sc[p] = expf(sc[p] - m);
              den += sc[p];
            }
          float o[DEPL];
#pragma unroll
          for (int i = 0; i < DEPL; ++i) o[i] = 0.f;
#pragma unroll
          for (int p = 0; p < PQ; ++p)
            if (p < npos) {
              const float wgt = sc[p] / den;
#pragma unroll
              for (int i = 0; i < DEPL; ++i) o[i] = fmaf(wgt, vv[p][i], o[i]);
            }
#pragma unroll
          for (int i = 0; i < DEPL; ++i) xs[e0 + i] = o[i];
        }
#pragma unroll
        for (int uu = 0; uu < UY; ++uu) {
          const int i = uu * PBLOCK + threadIdx.x;
          if (i < Y2) {
            ll_settle(yv[uu], rll, (int)((yin + 2 * i) * 8), ft, a, bad);
            ys[2 * i] = yv[uu].x;
            ys[2 * i + 1] = yv[uu].z;
          }
        }
        if (ll_fail(a, bad)) return;
        ll_done(a, P);
      }
      rs.run(xs, [&](int row, float v) {
        if (lane == 0) st_ll(u + 3 * d.Dd + row, ys[row] + v, ft);
      });
      ll_arrive(a, P + 1);
      p_begin(rs, lp.w_gin, lp.s_gin, d.Dd, d.Fd, 2);

      // norm2 + gate_in + silu * mult (rows interleaved)
      if (!ll_stage_rms<2 * UDd>(u + 3 * d.Dd, lp.norm2, d.Dd, d.eps, xs, red, ft, a)) return;
      ll_done(a, P + 1);
      {
        float gv = 0.f;
        rs.run(xs, [&](int row, float v) {
          if (lane != 0) return;
          if ((row & 1) == 0)
            gv = v;
          else
            st_ll(u + 4 * d.Dd + (row >> 1), silu(gv) * v, ft);
        });
      }
      ll_arrive(a, P + 2);
      p_begin(rs, lp.w_gout, lp.s_gout, d.Fd, d.Dd, 1);

      // gate_out + residual (y1 staged next to a)
      {
        int bad = 0;
        (void)ll_copy<2 * UFd>(u + 4 * d.Dd, d.Fd, ft, xs, a, bad);
        (void)ll_copy<2 * UDd>(u + 3 * d.Dd, d.Dd, ft, xs + d.Fd, a, bad);
        if (ll_fail(a, bad)) return;
        ll_done(a, P + 2);
      }
      rs.run(xs, [&](int row, float v) {
        if (lane == 0) st_ll(u + 4 * d.Dd + d.Fd + row, xs[d.Fd + row] + v, ft);
      });
      ll_arrive(a, P + 3);
      if (j + 1 < d.Ld)
        p_begin(rs, a.dl[(j + 1) * d.Q + cb].w_in, a.dl[(j + 1) * d.Q + cb].s_in, d.Dd, 3 * d.Dd, 1);
      else
        p_begin(rs, a.w_lin[cb], a.s_lin[cb], d.Dd, d.Va, 1);
    }
    // codebook head (no norm) with argmax partials
    {
      const int P = PC + 4 * d.Ld;
      {
        int bad = 0;
        (void)ll_copy<2 * UDd>(a.ll + ll_unit(d, d.Ld - 1, cb) + 4 * d.Dd + d.Fd, d.Dd, ft, xs, a, bad);
        if (ll_fail(a, bad)) return;
        ll_done(a, P - 1);
      }
      ArgBest best = arg_none();
      float *lg = s.audio_logits + (size_t)cb * d.Va;
      const bool gumbel = s.samp[0].mode == PICK_GUMBEL;
      uint64_t gx = 0;
      float gt = 1.f;
      if (gumbel) {
        int lo, hi;
        wave_rows(gwave(), nwaves(), d.Va, 1, lo, hi);
        gx = wave_xs_jump(s.rng[0], (uint32_t)(d.Vt + cb * d.Va + lo), s.jump);
        gt = s.samp[0].temp;
      }
      rs.run(xs, [&](int row, float v) {
        const float sc = gumbel ? gumbel_score(v, gt, gx) : v;
        if (lane != 0) return;
        lg[row] = v;
        best = arg_take(best, sc, row);
      });
      best = wave_arg(best);
      best = block_arg(best, wb);
      if (threadIdx.x == 0) st_sys_arg(s.am_part + (size_t)(1 + cb) * AM_MAX_BLOCKS + blockIdx.x, best);
      p_arrive(a, p_tag(serial, NPH, P), P);
      if (cb + 1 < d.Q) {
        p_begin(rs, a.dl[cb + 1].w_in, a.dl[cb + 1].s_in, d.Dd, 3 * d.Dd, 1);
        if (!p_wait(a, p_tag(serial, NPH, P), P, &s_ok)) return;
      }
    }
  }

  // ---- a9: frame end (block 0) ----
  if (blockIdx.x != 0) return;
  const int P_LAST = NPH - 1;
  if (!p_wait(a, p_tag(serial, NPH, P_LAST), P_LAST, &s_ok)) return;
  const int last = merge_head(s.am_part + (size_t)d.Q * AM_MAX_BLOCKS, gridDim.x, wb);
  if (threadIdx.x == 0) {
    s.tokens[d.Q] = last;
    if (s.samp[0].mode == PICK_GUMBEL) s.rng[0] = xs_jump(s.rng[0], (uint32_t)(d.Vt + d.Q * d.Va), s.jump);
    const int64_t off = pos + 1;
    s.offset[0] = off;
    const int p = (int)(off % 3);
    int32_t *tk = s.tokens;
    for (int st = 0; st <= d.Q; ++st) s.ring[st * 3 + p] = tk[st];
    int32_t *has = s.outpack + (1 + d.Q);
    if (off > 1) {
      for (int st = 0; st <= d.Q; ++st) s.outpack[st] = s.ring[st * 3 + (int)((off - 1 + stream_delay(st, d.Q)) % 3)];
      *has = 1;
    } else {
      *has = 0;
    }
  }
}

}  // namespace mk
