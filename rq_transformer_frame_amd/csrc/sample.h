// Sampled token picks for gfx950: the seeded xorshift stream, full-vocabulary Gumbel-max and
// top-k temperature sampling, as the docs.rs page "inferencelayer 0.2.4 src/moshi_lm.rs" ([LM])
// defines them in xorshift_u01, gumbel_full_pick, topk_sample and MoshiLm::pick.
//
// The sampler draws from one xorshift stream per conversation, in pick order: the text head,
// then codebooks 0..Q-1.  Gumbel-max draws one uniform per logit in index order, top-k one per
// pick.  The step x -> x ^= x << 13, x ^= x >> 7, x ^= x << 17 is linear over GF(2)^64, so the
// state n draws ahead is M^n x; a table of the columns of M^(2^i) lets any thread start at its
// own index (xs_jump) instead of walking the stream from the start.
#pragma once
#include "kernels.h"

namespace mk {

constexpr int JUMP_POW = 32;     // powers M^(2^i), i < 32, in the jump table
constexpr int TOPK_MAX = 1024;   // most candidates of a top-k pick
constexpr int PICK_BLOCK = 512;  // threads of k_pick

__device__ __forceinline__ uint64_t xs_next(uint64_t x) {
  x ^= x << 13;
  x ^= x >> 7;
  x ^= x << 17;
  return x;
}

// The uniform in [0, 1) of a drawn state: its top 53 bits over 2^53.
__device__ __forceinline__ double xs_unit(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

// x advanced n draws: for each set bit i of n, x <- M^(2^i) x, the XOR of the columns of
// M^(2^i) selected by the bits of x.  One thread, 64 steps per set bit.
__device__ __forceinline__ uint64_t xs_jump(uint64_t x, uint32_t n, const uint64_t *__restrict__ tab) {
  for (int i = 0; n != 0; ++i, n >>= 1) {
    if (!(n & 1u)) continue;
    const uint64_t *c = tab + (size_t)i * 64;
    uint64_t y = 0;
#pragma unroll 16
    for (int j = 0; j < 64; ++j) y ^= c[j] & (0ull - ((x >> j) & 1ull));
    x = y;
  }
  return x;
}

// The same with the wave's 64 lanes taking one column each (x and n wave-uniform).
__device__ __forceinline__ uint64_t wave_xs_jump(uint64_t x, uint32_t n, const uint64_t *__restrict__ tab) {
  const int lane = threadIdx.x & 63;
  for (int i = 0; n != 0; ++i, n >>= 1) {
    if (!(n & 1u)) continue;
    uint64_t y = ((x >> lane) & 1ull) ? tab[(size_t)i * 64 + lane] : 0ull;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)y, o, WAVE), hi = __shfl_xor((uint32_t)(y >> 32), o, WAVE);
      y ^= ((uint64_t)hi << 32) | lo;
    }
    x = y;
  }
  return x;
}

// [LM] gumbel_full_pick for one logit: draw, g = float32(-ln(-ln(max(u, 1e-300)))) in double,
// score float32(v / T) + g.
__device__ __forceinline__ float gumbel_score(float v, float temp, uint64_t &x) {
  x = xs_next(x);
  const double u = fmax(xs_unit(x), 1e-300);
  const float g = (float)(-log(-log(u)));
  const float q = v / temp;
  return q + g;
}

// Order-preserving key of a float32 (the total order of [LM]'s total_cmp): larger key, larger value.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t b = __float_as_uint(f);
  return b ^ ((b & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float fkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

struct PickScratch {
  uint32_t hist[256];
  int misc[4];
  int wsum[2][32];
  double total;
  uint64_t cand[TOPK_MAX];  // (key << 32) | (2^32 - 1 - index): descending order = larger value, then lower index
  double p[TOPK_MAX];
};

// Exclusive block-wide prefix sums of two counts.
template <int NT>
__device__ __forceinline__ void block_exscan2(int a, int b, int &ea, int &eb, PickScratch &sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ta = __shfl_up(ia, o, WAVE), tb = __shfl_up(ib, o, WAVE);
    if (lane >= o) {
      ia += ta;
      ib += tb;
    }
  }
  if (lane == 63) {
    sm.wsum[0][w] = ia;
    sm.wsum[1][w] = ib;
  }
  __syncthreads();
  int oa = 0, ob = 0;
  for (int i = 0; i < w; ++i) {
    oa += sm.wsum[0][i];
    ob += sm.wsum[1][i];
  }
  ea = oa + ia - a;
  eb = ob + ib - b;
  __syncthreads();
}

// [LM] topk_sample over keys[0..N) (fkey of the logits, in LDS): the k largest (equal values at the
// k-th place by increasing index), ordered by decreasing value then increasing index; weights
// exp(double((v - max) / T)) summed in that order, normalised, and the first candidate at which
// the running u - p_1 - ... reaches <= 0 (else the last).  Every thread returns the token.
template <int NT>
__device__ int block_topk(const uint32_t *keys, int N, int k, float temp, double u, PickScratch &sm) {
  const int tid = threadIdx.x;
  // 1. radix select of the k-th largest key, 8 bits a pass from the top
  uint32_t prefix = 0, mask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += NT) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < WAVE) {
      const int l = tid;
      const uint32_t c0 = sm.hist[4 * l], c1 = sm.hist[4 * l + 1], c2 = sm.hist[4 * l + 2], c3 = sm.hist[4 * l + 3];
      uint32_t S = c0 + c1 + c2 + c3;  // inclusive suffix sums over lanes: bins 4l .. 255
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(S, o, WAVE);
        if (l + o < 64) S += t;
      }
      uint32_t Sn = __shfl_down(S, 1, WAVE);
      if (l == 63) Sn = 0;
      if (S >= (uint32_t)need && Sn < (uint32_t)need) {
        uint32_t rem = (uint32_t)need - Sn;
        const uint32_t cs[4] = {c0, c1, c2, c3};
        int dg = 4 * l;
        for (int q = 3; q >= 0; --q) {
          if (cs[q] >= rem) {
            dg = 4 * l + q;
            break;
          }
          rem -= cs[q];
        }
        sm.misc[0] = dg;
        sm.misc[1] = (int)rem;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sm.misc[0] << shift;
    mask |= 0xFFu << shift;
    need = sm.misc[1];
    __syncthreads();
  }
  // prefix is the k-th largest key; `need` of the keys equal to it are taken, the lowest indexes
  const int ngt = k - need;
  // 2. compaction in index order: thread t owns a contiguous run of indexes
  const int ch = (N + NT - 1) / NT;
  const int lo = min(N, tid * ch), hi = min(N, lo + ch);
  int gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    gt += key > prefix;
    eq += key == prefix;
  }
  int gb, eb;
  block_exscan2<NT>(gt, eq, gb, eb, sm);
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    const uint64_t c = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
    if (key > prefix) {
      sm.cand[gb++] = c;
    } else if (key == prefix) {
      if (eb < need) sm.cand[ngt + eb] = c;
      ++eb;
    }
  }
  // 3. bitonic sort, descending, of P >= k entries (padding sorts last)
  int P = 1;
  while (P < k) P <<= 1;
  for (int t = k + tid; t < P; t += NT) sm.cand[t] = 0;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += NT) {
        const int i = 2 * t - (t & (stride - 1)), j = i + stride;
        const uint64_t a = sm.cand[i], b = sm.cand[j];
        const bool up = (i & size) == 0;
        if (up ? (a < b) : (a > b)) {
          sm.cand[i] = b;
          sm.cand[j] = a;
        }
      }
      __syncthreads();
    }
  }
  // 4. weights, their sum in candidate order, normalisation, the inverse-CDF walk
  const float mx = fkey_value((uint32_t)(sm.cand[0] >> 32));
  for (int t = tid; t < k; t += NT) {
    const float v = fkey_value((uint32_t)(sm.cand[t] >> 32));
    const float z = (v - mx) / temp;
    sm.p[t] = exp((double)z);
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int t = 0; t < k; ++t) tot += sm.p[t];
    sm.total = tot;
  }
  __syncthreads();
  const double tot = sm.total;
  for (int t = tid; t < k; t += NT) sm.p[t] = sm.p[t] / tot;
  __syncthreads();
  if (tid == 0) {
    int pick = k - 1;
    double r = u;
    for (int t = 0; t < k; ++t) {
      r -= sm.p[t];
      if (r <= 0.0) {
        pick = t;
        break;
      }
    }
    sm.misc[2] = (int)(0xFFFFFFFFu - (uint32_t)sm.cand[pick]);
  }
  __syncthreads();
  const int tok = sm.misc[2];
  __syncthreads();
  return tok;
}

// --------------------------------------------------------------------------------------------
// The token of head `head` (0 text, 1 + cb codebook cb) of conversation b0 + blockIdx.x, from its
// logits row L + blockIdx.x * ld (N values): greedy (the merge of the head's nparts argmax
// partials, or with nparts = 0 the argmax of the row), top-k temperature sampling or
// full-vocabulary Gumbel-max, as the conversation's SampleCfg says; the conversation's xorshift
// state advances by the draws made.  The token is stored as the single partial part[blockIdx.x *
// stride] that the consumers of the head merge.  Dynamic LDS: N x 4 bytes (top-k keys).
// --------------------------------------------------------------------------------------------
static __global__ __launch_bounds__(PICK_BLOCK) void k_pick(Dims d, Bufs s, int head, const float *__restrict__ L, int ld,
                                                            int N, ArgBest *__restrict__ part, int stride, int nparts,
                                                            int b0) {
  extern __shared__ uint32_t keys[];
  __shared__ PickScratch sm;
  __shared__ ArgBest wb[PICK_BLOCK / WAVE];
  __shared__ uint64_t s_state;
  const int m = blockIdx.x, b = b0 + m;
  const SampleCfg c = s.samp[b];
  const float *l = L + (size_t)m * ld;
  ArgBest *pp = part + (size_t)m * stride;
  if (threadIdx.x == 0) s_state = s.rng[b];
  __syncthreads();
  const uint64_t st0 = s_state;
  const float temp = head == 0 ? c.temp_text : c.temp;
  int tok;
  if (c.mode == PICK_TOPK) {
    for (int i = threadIdx.x; i < N; i += PICK_BLOCK) keys[i] = fkey(l[i]);
    __syncthreads();
    const uint64_t x = xs_next(st0);
    const int k = min(head == 0 ? c.top_k_text : c.top_k, N);
    tok = block_topk<PICK_BLOCK>(keys, N, k, temp, xs_unit(x), sm);
    if (threadIdx.x == 0) s.rng[b] = x;
  } else {
    ArgBest best = arg_none();
    if (c.mode == PICK_GUMBEL) {
      const int ch = (N + PICK_BLOCK - 1) / PICK_BLOCK;
      const int lo = min(N, (int)threadIdx.x * ch), hi = min(N, lo + ch);
      uint64_t x = xs_jump(st0, (uint32_t)lo, s.jump);
      for (int i = lo; i < hi; ++i) best = arg_take(best, gumbel_score(l[i], temp, x), i);
      if (lo < hi && hi == N) s.rng[b] = x;  // the state after N draws
    } else if (nparts > 0) {
      for (int i = threadIdx.x; i < nparts; i += PICK_BLOCK) best = arg_merge(best, pp[i]);
    } else {
      for (int i = threadIdx.x; i < N; i += PICK_BLOCK) best = arg_take(best, l[i], i);
    }
    best = wave_arg(best);
    if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = best;
    __syncthreads();
    ArgBest t = wb[0];
#pragma unroll
    for (int w = 1; w < PICK_BLOCK / WAVE; ++w) t = arg_merge(t, wb[w]);
    tok = t.i < 0 ? 0 : t.i;
  }
  __syncthreads();
  if (threadIdx.x == 0) pp[0] = ArgBest{0.f, tok};
}

}  // namespace mk
