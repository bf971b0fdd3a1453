// Causal attention of a teacher-forced prefill chunk on the matrix cores ([LM] attend for every
// position of the chunk: softmax(q . k_j / sqrt(hd)) . v_j over the cached positions j <= pos).
//
// The chunk's rows sit at positions pos0 .. pos0 + rows - 1 of one conversation, all below the
// window and the cache capacity (the caller runs only such chunks as row batches), so cache slot j
// holds position j and row r attends to slots 0 .. pos0 + r.  A block takes one head and
// PFA_WAVES * 32 consecutive rows; a wave owns 32 rows.  The block walks the keys in tiles of 32
// positions, staged in LDS (float32) and shared by its waves; each wave forms
//   S^T = K Q^T     (v_mfma_f32_32x32x2_f32: A = the key tile, B = its 32 query rows)
//   O^T += V^T P^T  (A = the value tile, B = the tile's probabilities)
// in float32 with an online softmax (running max and sum per row, the partial output rescaled
// when the max grows).  With the transposed products a lane's column is its own query row in both,
// so the probabilities a lane computes are the B operand it supplies: lane l holds, for query
// l % 32, the keys (i / 4) * 8 + 4 (l / 32) + i % 4 (i < 16) of the score tile, and the value
// product takes the key of its step from the same slot.  The head dimensions are summed in the
// order a lane holds them: step s of the score product pairs dimension (hd / 2) (l / 32) + s of
// both operands.
#pragma once
#include "gemm.h"
#include "kernels.h"

namespace mk {

constexpr int PFA_WAVES = 4;             // waves per block (32 query rows each)
constexpr int PFA_KT = 32;               // key positions per tile
constexpr int PFA_ROWS = PFA_WAVES * 32;  // query rows per block

typedef float pfa_f32x16 __attribute__((ext_vector_type(16)));

// Grid (H, ceil(rows / PFA_ROWS)), PFA_WAVES * 64 threads.  Reads aq.q (rows x D, roped queries)
// and the conversation's cache of `layer`; writes row r's head slice of the output to aq.xo (bf16
// hi and lo planes, row stride aq.ldxo) when set, else to aq.o (rows x D floats).
template <typename KT, int HD>
__global__ __launch_bounds__(PFA_WAVES * 64) void k_attn_pf(Dims d, KV<KT> kv, int layer, AttnQ aq, int rows) {
  constexpr int LD = HD + 4;      // padded LDS row: the key-tile reads of 8 lanes hit distinct banks
  constexpr int QH = HD / 2;      // score-product steps per lane half
  constexpr int DT = HD / 32;     // output tiles of 32 dimensions; tile t, row m holds dim DT m + t
  constexpr int NT = PFA_WAVES * 64;
  constexpr int LPR = HD / 4;     // float4 pieces per cached row
  constexpr int PPT = PFA_KT * LPR / NT;  // pieces per thread per tile, of K and of V
  static_assert(HD % 32 == 0 && PPT >= 1 && (PFA_KT * LPR) % NT == 0, "tile shape");
  __shared__ __align__(16) float ks[2][PFA_KT][LD];
  __shared__ __align__(16) float vs[2][PFA_KT][LD];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int rb0 = blockIdx.y * PFA_ROWS;
  const int rb1 = min(rows, rb0 + PFA_ROWS);
  const int qw0 = rb0 + wave * 32;
  const int nkeys = (int)(aq.pos0 + rb1);  // keys of the block's last row: slots 0 .. pos0 + rb1 - 1
  const int ntiles = (nkeys + PFA_KT - 1) / PFA_KT;
  const size_t base = kv_index(d, aq.conv, layer, 0, h, 0);
  constexpr int PS = HD;  // elements from one cached position of the head to the next
  const float scale = 1.0f / sqrtf((float)HD);

  // this lane's query: row qw0 + l32 (zero past the chunk), dims QH g .. QH g + QH - 1
  const int qrow = qw0 + l32;
  const bool qok = qrow < rows;
  const int64_t qpos = aq.pos0 + qrow;
  float qr[QH];
  {
    const float *qp = aq.q + (size_t)(qok ? qrow : 0) * d.D + h * HD + QH * g;
#pragma unroll
    for (int s = 0; s < QH; s += 4) {
      const float4 t = qok ? *reinterpret_cast<const float4 *>(qp + s) : float4{0.f, 0.f, 0.f, 0.f};
      qr[s] = t.x;
      qr[s + 1] = t.y;
      qr[s + 2] = t.z;
      qr[s + 3] = t.w;
    }
  }
  // the wave's last row's position: tiles past it hold no key of its rows
  const int64_t wlast = aq.pos0 + min(qw0 + 31, rows - 1);
  const bool wactive = qw0 < rows;

  // a tile's loads: thread t takes pieces t + NT i of the K and of the V tile (piece p: key p / LPR,
  // dims 4 (p % LPR) ..), positions past nkeys read as zero
  float4 kreg[PPT], vreg[PPT];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = threadIdx.x + NT * i;
      const int key = tile * PFA_KT + p / LPR, c = 4 * (p % LPR);
      float kf[4] = {0.f, 0.f, 0.f, 0.f}, vf[4] = {0.f, 0.f, 0.f, 0.f};
      if (key < nkeys) {
        ld_row<4>(kv.k + base + (size_t)key * PS + c, kf);
        ld_row<4>(kv.v + base + (size_t)key * PS + c, vf);
      }
      kreg[i] = float4{kf[0], kf[1], kf[2], kf[3]};
      vreg[i] = float4{vf[0], vf[1], vf[2], vf[3]};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = threadIdx.x + NT * i;
      *reinterpret_cast<float4 *>(&ks[buf][p / LPR][4 * (p % LPR)]) = kreg[i];
      *reinterpret_cast<float4 *>(&vs[buf][p / LPR][4 * (p % LPR)]) = vreg[i];
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  pfa_f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) load_tile(tile + 1);
    const int k0 = tile * PFA_KT;
    if (wactive && (int64_t)k0 <= wlast) {
      // scores: S^T[key][query] over the head dims
      pfa_f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      const float *krow = &ks[buf][l32][QH * g];
#pragma unroll
      for (int s = 0; s < QH; s += 4) {
        const float4 k4 = *reinterpret_cast<const float4 *>(krow + s);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.x, qr[s], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.y, qr[s + 1], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.z, qr[s + 2], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.w, qr[s + 3], sacc, 0, 0, 0);
      }
      // scale, causal mask, online softmax for this lane's query
      float p[16];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + (i >> 2) * 8 + 4 * g + (i & 3);
        p[i] = (int64_t)key <= qpos ? sacc[i] * scale : -INFINITY;
        mx = fmaxf(mx, p[i]);
      }
      mx = xor32_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float corr = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = p[i] == -INFINITY ? 0.f : expf(p[i] - m_new);
        rs += p[i];
      }
      rs = xor32_sum(rs);
      l_run = l_run * corr + rs;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= corr;
      // O^T[dim][query] += V^T P^T: step i takes key (i / 4) * 8 + 4 g + i % 4 of the tile
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float *vrow = &vs[buf][(i >> 2) * 8 + 4 * g + (i & 3)][DT * l32];
        float vv[DT];
        if constexpr (DT % 4 == 0) {
#pragma unroll
          for (int t = 0; t < DT; t += 4) {
            const float4 v4 = *reinterpret_cast<const float4 *>(vrow + t);
            vv[t] = v4.x;
            vv[t + 1] = v4.y;
            vv[t + 2] = v4.z;
            vv[t + 3] = v4.w;
          }
        } else {
#pragma unroll
          for (int t = 0; t < DT; t += 2) {
            const float2 v2 = *reinterpret_cast<const float2 *>(vrow + t);
            vv[t] = v2.x;
            vv[t + 1] = v2.y;
          }
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) o[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[t], p[i], o[t], 0, 0, 0);
      }
    }
    if (tile + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
  if (!qok) return;
  // lane l holds dims DT ((i / 4) * 8 + 4 g + i % 4) + t of query row qw0 + l32
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = (i >> 2) * 8 + 4 * g + (i & 3);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int e = h * HD + DT * m + t;
      const float v = o[t][i] / l_run;
      if (aq.xo) {
        bf16_t *row = aq.xo + (size_t)qrow * aq.ldxo;
        const bf16_t hi = f2bf(v);
        row[e] = hi;
        row[d.D + e] = f2bf(v - bf2f(hi));
      } else {
        aq.o[(size_t)qrow * d.D + e] = v;
      }
    }
  }
}

// The same attention on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) for 128-dim heads: q, k, v
// and the probabilities are split into bf16 hi = bf16(x) and lo = bf16(x - hi) parts (the
// hardware's round-to-nearest-even conversion, two values per instruction), and every product is
// formed as hi.hi + hi.lo + lo.hi with float32 accumulation (about 16 significant bits, the lo.lo
// term below 2^-16 of the product), at a sixth of the float32 matrix cores' cycles per tile.  Keys,
// queries and the lane layout are those of k_attn_pf: S^T = K Q^T (step s of 16 head dimensions
// takes, in lane half g, dimensions 16 s + 8 g .. + 7 of both operands) and O^T += V^T P^T, whose
// step s2 of 16 keys takes, in lane half g, the lane's own probabilities i = 8 s2 .. 8 s2 + 7
// (keys (i / 4) * 8 + 4 g + i % 4).  The value tile is stored transposed ([dim][key]) so that those
// keys are two 8-byte runs of one LDS row.
__device__ __forceinline__ void pfa_split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  const __bf16 la = (__bf16)(a - (float)ha), lb = (__bf16)(b - (float)hb);
  hi = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
  lo = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
}

template <typename KT>
__global__ __launch_bounds__(PFA_WAVES * 64) void k_attn_pf3(Dims d, KV<KT> kv, int layer, AttnQ aq, int rows) {
  constexpr int HD = 128;
  constexpr int KLD = HD + 8;      // bf16 per key row: 16 lanes' 16-byte reads land on 16 slots
  constexpr int VLD = PFA_KT + 4;  // bf16 per transposed value row: 32 lanes' 8-byte reads on 32 bank pairs
  constexpr int NT = PFA_WAVES * 64;
  constexpr int LPR = HD / 4;
  constexpr int PPT = PFA_KT * LPR / NT;
  static_assert(PPT >= 1 && (PFA_KT * LPR) % NT == 0, "tile shape");
  __shared__ __align__(16) bf16_t kh[2][PFA_KT][KLD], kl[2][PFA_KT][KLD];
  __shared__ __align__(16) bf16_t vh[2][HD][VLD], vl[2][HD][VLD];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int rb0 = blockIdx.y * PFA_ROWS;
  const int rb1 = min(rows, rb0 + PFA_ROWS);
  const int qw0 = rb0 + wave * 32;
  const int nkeys = (int)(aq.pos0 + rb1);
  const int ntiles = (nkeys + PFA_KT - 1) / PFA_KT;
  const size_t base = kv_index(d, aq.conv, layer, 0, h, 0);
  constexpr int PS = HD;
  const float scale = 1.0f / sqrtf((float)HD);

  // this lane's query (row qw0 + l32, zero past the chunk): step s holds dims 16 s + 8 g .. + 7
  const int qrow = qw0 + l32;
  const bool qok = qrow < rows;
  const int64_t qpos = aq.pos0 + qrow;
  uint4 qh[HD / 16], ql[HD / 16];
  {
    const float *qp = aq.q + (size_t)(qok ? qrow : 0) * d.D + h * HD + 8 * g;
#pragma unroll
    for (int st = 0; st < HD / 16; ++st) {
      const float4 t0 = qok ? *reinterpret_cast<const float4 *>(qp + 16 * st) : float4{0.f, 0.f, 0.f, 0.f};
      const float4 t1 = qok ? *reinterpret_cast<const float4 *>(qp + 16 * st + 4) : float4{0.f, 0.f, 0.f, 0.f};
      pfa_split2(t0.x, t0.y, qh[st].x, ql[st].x);
      pfa_split2(t0.z, t0.w, qh[st].y, ql[st].y);
      pfa_split2(t1.x, t1.y, qh[st].z, ql[st].z);
      pfa_split2(t1.z, t1.w, qh[st].w, ql[st].w);
    }
  }
  const int64_t wlast = aq.pos0 + min(qw0 + 31, rows - 1);
  const bool wactive = qw0 < rows;

  // keys: four dims of one key per piece; values: thread t takes dim t % HD of VK keys, so that
  // its transposed-tile writes are 8-byte runs of four keys and a wave's lanes write consecutive
  // rows (the stride the reads use: no bank conflicts)
  constexpr int VK = PFA_KT * HD / NT;
  static_assert(NT % HD == 0 && VK % 4 == 0, "value tile shape");
  const int vd = threadIdx.x % HD, vk0 = VK * (threadIdx.x / HD);
  float4 kreg[PPT];
  float vreg[VK];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = threadIdx.x + NT * i;
      const int key = tile * PFA_KT + p / LPR, c = 4 * (p % LPR);
      float kf[4] = {0.f, 0.f, 0.f, 0.f};
      if (key < nkeys) ld_row<4>(kv.k + base + (size_t)key * PS + c, kf);
      kreg[i] = float4{kf[0], kf[1], kf[2], kf[3]};
    }
#pragma unroll
    for (int j = 0; j < VK; ++j) {
      const int key = tile * PFA_KT + vk0 + j;
      vreg[j] = key < nkeys ? to_f(kv.v[base + (size_t)key * PS + vd]) : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = threadIdx.x + NT * i;
      const int key = p / LPR, c = 4 * (p % LPR);
      uint32_t h0, l0, h1, l1;
      pfa_split2(kreg[i].x, kreg[i].y, h0, l0);
      pfa_split2(kreg[i].z, kreg[i].w, h1, l1);
      *reinterpret_cast<uint2 *>(&kh[buf][key][c]) = uint2{h0, h1};
      *reinterpret_cast<uint2 *>(&kl[buf][key][c]) = uint2{l0, l1};
    }
#pragma unroll
    for (int q = 0; q < VK / 4; ++q) {
      uint32_t h0, l0, h1, l1;
      pfa_split2(vreg[4 * q], vreg[4 * q + 1], h0, l0);
      pfa_split2(vreg[4 * q + 2], vreg[4 * q + 3], h1, l1);
      *reinterpret_cast<uint2 *>(&vh[buf][vd][vk0 + 4 * q]) = uint2{h0, h1};
      *reinterpret_cast<uint2 *>(&vl[buf][vd][vk0 + 4 * q]) = uint2{l0, l1};
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  pfa_f32x16 o[HD / 32];
#pragma unroll
  for (int t = 0; t < HD / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) load_tile(tile + 1);
    const int k0 = tile * PFA_KT;
    if (wactive && (int64_t)k0 <= wlast) {
      pfa_f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int st = 0; st < HD / 16; ++st) {
        const uint4 ah = *reinterpret_cast<const uint4 *>(&kh[buf][l32][16 * st + 8 * g]);
        const uint4 al = *reinterpret_cast<const uint4 *>(&kl[buf][l32][16 * st + 8 * g]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(qh[st]), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(ql[st]), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al), as_bf16x8(qh[st]), sacc, 0, 0, 0);
      }
      float p[16];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + (i >> 2) * 8 + 4 * g + (i & 3);
        p[i] = (int64_t)key <= qpos ? sacc[i] * scale : -INFINITY;
        mx = fmaxf(mx, p[i]);
      }
      mx = xor32_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float corr = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = p[i] == -INFINITY ? 0.f : expf(p[i] - m_new);
        rs += p[i];
      }
      rs = xor32_sum(rs);
      l_run = l_run * corr + rs;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < HD / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= corr;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint4 ph, pl;
        pfa_split2(p[8 * s2], p[8 * s2 + 1], ph.x, pl.x);
        pfa_split2(p[8 * s2 + 2], p[8 * s2 + 3], ph.y, pl.y);
        pfa_split2(p[8 * s2 + 4], p[8 * s2 + 5], ph.z, pl.z);
        pfa_split2(p[8 * s2 + 6], p[8 * s2 + 7], ph.w, pl.w);
        const int ka = 16 * s2 + 4 * g;  // keys ka .. ka + 3 and ka + 8 .. ka + 11
#pragma unroll
        for (int t = 0; t < HD / 32; ++t) {
          const int dm = 32 * t + l32;
          const uint2 h0 = *reinterpret_cast<const uint2 *>(&vh[buf][dm][ka]);
          const uint2 h1 = *reinterpret_cast<const uint2 *>(&vh[buf][dm][ka + 8]);
          const uint2 l0 = *reinterpret_cast<const uint2 *>(&vl[buf][dm][ka]);
          const uint2 l1 = *reinterpret_cast<const uint2 *>(&vl[buf][dm][ka + 8]);
          const uint4 vhh{h0.x, h0.y, h1.x, h1.y}, vll{l0.x, l0.y, l1.x, l1.y};
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vhh), as_bf16x8(ph), o[t], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vhh), as_bf16x8(pl), o[t], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vll), as_bf16x8(ph), o[t], 0, 0, 0);
        }
      }
    }
    if (tile + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
  if (!qok) return;
  // lane l holds dims 32 t + (i / 4) * 8 + 4 g + i % 4 of query row qw0 + l32
#pragma unroll
  for (int t = 0; t < HD / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = h * HD + 32 * t + (i >> 2) * 8 + 4 * g + (i & 3);
      const float v = o[t][i] / l_run;
      if (aq.xo) {
        bf16_t *row = aq.xo + (size_t)qrow * aq.ldxo;
        const bf16_t hi = f2bf(v);
        row[e] = hi;
        row[d.D + e] = f2bf(v - bf2f(hi));
      } else {
        aq.o[(size_t)qrow * d.D + e] = v;
      }
    }
}

}  // namespace mk
