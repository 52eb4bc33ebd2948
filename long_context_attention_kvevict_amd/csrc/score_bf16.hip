// Two-pass fused eviction scorer, bf16 inputs, gfx950 MFMA.
//
// Pass 1 (score_p1_bf16): flash-style online softmax of every window row of a
//   GQA group against one chunk of keys, producing per-chunk (max, sum, o)
//   partials, plus ||v_j||^2 for pass 2.  ("DropKV" page, §3.4: a
//   FlashAttention-2 style forward pass yields each row's log-sum-exp and
//   output; split-K partials are merged afterwards.)
// Merge (score_merge): combines the chunk partials of each row into its
//   log2-sum-exp, o (fp32), ||o||^2 and a bf16 hi/lo split of -2 o.
// Pass 2 (score_p2_bf16): recomputes the logits, forms the softmax weight
//   p = 2^(x - lse2), the distance ||o - v||^2 = ||o||^2 + ||v||^2 - 2 <o, v>
//   with <o, v> from an MFMA contraction, and accumulates
//   (p / (1 - p))^2 ||o - v||^2 over all rows of the group for each key
//   ("DropKV" page, §3.3 window score and §3.4 scoring kernel).
//
// Work decomposition: a workgroup of 4 waves owns one (sequence, KV head,
// row group of 128 rows, key chunk).  Each wave owns 32 rows; the K/V tile of
// 64 keys is staged once in LDS and read by all 4 waves.
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

constexpr int D = 128;          // head dim of the bf16 path
constexpr int KT = 64;          // keys per tile
constexpr int KS = D + 8;       // LDS row stride (bf16 elements) of K/V [key][d] tiles
constexpr int VTS = KT + 8;     // LDS row stride of the transposed V tile [d][key]
constexpr int ROWS = 128;       // rows per workgroup (4 waves x 32)

// Slot s of a 32-key block holds key keymap(s): bits 2 and 3 swapped.  With
// this order the P values a lane holds after the K.Q^T MFMA are 8
// consecutive keys, so the V^T operand of P.V is one 16-byte LDS read.
__device__ __forceinline__ int keymap(int s) {
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}

// Key (within a 32-key block) of accumulator register r of lane half hl in
// the K.Q^T output (slot 8(r/4) + 4hl + r%4 mapped through keymap).
__device__ __forceinline__ int p1_key_of(int r, int hl) {
  return (r & 3) + 4 * ((r >> 2) & 1) + 8 * hl + 16 * (r >> 3);
}

struct ScoreArgs {
  const uint16_t* q_win;   // [S][Hq][w][D]
  const uint16_t* k;       // [Hkv][T][D]
  const uint16_t* v;
  const int32_t* seq_off;  // [S+1]
  int S, Hq, Hkv, w, T, RG, CH, P, causal;
  float c2;                // sm_scale * log2(e)
  float* part_ml;          // [S*Hkv*RG][P][ROWS][2]
  float* part_o;           // [S*Hkv*RG][P][ROWS][D]
  float* vnorm;            // [Hkv][T]
  float* lse2;             // [S*Hkv*RG][ROWS]
  float* no2;              // [S*Hkv*RG][ROWS]
  uint16_t* ohi;           // [S*Hkv*RG][ROWS][D]  bf16 of -2 o
  uint16_t* olo;           // residual
  float* sraw;             // [RG][Hkv][T]
};

// ---------------------------------------------------------------- pass 1
__global__ __launch_bounds__(256, 2) void score_p1_bf16(ScoreArgs a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y / a.RG;
  const int rg = blockIdx.y % a.RG;
  const int s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int c0 = c * a.CH;
  if (c0 >= n) return;
  const int c1 = min(c0 + a.CH, n);

  __shared__ __align__(16) uint16_t Ks[KT * KS];
  __shared__ __align__(16) uint16_t Vt[D * VTS];
  __shared__ __align__(16) float vred[16 * KT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int g = a.Hq / a.Hkv;
  const int R = g * a.w;

  // this lane's query row (N index of the K.Q^T MFMA)
  const int row = rg * ROWS + wave * 32 + col;
  const bool row_ok = row < R;
  const int qh = h * g + (row_ok ? row / a.w : 0);
  const int wi = row_ok ? row % a.w : 0;
  const int pos = n - a.w + wi;   // causal horizon of this row

  bf16x8 qreg[D / 16];
  {
    const uint16_t* qp = a.q_win + ((static_cast<size_t>(s) * a.Hq + qh) * a.w + wi) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (row_ok) t = *reinterpret_cast<const u32x4*>(qp + 16 * kk + 8 * hl);
      qreg[kk] = as_bf16x8(t);
    }
  }

  const uint16_t* kbase = a.k + (static_cast<size_t>(h) * a.T + base) * D;
  const uint16_t* vbase = a.v + (static_cast<size_t>(h) * a.T + base) * D;

  // tile loaders: K as [key][d] (thread -> key tid/16 + 16u, d chunk tid%16);
  // V transposed (thread -> key group kg = tid%16 of 4 keys, d chunk tid/16)
  const int kkey = tid >> 4, kdc = tid & 15;
  const int vkg = tid & 15, vdc = tid >> 4;
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = kt0 + kkey + 16 * u;
      u32x4 t = {0u, 0u, 0u, 0u};
      if (key < c1) t = *reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(key) * D + 8 * kdc);
      kreg[u] = t;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kt0 + 4 * vkg + i;
      u32x4 t = {0u, 0u, 0u, 0u};
      if (key < c1) t = *reinterpret_cast<const u32x4*>(vbase + static_cast<size_t>(key) * D + 8 * vdc);
      vreg[i] = t;
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  load_tile(c0);
  for (int kt0 = c0; kt0 < c1; kt0 += KT) {
    __syncthreads();   // previous tile fully consumed
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<u32x4*>(&Ks[(kkey + 16 * u) * KS + 8 * kdc]) = kreg[u];
    {
      // transpose 4 keys x 8 d into Vt[d][key]; also ||v||^2 partials
      float vsq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = vreg[i][e];
          const float lo = __uint_as_float(wv << 16), hi = __uint_as_float(wv & 0xffff0000u);
          acc = fmaf(lo, lo, acc);
          acc = fmaf(hi, hi, acc);
        }
        vsq[i] = acc;
      }
      *reinterpret_cast<f32x4*>(&vred[vdc * KT + 4 * vkg]) = f32x4{vsq[0], vsq[1], vsq[2], vsq[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // d = 8*vdc + 2e (low halves) and 2e+1 (high halves)
        const uint32_t k0 = vreg[0][e], k1 = vreg[1][e], k2 = vreg[2][e], k3 = vreg[3][e];
        const uint32_t lo01 = (k0 & 0xffffu) | (k1 << 16);
        const uint32_t lo23 = (k2 & 0xffffu) | (k3 << 16);
        const uint32_t hi01 = (k0 >> 16) | (k1 & 0xffff0000u);
        const uint32_t hi23 = (k2 >> 16) | (k3 & 0xffff0000u);
        const int d0 = 8 * vdc + 2 * e;
        *reinterpret_cast<uint2*>(&Vt[d0 * VTS + 4 * vkg]) = make_uint2(lo01, lo23);
        *reinterpret_cast<uint2*>(&Vt[(d0 + 1) * VTS + 4 * vkg]) = make_uint2(hi01, hi23);
      }
    }
    __syncthreads();
    if (tid < KT) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) sum += vred[q * KT + tid];
      if (kt0 + tid < c1) a.vnorm[static_cast<size_t>(h) * a.T + base + kt0 + tid] = sum;
    }
    if (kt0 + KT < c1) load_tile(kt0 + KT);   // prefetch next tile into registers

    // S^T = K . Q^T for the two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sacc[b] = f32x16{};
      const uint16_t* kr = &Ks[(b * 32 + keymap(col)) * KS + 8 * hl];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 16 * kk));
        sacc[b] = mfma32(av, qreg[kk], sacc[b]);
      }
    }
    // scale to log2 units; mask keys past the chunk or the causal horizon
    const bool edge = (kt0 + KT > c1) || (a.causal && kt0 + KT - 1 > n - a.w);
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[b][r] * a.c2;
        if (edge) {
          const int key = kt0 + b * 32 + p1_key_of(r, hl);
          if (key >= c1 || (a.causal && key > pos)) x = -INFINITY;
        }
        sacc[b][r] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, xor32(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float scale = exp2f(m_run - m_use);
    if (__any(scale != 1.f)) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= scale;
    }
    l_run *= scale;
    m_run = m_new;

    bf16x8 pb[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2f(sacc[b][8 * t + 2 * e] - m_use);
          const float p1 = exp2f(sacc[b][8 * t + 2 * e + 1] - m_use);
          l_run += p0 + p1;
          pk[e] = pack_bf16x2(p0, p1);
        }
        pb[b][t] = as_bf16x8(pk);
      }
    }
    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint16_t* vr = &Vt[(db * 32 + col) * VTS + 8 * hl];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4*>(vr + b * 32 + 16 * t));
          oacc[db] = mfma32(av, pb[b][t], oacc[db]);
        }
      }
    }
  }

  const float l_tot = l_run + xor32(l_run);
  if (!row_ok) return;
  const size_t part = (static_cast<size_t>((s * a.Hkv + h) * a.RG + rg)) * a.P + c;
  const int rl = wave * 32 + col;
  if (hl == 0) {
    a.part_ml[(part * ROWS + rl) * 2 + 0] = m_run;
    a.part_ml[(part * ROWS + rl) * 2 + 1] = l_tot;
  }
  float* op = a.part_o + (part * ROWS + rl) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = db * 32 + 8 * q4 + 4 * hl;
      *reinterpret_cast<f32x4*>(op + d) =
          f32x4{oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]};
    }
  }
}

// ---------------------------------------------------------------- merge
// One wave per window row.  Lanes l and l + 32 take alternate chunks (two
// independent load streams); each lane holds DD/32 consecutive features.
// Chunks wholly beyond a row's causal horizon carry max = -inf and weight 0.
template <int DD, bool BF16OUT>
__global__ __launch_bounds__(256) void score_merge(ScoreArgs a, float* o32) {
  constexpr int F = DD / 32;
  const int gr = blockIdx.x * 4 + (threadIdx.x >> 6);   // grp * ROWS + rl
  const int grp = gr / ROWS;
  const int rl = gr % ROWS;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, ln = lane & 31;
  const int s = grp / (a.Hkv * a.RG);
  const int rg = grp % a.RG;
  const int n = a.seq_off[s + 1] - a.seq_off[s];
  const int nch = (n + a.CH - 1) / a.CH;
  const int R = (a.Hq / a.Hkv) * a.w;
  const size_t ro = static_cast<size_t>(gr);
  if (rg * ROWS + rl >= R) {   // padding row of the last row group
    if (lane == 0) { a.lse2[ro] = INFINITY; a.no2[ro] = 0.f; }
    if (half == 0) {
#pragma unroll
      for (int f = 0; f < F; ++f) {
        if (BF16OUT) { a.ohi[ro * DD + ln * F + f] = 0; a.olo[ro * DD + ln * F + f] = 0; }
        else o32[ro * DD + ln * F + f] = 0.f;
      }
    }
    return;
  }
  const size_t cstride_ml = static_cast<size_t>(ROWS) * 2;
  const size_t cstride_o = static_cast<size_t>(ROWS) * DD;
  const float* ml = a.part_ml + (static_cast<size_t>(grp) * a.P * ROWS + rl) * 2;
  const float* po = a.part_o + (static_cast<size_t>(grp) * a.P * ROWS + rl) * DD + ln * F;
  float M = -INFINITY;
  for (int c = lane; c < nch; c += 64) M = fmaxf(M, ml[c * cstride_ml]);
  M = wave_max(M);
  float L = 0.f;
  float acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = 0.f;
#pragma unroll 8
  for (int c = half; c < nch; c += 2) {
    const float m = ml[c * cstride_ml];
    const float l = ml[c * cstride_ml + 1];
    const float wgt = (m == -INFINITY) ? 0.f : exp2f(m - M);
    L = fmaf(l, wgt, L);
    if (F == 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(po + c * cstride_o);
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = fmaf(x[f], wgt, acc[f]);
    } else {
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = fmaf(po[c * cstride_o + f], wgt, acc[f]);
    }
  }
  L += xor32(L);
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] += xor32(acc[f]);
  const float inv = 1.f / L;
  float sq = 0.f;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    acc[f] *= inv;
    sq = fmaf(acc[f], acc[f], sq);
  }
  // sum over the 32 lanes of one half (both halves hold identical values)
  for (int o = 16; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
  if (lane == 0) {
    a.no2[ro] = sq;
    a.lse2[ro] = M + log2f(L);
  }
  if (half == 0) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      if (BF16OUT) {
        const float x = -2.f * acc[f];
        const uint16_t hi = f32_to_bf16(x);
        a.ohi[ro * DD + ln * F + f] = hi;
        a.olo[ro * DD + ln * F + f] = f32_to_bf16(x - bf16_to_f32(hi));
      } else {
        o32[ro * DD + ln * F + f] = acc[f];
      }
    }
  }
}

// ---------------------------------------------------------------- pass 2
__global__ __launch_bounds__(256, 2) void score_p2_bf16(ScoreArgs a) {
  const int c = blockIdx.x;
  const int h = blockIdx.y / a.RG;
  const int rg = blockIdx.y % a.RG;
  const int s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int c0 = c * a.CH;
  if (c0 >= n) return;
  const int c1 = min(c0 + a.CH, n);

  __shared__ __align__(16) uint16_t Ks[KT * KS];
  __shared__ __align__(16) uint16_t Vs[KT * KS];
  __shared__ float red[4 * KT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int g = a.Hq / a.Hkv;
  const int R = g * a.w;
  const size_t grp = static_cast<size_t>((s * a.Hkv + h) * a.RG + rg);

  // A operands: rows wave*32 + col (M index)
  const int arow = rg * ROWS + wave * 32 + col;
  const bool arow_ok = arow < R;
  bf16x8 qa[D / 16], oha[D / 16], ola[D / 16];
  {
    const int qh = h * g + (arow_ok ? arow / a.w : 0);
    const int wi = arow_ok ? arow % a.w : 0;
    const uint16_t* qp = a.q_win + ((static_cast<size_t>(s) * a.Hq + qh) * a.w + wi) * D;
    const uint16_t* hp = a.ohi + (grp * ROWS + wave * 32 + col) * D;
    const uint16_t* lp = a.olo + (grp * ROWS + wave * 32 + col) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (arow_ok) t = *reinterpret_cast<const u32x4*>(qp + 16 * kk + 8 * hl);
      qa[kk] = as_bf16x8(t);
      oha[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(hp + 16 * kk + 8 * hl));
      ola[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(lp + 16 * kk + 8 * hl));
    }
  }
  // per-row constants of the output layout: rows 8(r/4) + 4hl + r%4
  float lse2c[16], no2c[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rl = wave * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
    lse2c[r] = a.lse2[grp * ROWS + rl];
    no2c[r] = a.no2[grp * ROWS + rl];
  }

  const uint16_t* kbase = a.k + (static_cast<size_t>(h) * a.T + base) * D;
  const uint16_t* vbase = a.v + (static_cast<size_t>(h) * a.T + base) * D;
  const float* vnb = a.vnorm + static_cast<size_t>(h) * a.T + base;
  float* sout = a.sraw + (static_cast<size_t>(rg) * a.Hkv + h) * a.T + base;

  const int lkey = tid >> 4, ldc = tid & 15;
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = kt0 + lkey + 16 * u;
      u32x4 tk = {0u, 0u, 0u, 0u}, tv = {0u, 0u, 0u, 0u};
      if (key < c1) {
        tk = *reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(key) * D + 8 * ldc);
        tv = *reinterpret_cast<const u32x4*>(vbase + static_cast<size_t>(key) * D + 8 * ldc);
      }
      kreg[u] = tk;
      vreg[u] = tv;
    }
  };

  load_tile(c0);
  for (int kt0 = c0; kt0 < c1; kt0 += KT) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<u32x4*>(&Ks[(lkey + 16 * u) * KS + 8 * ldc]) = kreg[u];
      *reinterpret_cast<u32x4*>(&Vs[(lkey + 16 * u) * KS + 8 * ldc]) = vreg[u];
    }
    __syncthreads();
    if (kt0 + KT < c1) load_tile(kt0 + KT);
    const bool edge = (kt0 + KT > c1) || (a.causal && kt0 + KT - 1 > n - a.w);

#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int key = kt0 + b * 32 + col;
      const float vn2 = (key < c1) ? vnb[key] : 0.f;
      f32x16 sacc = f32x16{};
      f32x16 gacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) gacc[r] = no2c[r];
      const uint16_t* kr = &Ks[(b * 32 + col) * KS + 8 * hl];
      const uint16_t* vr = &Vs[(b * 32 + col) * KS + 8 * hl];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 kb = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 16 * kk));
        const bf16x8 vb = as_bf16x8(*reinterpret_cast<const u32x4*>(vr + 16 * kk));
        sacc = mfma32(qa[kk], kb, sacc);
        gacc = mfma32(oha[kk], vb, gacc);
        gacc = mfma32(ola[kk], vb, gacc);
      }
      float sc = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fmaf(sacc[r], a.c2, -lse2c[r]);
        if (edge) {
          bool ok = key < c1;
          if (a.causal) {
            const int rrow = rg * ROWS + wave * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const int wi = (rrow < R) ? rrow % a.w : 0;
            ok = ok && (key <= n - a.w + wi);
          }
          if (!ok) x = -INFINITY;
        }
        const float y = exp2f(-x) - 1.f;                 // (1 - p) / p
        const float y2 = fmaf(y, y, 9.094947e-13f);       // + 2^-40 keeps 1/y2 finite
        const float d2 = gacc[r] + vn2;                   // ||o - v||^2
        sc = fmaf(d2, __builtin_amdgcn_rcpf(y2), sc);
      }
      sc += xor32(sc);
      if (hl == 0) red[wave * KT + b * 32 + col] = sc;
    }
    __syncthreads();
    if (tid < KT && kt0 + tid < c1)
      sout[kt0 + tid] = (red[tid] + red[KT + tid]) + (red[2 * KT + tid] + red[3 * KT + tid]);
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_score_bf16(const ScoreGeom& G, const void* q_win, const void* k, const void* v,
                             const int32_t* seq_off, float sm_scale, int causal, void* ws,
                             hipStream_t st) {
  ScoreArgs a;
  a.q_win = static_cast<const uint16_t*>(q_win);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.seq_off = seq_off;
  a.S = G.S; a.Hq = G.Hq; a.Hkv = G.Hkv; a.w = G.w; a.T = G.T;
  a.RG = G.RG; a.CH = G.CH; a.P = G.P; a.causal = causal;
  a.c2 = sm_scale * kLog2e;
  char* base = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float*>(base + G.off_part_ml);
  a.part_o = reinterpret_cast<float*>(base + G.off_part_o);
  a.vnorm = reinterpret_cast<float*>(base + G.off_vnorm);
  a.lse2 = reinterpret_cast<float*>(base + G.off_lse2);
  a.no2 = reinterpret_cast<float*>(base + G.off_no2);
  a.ohi = reinterpret_cast<uint16_t*>(base + G.off_ohi);
  a.olo = reinterpret_cast<uint16_t*>(base + G.off_olo);
  a.sraw = reinterpret_cast<float*>(base + G.off_sraw);

  dim3 grid(G.P, G.Hkv * G.RG, G.S);
  stage_begin(ST_SCORE_P1, st);
  hipLaunchKernelGGL(score_p1_bf16, grid, dim3(256), 0, st, a);
  stage_end(ST_SCORE_P1, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(ST_SCORE_MERGE, st);
  hipLaunchKernelGGL((score_merge<D, true>), dim3(G.S * G.Hkv * G.RG * (ROWS / 4)), dim3(256), 0, st, a,
                     static_cast<float*>(nullptr));
  stage_end(ST_SCORE_MERGE, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(ST_SCORE_P2, st);
  hipLaunchKernelGGL(score_p2_bf16, grid, dim3(256), 0, st, a);
  stage_end(ST_SCORE_P2, st);
  return hipGetLastError();
}

hipError_t launch_merge_f32(const ScoreGeom& G, const int32_t* seq_off, void* ws, hipStream_t st) {
  ScoreArgs a = {};
  a.seq_off = seq_off;
  a.S = G.S; a.Hq = G.Hq; a.Hkv = G.Hkv; a.w = G.w; a.T = G.T;
  a.RG = G.RG; a.CH = G.CH; a.P = G.P;
  char* base = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float*>(base + G.off_part_ml);
  a.part_o = reinterpret_cast<float*>(base + G.off_part_o);
  a.lse2 = reinterpret_cast<float*>(base + G.off_lse2);
  a.no2 = reinterpret_cast<float*>(base + G.off_no2);
  float* o32 = reinterpret_cast<float*>(base + G.off_ohi);
  dim3 grid(G.S * G.Hkv * G.RG * (ROWS / 4));
  if (G.d == 64) hipLaunchKernelGGL((score_merge<64, false>), grid, dim3(256), 0, st, a, o32);
  else hipLaunchKernelGGL((score_merge<128, false>), grid, dim3(256), 0, st, a, o32);
  return hipGetLastError();
}

}  // namespace kve
