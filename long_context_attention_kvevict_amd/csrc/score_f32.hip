// fp32 eviction scorer (vector ALU; used for fp32 inputs, d in {64, 128}).
//
// Same two passes as the bf16 MFMA path ("DropKV" page, §3.4), written for
// plain fp32 arithmetic: pass 1 produces per-chunk softmax partials of every
// window row (merged by score_merge into lse2 and o), pass 2 assigns one key
// per thread and accumulates (p / (1 - p))^2 ||o - v||^2 over all rows of the
// GQA group, forming o - v explicitly.
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

constexpr int ROWS32 = 128;

struct F32Args {
  const float* q_win;
  const float* k;
  const float* v;
  const int32_t* seq_off;
  int S, Hq, Hkv, w, T, RG, CH, P, causal;
  float c2;
  float* part_ml;
  float* part_o;
  float* lse2;
  float* no2;
  float* o32;
  float* sraw;
};

// One wave per window row, four rows per workgroup (blockIdx.y = (KV head,
// row group, block of 4 rows)): the wave's lanes take 64 keys per step, each
// forming its key's logit against the row's query (broadcast a feature at a
// time from the lane that holds it), then the wave's online softmax and
// o += p v, where lane l owns features l, l + 64, ...
constexpr int P1F32_ROWS = 4;

template <int DD>
__global__ __launch_bounds__(256) void score_p1_f32(F32Args a) {
  static_assert(DD % 64 == 0, "whole features per lane");
  constexpr int F = DD / 64;
  const int c = blockIdx.x;
  const int rb = blockIdx.y % (ROWS32 / P1F32_ROWS);
  const int hg = blockIdx.y / (ROWS32 / P1F32_ROWS);
  const int h = hg / a.RG;
  const int rg = hg % a.RG;
  const int s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int c0 = c * a.CH;
  if (c0 >= n) return;
  const int c1 = min(c0 + a.CH, n);
  const int g = a.Hq / a.Hkv;
  const int R = g * a.w;
  const int lane = threadIdx.x & 63;
  const int rl = rb * P1F32_ROWS + (threadIdx.x >> 6);
  const int row = rg * ROWS32 + rl;
  if (row >= R) return;   // whole waves; no workgroup barrier below
  const int qh = h * g + row / a.w;
  const int wi = row % a.w;
  const int pos = n - a.w + wi;
  const float* kb = a.k + (static_cast<size_t>(h) * a.T + base) * DD;
  const float* vb = a.v + (static_cast<size_t>(h) * a.T + base) * DD;
  const float* qp = a.q_win + ((static_cast<size_t>(s) * a.Hq + qh) * a.w + wi) * DD;
  float qv[F];
#pragma unroll
  for (int f = 0; f < F; ++f) qv[f] = qp[64 * f + lane];

  float m_run = -INFINITY, l_run = 0.f;
  float o[F];
#pragma unroll
  for (int f = 0; f < F; ++f) o[f] = 0.f;
  for (int t0 = c0; t0 < c1; t0 += 64) {
    const int key = t0 + lane;
    // the step's 64 value rows are loaded with its keys (they do not depend
    // on the weights); rows past the chunk read its last row, with p = 0
    float vv[64][F];
#pragma unroll
    for (int jj = 0; jj < 64; ++jj) {
      const float* vr = vb + static_cast<size_t>(min(t0 + jj, c1 - 1)) * DD;
#pragma unroll
      for (int f = 0; f < F; ++f) vv[jj][f] = vr[64 * f + lane];
    }
    float x = -INFINITY;
    if (key < c1 && !(a.causal && key > pos)) {
      const float4* kr = reinterpret_cast<const float4*>(kb + static_cast<size_t>(key) * DD);
      float acc = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < DD / 4; ++e4) {
        const float4 kk = kr[e4];
        const int e = 4 * e4;
        acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv[e / 64]), e % 64)), kk.x, acc);
        acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv[e / 64]), e % 64 + 1)), kk.y, acc);
        acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv[e / 64]), e % 64 + 2)), kk.z, acc);
        acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv[e / 64]), e % 64 + 3)), kk.w, acc);
      }
      x = acc * a.c2;
    }
    const float m_new = fmaxf(m_run, wave_max(x));
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float scale = exp2f(m_run - m_use);
    const float p = exp2f(x - m_use);
    l_run = l_run * scale + p;       // per-lane partial, summed at the end
#pragma unroll
    for (int f = 0; f < F; ++f) o[f] *= scale;
    m_run = m_new;
    // keys past the chunk (or hidden) have p = 0
#pragma unroll
    for (int jj = 0; jj < 64; ++jj) {
      const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), jj));
#pragma unroll
      for (int f = 0; f < F; ++f) o[f] = fmaf(pj, vv[jj][f], o[f]);
    }
  }
  const float lt = wave_sum(l_run);
  const size_t grp = static_cast<size_t>((s * a.Hkv + h) * a.RG + rg);
  const size_t pr = (grp * a.P + c) * ROWS32 + rl;
  if (lane == 0) {   // the record of the bf16 path with no dominant-key candidate
    float* rec = a.part_ml + pr * kScoreRec;
    rec[0] = m_run;
    rec[1] = lt;
    rec[2] = 0.f;
    rec[3] = __uint_as_float(0xffffffffu);   // key -1
  }
#pragma unroll
  for (int f = 0; f < F; ++f) a.part_o[pr * DD + 64 * f + lane] = o[f];
}

// One key per lane, 64 keys per workgroup slice (blockIdx.x = chunk x 4
// slices); the 4 waves take the same keys and every 4th row of the group
// (rows staged in LDS 32 at a time), and their sums are added in wave order.
template <int DD>
__global__ __launch_bounds__(256) void score_p2_f32(F32Args a) {
  const int c = blockIdx.x >> 2, slice = blockIdx.x & 3;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int c0 = c * a.CH;
  if (c0 >= n) return;
  const int c1 = min(c0 + a.CH, n);
  const int g = a.Hq / a.Hkv;
  const int R = g * a.w;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  __shared__ float qs[32 * DD];
  __shared__ float os[32 * DD];
  __shared__ float ls[32];
  __shared__ int ps[32];
  __shared__ float part[4][64];

  const float* kb = a.k + (static_cast<size_t>(h) * a.T + base) * DD;
  const float* vb = a.v + (static_cast<size_t>(h) * a.T + base) * DD;

  for (int t0 = c0 + 64 * slice; t0 < c1; t0 += 256) {
    const int key = t0 + lane;
    const bool kok = key < c1;
    float kr[DD], vr[DD];
#pragma unroll
    for (int e = 0; e < DD; ++e) {
      kr[e] = kok ? kb[static_cast<size_t>(key) * DD + e] : 0.f;
      vr[e] = kok ? vb[static_cast<size_t>(key) * DD + e] : 0.f;
    }
    float sc = 0.f;
    for (int r0 = 0; r0 < R; r0 += 32) {
      __syncthreads();
      for (int i = tid; i < 32 * DD; i += 256) {
        const int rr = r0 + i / DD, e = i % DD;
        float qv = 0.f, ov = 0.f;
        if (rr < R) {
          const int qh = h * g + rr / a.w, wi = rr % a.w;
          qv = a.q_win[((static_cast<size_t>(s) * a.Hq + qh) * a.w + wi) * DD + e];
          const size_t grp = static_cast<size_t>((s * a.Hkv + h) * a.RG + rr / ROWS32);
          ov = a.o32[(grp * ROWS32 + rr % ROWS32) * DD + e];
        }
        qs[i] = qv;
        os[i] = ov;
      }
      if (tid < 32) {
        const int rr = r0 + tid;
        if (rr < R) {
          const size_t grp = static_cast<size_t>((s * a.Hkv + h) * a.RG + rr / ROWS32);
          ls[tid] = a.lse2[grp * ROWS32 + rr % ROWS32];
          ps[tid] = n - a.w + rr % a.w;
        } else {
          ls[tid] = INFINITY;
          ps[tid] = -1;
        }
      }
      __syncthreads();
      if (!kok) continue;
      const int rn = min(32, R - r0);
      for (int r = wave; r < rn; r += 4) {
        if (a.causal && key > ps[r]) continue;
        float dot = 0.f, d2 = 0.f;
#pragma unroll
        for (int e = 0; e < DD; ++e) {
          dot = fmaf(qs[r * DD + e], kr[e], dot);
          const float df = os[r * DD + e] - vr[e];
          d2 = fmaf(df, df, d2);
        }
        const float x = fmaf(dot, a.c2, -ls[r]);
        const float y = exp2f(-x) - 1.f;
        const float y2 = fmaf(y, y, 9.094947e-13f);
        sc = fmaf(d2, 1.f / y2, sc);
      }
    }
    __syncthreads();   // every wave's rows of these keys done
    part[wave][lane] = sc;
    __syncthreads();
    if (wave == 0 && kok)
      a.sraw[static_cast<size_t>(h) * a.T + base + key] = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
  }
}

hipError_t launch_score_f32(const ScoreGeom& G, const void* q_win, const void* k, const void* v,
                            const int32_t* seq_off, float sm_scale, int causal, void* ws,
                            hipStream_t st) {
  F32Args a;
  a.q_win = static_cast<const float*>(q_win);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.seq_off = seq_off;
  a.S = G.S; a.Hq = G.Hq; a.Hkv = G.Hkv; a.w = G.w; a.T = G.T;
  a.RG = G.RG; a.CH = G.CH; a.P = G.P; a.causal = causal;
  a.c2 = sm_scale * kLog2e;
  char* base = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float*>(base + G.off_part_ml);
  a.part_o = reinterpret_cast<float*>(base + G.off_part_o);
  a.lse2 = reinterpret_cast<float*>(base + G.off_lse2);
  a.no2 = reinterpret_cast<float*>(base + G.off_no2);
  a.o32 = reinterpret_cast<float*>(base + G.off_ohi);
  a.sraw = reinterpret_cast<float*>(base + G.off_sraw);
  dim3 grid(G.P, G.Hkv * G.RG * (ROWS32 / P1F32_ROWS), G.S);
  stage_begin(ST_SCORE_P1, st);
  if (G.d == 64) hipLaunchKernelGGL(score_p1_f32<64>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(score_p1_f32<128>, grid, dim3(256), 0, st, a);
  stage_end(ST_SCORE_P1, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(ST_SCORE_MERGE, st);
  e = launch_merge_f32(G, seq_off, ws, st);
  stage_end(ST_SCORE_MERGE, st);
  if (e != hipSuccess) return e;
  dim3 grid2(G.P * 4, G.Hkv, G.S);
  stage_begin(ST_SCORE_P2, st);
  if (G.d == 64) hipLaunchKernelGGL(score_p2_f32<64>, grid2, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(score_p2_f32<128>, grid2, dim3(256), 0, st, a);
  stage_end(ST_SCORE_P2, st);
  return hipGetLastError();
}

}  // namespace kve
