// Key-axis max pooling of the raw window scores ("A Probabilistic
// Interpretation of KV Cache Eviction", App. D, SnapKV: pooling along the
// key axis).  Width-k window centred on each key, clipped to the sequence.
// Also sums the per-row-group partial score planes in a fixed order.
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

__global__ __launch_bounds__(256) void pool_max(const float* __restrict__ sraw, const int32_t* __restrict__ seq_off,
                                                int S, int Hkv, int T, int planes, int radius,
                                                float* __restrict__ out) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (t >= T) return;
  int lo = 0, hi = S;   // find s with seq_off[s] <= t < seq_off[s+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seq_off[mid] <= t) lo = mid; else hi = mid;
  }
  const int a = seq_off[lo], b = seq_off[lo + 1];
  const int j0 = max(a, t - radius), j1 = min(b - 1, t + radius);
  float m = -INFINITY;
  for (int j = j0; j <= j1; ++j) {
    float v = 0.f;
    for (int p = 0; p < planes; ++p) v += sraw[(static_cast<size_t>(p) * Hkv + h) * T + j];
    m = fmaxf(m, v);
  }
  out[static_cast<size_t>(h) * T + t] = m;
}

hipError_t launch_pool(const ScoreGeom& G, const int32_t* seq_off, int pool_kernel, const void* ws,
                       float* scores, hipStream_t st) {
  const float* sraw = reinterpret_cast<const float*>(static_cast<const char*>(ws) + G.off_sraw);
  dim3 grid((G.T + 255) / 256, G.Hkv);
  stage_begin(ST_SCORE_POOL, st);
  hipLaunchKernelGGL(pool_max, grid, dim3(256), 0, st, sraw, seq_off, G.S, G.Hkv, G.T, G.pool_rg,
                     (pool_kernel - 1) / 2, scores);
  stage_end(ST_SCORE_POOL, st);
  return hipGetLastError();
}

}  // namespace kve
