// Key-axis pooling of the raw window scores ("A Probabilistic
// Interpretation of KV Cache Eviction", App. D, SnapKV: pooling along the
// key axis): maximum or mean over a width-k window centred on each key,
// clipped to the sequence.  Also sums the per-row-group partial score planes
// in a fixed order.
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

// One workgroup per 256 tokens of one head: the row-group planes of the
// tile plus a halo of `radius` tokens are summed once into LDS, then every
// thread takes the maximum over its window clipped to its sequence.
constexpr int POOL_TILE = 256;
constexpr int POOL_MAX_RADIUS = 15;

template <bool AVG>
__global__ __launch_bounds__(POOL_TILE) void pool_window(const float* __restrict__ sraw,
                                                      const int32_t* __restrict__ seq_off, int S, int Hkv, int T,
                                                      int planes, int radius, float* __restrict__ out) {
  __shared__ float v[POOL_TILE + 2 * POOL_MAX_RADIUS];
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * POOL_TILE;
  for (int i = threadIdx.x; i < POOL_TILE + 2 * radius; i += POOL_TILE) {
    const int j = t0 - radius + i;
    float x = -INFINITY;
    if (j >= 0 && j < T) {
      x = 0.f;
      for (int p = 0; p < planes; ++p) x += sraw[(static_cast<size_t>(p) * Hkv + h) * T + j];
    }
    v[i] = x;
  }
  __syncthreads();
  const int t = t0 + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = S;   // find s with seq_off[s] <= t < seq_off[s+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seq_off[mid] <= t) lo = mid; else hi = mid;
  }
  const int j0 = max(seq_off[lo], t - radius), j1 = min(seq_off[lo + 1] - 1, t + radius);
  float m;
  if (AVG) {
    m = 0.f;
    for (int j = j0; j <= j1; ++j) m += v[j - t0 + radius];
    m /= static_cast<float>(j1 - j0 + 1);
  } else {
    m = -INFINITY;
    for (int j = j0; j <= j1; ++j) m = fmaxf(m, v[j - t0 + radius]);
  }
  out[static_cast<size_t>(h) * T + t] = m;
}

hipError_t launch_pool(const ScoreGeom& G, const int32_t* seq_off, int pool_kernel, int pool_mode, int planes,
                       const void* ws, float* scores, hipStream_t st) {
  const float* sraw = reinterpret_cast<const float*>(static_cast<const char*>(ws) + G.off_sraw);
  if ((pool_kernel - 1) / 2 > POOL_MAX_RADIUS) return hipErrorInvalidValue;
  dim3 grid((G.T + POOL_TILE - 1) / POOL_TILE, G.Hkv);
  stage_begin(ST_SCORE_POOL, st);
  if (pool_mode == KVE_POOL_AVG)
    hipLaunchKernelGGL((pool_window<true>), grid, dim3(POOL_TILE), 0, st, sraw, seq_off, G.S, G.Hkv, G.T, planes,
                       (pool_kernel - 1) / 2, scores);
  else
    hipLaunchKernelGGL((pool_window<false>), grid, dim3(POOL_TILE), 0, st, sraw, seq_off, G.S, G.Hkv, G.T,
                       planes, (pool_kernel - 1) / 2, scores);
  stage_end(ST_SCORE_POOL, st);
  return hipGetLastError();
}

}  // namespace kve
