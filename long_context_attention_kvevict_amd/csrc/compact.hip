// Gather of the kept K/V rows and their logit bias ("A Probabilistic
// Interpretation of KV Cache Eviction", §2 Eq. 3: evicted attention indexes
// the rows of K and V with the kept set).  Out of place: one 16-byte chunk
// per thread, rows of one (sequence, KV head) per grid column.
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

__global__ __launch_bounds__(256) void compact_rows(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                    const int32_t* __restrict__ seq_off,
                                                    const int32_t* __restrict__ bud_off,
                                                    const int32_t* __restrict__ idx,
                                                    const float* __restrict__ bias,
                                                    const int32_t* __restrict__ cap_off, int Hkv, int T,
                                                    int64_t totalB, int64_t totalC, int row_bytes,
                                                    uint8_t* __restrict__ k_c, uint8_t* __restrict__ v_c,
                                                    float* __restrict__ bias_c) {
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int B = bud_off[s + 1] - bud_off[s];
  const int chunks = row_bytes / 16;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int r = static_cast<int>(item / chunks);
  const int q = static_cast<int>(item % chunks);
  if (r >= B) return;
  const int j = idx[h * totalB + bud_off[s] + r];
  const int64_t dst_row = static_cast<int64_t>(h) * totalC + cap_off[s] + r;
  if (j < 0) {   // empty slot (a soft budget's unused capacity): zero row, weight 0
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(k_c + dst_row * row_bytes + 16 * q) = z;
    *reinterpret_cast<u32x4*>(v_c + dst_row * row_bytes + 16 * q) = z;
    if (q == 0) bias_c[dst_row] = -INFINITY;
    return;
  }
  if (j >= seq_off[s + 1] - seq_off[s]) return;   // out-of-range index: slot untouched
  const int64_t src_row = static_cast<int64_t>(h) * T + seq_off[s] + j;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(k + src_row * row_bytes + 16 * q);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v + src_row * row_bytes + 16 * q);
  *reinterpret_cast<u32x4*>(k_c + dst_row * row_bytes + 16 * q) = kv;
  *reinterpret_cast<u32x4*>(v_c + dst_row * row_bytes + 16 * q) = vv;
  if (q == 0) bias_c[dst_row] = bias[h * totalB + bud_off[s] + r];
}

hipError_t launch_compact(int S, int Hkv, int d, int esize, int T, int64_t totalB, int64_t totalC,
                          int maxB, const void* k, const void* v, const int32_t* seq_off,
                          const int32_t* bud_off, const int32_t* idx, const float* bias,
                          const int32_t* cap_off, void* k_c, void* v_c, float* bias_c,
                          hipStream_t st) {
  if (maxB <= 0) return hipSuccess;
  const int row_bytes = d * esize;
  const int64_t items = static_cast<int64_t>(maxB) * (row_bytes / 16);
  dim3 grid(static_cast<unsigned>((items + 255) / 256), Hkv, S);
  stage_begin(ST_COMPACT, st);
  hipLaunchKernelGGL(compact_rows, grid, dim3(256), 0, st, static_cast<const uint8_t*>(k),
                     static_cast<const uint8_t*>(v), seq_off, bud_off, idx, bias, cap_off, Hkv, T,
                     totalB, totalC, row_bytes, static_cast<uint8_t*>(k_c), static_cast<uint8_t*>(v_c),
                     bias_c);
  stage_end(ST_COMPACT, st);
  return hipGetLastError();
}

}  // namespace kve
