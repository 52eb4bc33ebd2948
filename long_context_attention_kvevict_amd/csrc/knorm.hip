// K-norm eviction score ("A Probabilistic Interpretation of KV Cache
// Eviction", App. D, Eq. 18; the related-work section of "DropKV:
// Decoupling Residual-Output Perturbation for Near-Optimal KV-Cache
// Eviction" describes the method as keeping the entries with the smaller
// KEY norms): per key,
// exp(kKnormShift - ||k_j||), a positive score whose largest values are the
// smallest norms and whose tempered proposal s^(1/tau) is the softmax of
// -||k|| / tau.  The constant shift leaves the ranking and the normalised
// proposal unchanged and keeps norms up to about 167 in the fp32 normal
// range.  One streaming read of K; no attention.
#include "common.h"
#include "launch.h"

namespace kve {

constexpr float kKnormShift = 80.f;
constexpr int KN_THREADS = 256;
constexpr int KN_UNROLL = 4;

// L lanes share one key row (16 bytes each); a workgroup covers
// KN_UNROLL * KN_THREADS / L rows, each load instruction of a wave reading
// 1 KiB of consecutive rows.
template <typename E, int L>
__global__ __launch_bounds__(KN_THREADS) void knorm_rows(const E* __restrict__ k, size_t rows,
                                                         float* __restrict__ out) {
  constexpr int PER = 16 / sizeof(E);          // elements per lane and load
  constexpr int RPI = KN_THREADS / L;          // rows per unrolled step
  const int sub = threadIdx.x % L;
  const size_t r0 = static_cast<size_t>(blockIdx.x) * (KN_UNROLL * RPI) + threadIdx.x / L;
  u32x4 x[KN_UNROLL];
#pragma unroll
  for (int u = 0; u < KN_UNROLL; ++u) {
    const size_t r = r0 + static_cast<size_t>(u) * RPI;
    x[u] = u32x4{0u, 0u, 0u, 0u};
    if (r < rows) x[u] = *reinterpret_cast<const u32x4*>(k + r * (L * PER) + sub * PER);
  }
#pragma unroll
  for (int u = 0; u < KN_UNROLL; ++u) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(E) == 2) {
        const float a0 = __uint_as_float(x[u][e] << 16), a1 = __uint_as_float(x[u][e] & 0xffff0000u);
        acc = fmaf(a0, a0, acc);
        acc = fmaf(a1, a1, acc);
      } else {
        const float a0 = __uint_as_float(x[u][e]);
        acc = fmaf(a0, a0, acc);
      }
    }
#pragma unroll
    for (int m = 1; m < L; m <<= 1) acc += __shfl_xor(acc, m, 64);
    const size_t r = r0 + static_cast<size_t>(u) * RPI;
    if (sub == 0 && r < rows) out[r] = expf(kKnormShift - sqrtf(acc));
  }
}

template <typename E, int L>
static void launch_rows(const void* k, size_t rows, float* out, hipStream_t st) {
  constexpr int per_wg = KN_UNROLL * (KN_THREADS / L);
  const dim3 grid(static_cast<unsigned>((rows + per_wg - 1) / per_wg));
  hipLaunchKernelGGL((knorm_rows<E, L>), grid, dim3(KN_THREADS), 0, st, static_cast<const E*>(k), rows, out);
}

hipError_t launch_knorm(const ScoreGeom& G, const void* k, void* ws, hipStream_t st) {
  float* sraw = reinterpret_cast<float*>(static_cast<char*>(ws) + G.off_sraw);
  const size_t rows = static_cast<size_t>(G.Hkv) * G.T;
  if (rows == 0) return hipSuccess;
  const int row_bytes = G.d * (G.dtype == KVE_BF16 ? 2 : 4);
  if (G.dtype == KVE_BF16 && row_bytes == 256) launch_rows<uint16_t, 16>(k, rows, sraw, st);
  else if (G.dtype == KVE_F32 && row_bytes == 512) launch_rows<float, 32>(k, rows, sraw, st);
  else if (G.dtype == KVE_F32 && row_bytes == 256) launch_rows<float, 16>(k, rows, sraw, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kve
