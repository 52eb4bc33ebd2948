// Corrected decode attention over the compacted cache ("A Probabilistic
// Interpretation of KV Cache Eviction", §5, Definition 3-4 and Algorithm 1):
// o = (sum_hist w p~ v + sum_new p~ v) / (sum_hist w p~ + sum_new p~), computed
// as a softmax whose logits carry the additive bias log w per entry (0 for
// entries appended after eviction).  All q-heads of a GQA group share the
// KV head's entries and biases (§5, grouped-query attention paragraph).
//
// Split-K flash decoding: workgroup = (split, KV head, sequence), 4 waves;
// each 16-lane quarter of a wave handles one cache entry at a time (lane
// holds DD/16 features), keeps an online softmax per q-head row, and the
// 16 partial states of the workgroup are merged through LDS.  A second
// kernel merges the splits.
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }

template <typename T, int DD, int GMAX>
__global__ __launch_bounds__(256) void decode_split(const T* __restrict__ q, const T* __restrict__ k_c,
                                                    const T* __restrict__ v_c, const float* __restrict__ bias_c,
                                                    const int32_t* __restrict__ cap_off,
                                                    const int32_t* __restrict__ cache_len, int Hq, int Hkv,
                                                    int64_t totalC, int split_len, int splits, float c2,
                                                    float* __restrict__ part_ml, float* __restrict__ part_o) {
  constexpr int CPL = DD / 16;   // features per lane
  const int sp = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int g = Hq / Hkv;
  // never read past this sequence's capacity, whatever cache_len holds
  const int len = min(cache_len[s], cap_off[s + 1] - cap_off[s]);
  const int e0 = sp * split_len;
  const int e1 = min(e0 + split_len, len);
  const int tid = threadIdx.x;
  const int sub = tid >> 4;        // 16 entry streams per workgroup
  const int fl = tid & 15;         // feature chunk
  __shared__ float sm[4][GMAX];
  __shared__ float sl[4][GMAX];
  __shared__ float so[4][GMAX][DD];

  float qv[GMAX][CPL];
#pragma unroll
  for (int i = 0; i < GMAX; ++i) {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      qv[i][c] = (i < g) ? ld_elem<T>(q + (static_cast<size_t>(s) * Hq + h * g + i) * DD + fl * CPL + c) : 0.f;
  }
  float m[GMAX], l[GMAX], o[GMAX][CPL];
#pragma unroll
  for (int i = 0; i < GMAX; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[i][c] = 0.f;
  }
  const size_t rowbase = static_cast<size_t>(h) * totalC + cap_off[s];
  for (int e = e0 + sub; e < e1; e += 16) {
    float kr[CPL], vr[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      kr[c] = ld_elem<T>(k_c + (rowbase + e) * DD + fl * CPL + c);
      vr[c] = ld_elem<T>(v_c + (rowbase + e) * DD + fl * CPL + c);
    }
    const float bl2 = bias_c[rowbase + e] * kLog2e;
#pragma unroll
    for (int i = 0; i < GMAX; ++i) {
      if (i < g) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) dot = fmaf(qv[i][c], kr[c], dot);
      dot += __shfl_xor(dot, 8, 16);
      dot += __shfl_xor(dot, 4, 16);
      dot += __shfl_xor(dot, 2, 16);
      dot += __shfl_xor(dot, 1, 16);
      const float x = fmaf(dot, c2, bl2);
      const float mn = fmaxf(m[i], x);
      const float sc = exp2f(m[i] - mn);
      const float p = exp2f(x - mn);
      l[i] = l[i] * sc + p;
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[i][c] = fmaf(p, vr[c], o[i][c] * sc);
      m[i] = mn;
      }
    }
  }
  // merge the 4 entry streams of each wave (lanes 16 and 32 apart)
#pragma unroll
  for (int i = 0; i < GMAX; ++i) {
    if (i < g) {
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      const float mo = __shfl_xor(m[i], sh, 64);
      const float lo = __shfl_xor(l[i], sh, 64);
      const float mn = fmaxf(m[i], mo);
      const float fa = (m[i] == -INFINITY) ? 0.f : exp2f(m[i] - mn);
      const float fb = (mo == -INFINITY) ? 0.f : exp2f(mo - mn);
      l[i] = l[i] * fa + lo * fb;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float oo = __shfl_xor(o[i][c], sh, 64);
        o[i][c] = o[i][c] * fa + oo * fb;
      }
      m[i] = mn;
    }
    }
  }
  const int wave = tid >> 6;
  if ((tid & 63) < 16) {
#pragma unroll
    for (int i = 0; i < GMAX; ++i) {
      if (i < g) {
        if (fl == 0) { sm[wave][i] = m[i]; sl[wave][i] = l[i]; }
#pragma unroll
        for (int c = 0; c < CPL; ++c) so[wave][i][fl * CPL + c] = o[i][c];
      }
    }
  }
  __syncthreads();
  // merge the 4 waves: thread -> (row i, feature d)
  for (int t = tid; t < g * DD; t += 256) {
    const int i = t / DD, d = t % DD;
    float M = -INFINITY;
    for (int u = 0; u < 4; ++u) M = fmaxf(M, sm[u][i]);
    float L = 0.f, O = 0.f;
    for (int u = 0; u < 4; ++u) {
      const float f = (sm[u][i] == -INFINITY) ? 0.f : exp2f(sm[u][i] - M);
      L += sl[u][i] * f;
      O += so[u][i][d] * f;
    }
    const size_t row = (static_cast<size_t>(s) * Hq + h * g + i) * splits + sp;
    part_o[row * DD + d] = O;
    if (d == 0) { part_ml[row * 2] = M; part_ml[row * 2 + 1] = L; }
  }
}

template <int DD>
__global__ __launch_bounds__(DD) void decode_merge(const float* __restrict__ part_ml, const float* __restrict__ part_o,
                                                   const int32_t* __restrict__ cache_len,
                                                   const int32_t* __restrict__ cap_off, int Hq, int splits,
                                                   int split_len, float* __restrict__ out) {
  const int r = blockIdx.x;          // s * Hq + qh
  const int s = r / Hq;
  const int d = threadIdx.x;
  const int len = min(cache_len[s], cap_off[s + 1] - cap_off[s]);
  const int ns = max(0, min(splits, (len + split_len - 1) / split_len));
  float M = -INFINITY;
  for (int p = 0; p < ns; ++p) M = fmaxf(M, part_ml[(static_cast<size_t>(r) * splits + p) * 2]);
  float L = 0.f, O = 0.f;
  for (int p = 0; p < ns; ++p) {
    const size_t row = static_cast<size_t>(r) * splits + p;
    const float mm = part_ml[row * 2];
    const float f = (mm == -INFINITY) ? 0.f : exp2f(mm - M);
    L += part_ml[row * 2 + 1] * f;
    O += part_o[row * DD + d] * f;
  }
  out[static_cast<size_t>(r) * DD + d] = (L > 0.f) ? O / L : 0.f;   // empty cache -> 0
}

template <typename T, int DD>
static hipError_t launch_decode_t(const DecodeGeom& G, int64_t totalC, const void* q, const void* k_c,
                                  const void* v_c, const float* bias_c, const int32_t* cap_off,
                                  const int32_t* cache_len, float sm_scale, float* out, void* ws,
                                  hipStream_t st) {
  char* base = static_cast<char*>(ws);
  float* pml = reinterpret_cast<float*>(base + G.off_ml);
  float* po = reinterpret_cast<float*>(base + G.off_o);
  dim3 grid(G.splits, G.Hkv, G.S);
  const int g = G.Hq / G.Hkv;
  const float c2 = sm_scale * kLog2e;
  stage_begin(ST_DECODE_SPLIT, st);
  if (g <= 4)
    hipLaunchKernelGGL((decode_split<T, DD, 4>), grid, dim3(256), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k_c), static_cast<const T*>(v_c), bias_c, cap_off, cache_len,
                       G.Hq, G.Hkv, totalC, G.split_len, G.splits, c2, pml, po);
  else if (g <= 8)
    hipLaunchKernelGGL((decode_split<T, DD, 8>), grid, dim3(256), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k_c), static_cast<const T*>(v_c), bias_c, cap_off, cache_len,
                       G.Hq, G.Hkv, totalC, G.split_len, G.splits, c2, pml, po);
  else
    hipLaunchKernelGGL((decode_split<T, DD, 16>), grid, dim3(256), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k_c), static_cast<const T*>(v_c), bias_c, cap_off, cache_len,
                       G.Hq, G.Hkv, totalC, G.split_len, G.splits, c2, pml, po);
  stage_end(ST_DECODE_SPLIT, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(ST_DECODE_MERGE, st);
  hipLaunchKernelGGL((decode_merge<DD>), dim3(G.S * G.Hq), dim3(DD), 0, st, pml, po, cache_len, cap_off,
                     G.Hq, G.splits, G.split_len, out);
  stage_end(ST_DECODE_MERGE, st);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeGeom& G, int64_t totalC, const void* q, const void* k_c,
                         const void* v_c, const float* bias_c, const int32_t* cap_off,
                         const int32_t* cache_len, float sm_scale, float* out, void* ws,
                         hipStream_t st) {
  if (G.dtype == KVE_BF16) {
    if (G.d == 64)
      return launch_decode_t<uint16_t, 64>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st);
    return launch_decode_t<uint16_t, 128>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st);
  }
  if (G.d == 64)
    return launch_decode_t<float, 64>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st);
  return launch_decode_t<float, 128>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st);
}

}  // namespace kve
