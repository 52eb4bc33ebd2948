// Partition-conserving merge ("Information-Theoretic Token Eviction and
// KV-Cache Compression for Memory-Bounded Long-Context LLM Inference", §4.1):
// every evicted entry goes to the retained entry of its (sequence, KV head)
// with the largest key cosine similarity (lowest kept position on ties) when
// that similarity exceeds tau_merge, and each retained entry's bias grows by
// log(1 + number merged into it), so exact duplicates leave the softmax
// normaliser unchanged.
//
// The similarity search is a dense contraction (evicted keys x retained
// keys x d), done on bf16 MFMAs with fp32 accumulation: a workgroup holds 128
// retained keys in registers (the A operand, 32 per wave) and streams 4096
// tokens of the sequence in 32-token tiles (the B operand); per token it
// keeps the best similarity over its 128 keys and folds it into the token's
// running best with one 64-bit atomic max of (ordered similarity, inverted
// position), which makes the result independent of workgroup order.
#include "common.h"
#include "launch.h"

namespace kve {

constexpr int MRG_THREADS = 256;
constexpr int MRG_KB = 128;      // retained keys per workgroup
constexpr int MRG_TCH = 4096;    // tokens per workgroup
constexpr int MRG_TT = 32;       // tokens per tile
constexpr int MRG_D = 128;

struct MergeArgs {
  const uint16_t* k;        // [Hkv][T][128] bf16
  const int32_t* seq_off;
  const int32_t* bud_off;
  const int32_t* idx;       // [Hkv][totalB] kept positions, ascending per (sequence, head)
  float* bias;              // [Hkv][totalB] in / out
  int32_t* merged;          // [Hkv][totalB] out, or NULL
  int32_t* target;          // [Hkv][T] out, or NULL
  float tau;
  int S, Hkv, T, nkb, ntc;
  int64_t totalB;
  float* invn;              // [Hkv][T] 1 / ||k|| (0 for a zero key)
  int* flag;                // [Hkv][T] 1 for retained entries
  unsigned long long* best; // [Hkv][T] packed best (similarity, position)
  int* cnt;                 // [Hkv][totalB]
};

__device__ __forceinline__ uint32_t mrg_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float mrg_unorder(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// 1 / ||k|| per row (16 lanes per 256-byte row), flags and bests cleared.
__global__ __launch_bounds__(MRG_THREADS) void mrg_prep(MergeArgs a, int64_t rows) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (MRG_THREADS / 16) + threadIdx.x / 16;
  const int sub = threadIdx.x % 16;
  u32x4 x = {0u, 0u, 0u, 0u};
  if (r < rows) x = *reinterpret_cast<const u32x4*>(a.k + r * MRG_D + sub * 8);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = __uint_as_float(x[e] << 16), a1 = __uint_as_float(x[e] & 0xffff0000u);
    acc = fmaf(a0, a0, acc);
    acc = fmaf(a1, a1, acc);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (sub == 0 && r < rows) {
    a.invn[r] = acc > 0.f ? 1.f / sqrtf(acc) : 0.f;
    a.flag[r] = 0;
    a.best[r] = 0ull;
  }
}

__global__ __launch_bounds__(256) void mrg_zero(int* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0;
}

// Flags the retained entries.
__global__ __launch_bounds__(256) void mrg_mark(MergeArgs a) {
  const int h = blockIdx.y, s = blockIdx.z;
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int B = a.bud_off[s + 1] - a.bud_off[s];
  const int n = a.seq_off[s + 1] - a.seq_off[s];
  if (r >= B) return;
  const int j = a.idx[h * a.totalB + a.bud_off[s] + r];
  if (j >= 0 && j < n) a.flag[static_cast<size_t>(h) * a.T + a.seq_off[s] + j] = 1;
}

// Best retained key per token over one block of 128 retained keys.
__global__ __launch_bounds__(MRG_THREADS) void mrg_sim(MergeArgs a) {
  const int kb = blockIdx.x % a.nkb, tc = blockIdx.x / a.nkb;
  const int h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int B = a.bud_off[s + 1] - a.bud_off[s];
  if (kb * MRG_KB >= B || tc * MRG_TCH >= n || B >= n) return;
  __shared__ float kinv[MRG_KB];
  __shared__ float wbest[4][MRG_TT];
  __shared__ int wrow[4][MRG_TT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const size_t hrow = static_cast<size_t>(h) * a.T + base;
  const int32_t* kid = a.idx + h * a.totalB + a.bud_off[s];
  // A operand: retained key kb*128 + 32*wave + col
  const int rr = kb * MRG_KB + 32 * wave + col;
  const bool rr_ok = rr < B;
  int jr = rr_ok ? kid[rr] : 0;
  if (jr < 0 || jr >= n) jr = 0;
  bf16x8 qa[MRG_D / 16];
#pragma unroll
  for (int kk = 0; kk < MRG_D / 16; ++kk) {
    u32x4 t = {0u, 0u, 0u, 0u};
    if (rr_ok) t = *reinterpret_cast<const u32x4*>(a.k + (hrow + jr) * MRG_D + 16 * kk + 8 * hl);
    qa[kk] = as_bf16x8(t);
  }
  if (tid < MRG_KB) {
    const int r2 = kb * MRG_KB + tid;
    int j2 = r2 < B ? kid[r2] : -1;
    kinv[tid] = (j2 >= 0 && j2 < n) ? a.invn[hrow + j2] : -1.f;   // -1 marks a missing key
  }
  __syncthreads();
  float kiv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) kiv[r] = kinv[32 * wave + 8 * (r >> 2) + 4 * hl + (r & 3)];

  const int t1 = min(n, (tc + 1) * MRG_TCH);
  for (int t0 = tc * MRG_TCH; t0 < t1; t0 += MRG_TT) {
    const int tok = t0 + col;
    const int tk = tok < n ? tok : n - 1;
    bf16x8 kop[MRG_D / 16];
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk)
      kop[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(a.k + (hrow + tk) * MRG_D + 16 * kk + 8 * hl));
    const float tinv = a.invn[hrow + tk];
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk) acc = mfma32(qa[kk], kop[kk], acc);
    // best over this lane's 16 retained rows, in increasing row order
    float bv = -INFINITY;
    int br = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float kv = kiv[r];
      const float c = (kv >= 0.f) ? acc[r] * kv * tinv : -INFINITY;
      const int row = 32 * wave + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (c > bv || (c == bv && row < br)) { bv = c; br = row; }
    }
    const float ov = __shfl_xor(bv, 32, 64);
    const int orow = __shfl_xor(br, 32, 64);
    if (ov > bv || (ov == bv && orow < br)) { bv = ov; br = orow; }
    if (hl == 0) {
      wbest[wave][col] = bv;
      wrow[wave][col] = br;
    }
    __syncthreads();
    if (tid < MRG_TT) {
      float v = wbest[0][tid];
      int rw = wrow[0][tid];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float v2 = wbest[w][tid];
        if (v2 > v) { v = v2; rw = wrow[w][tid]; }   // later waves hold higher rows: ties stay
      }
      const int t = t0 + tid;
      if (t < n && v > -INFINITY && a.flag[hrow + t] == 0) {
        const uint32_t pos = static_cast<uint32_t>(kb * MRG_KB + rw);
        const unsigned long long key =
            (static_cast<unsigned long long>(mrg_order(v)) << 32) | static_cast<unsigned long long>(0xffffffffu - pos);
        atomicMax(&a.best[hrow + t], key);
      }
    }
    __syncthreads();
  }
}

// Per token: merge target (if above the threshold) and the counts.
__global__ __launch_bounds__(256) void mrg_apply(MergeArgs a) {
  const int h = blockIdx.y, s = blockIdx.z;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  if (j >= n) return;
  const size_t row = static_cast<size_t>(h) * a.T + base + j;
  const unsigned long long b = a.best[row];
  int tgt = -1;
  if (a.flag[row] == 0 && b != 0ull) {
    const float c = mrg_unorder(static_cast<uint32_t>(b >> 32));
    const int pos = static_cast<int>(0xffffffffu - static_cast<uint32_t>(b & 0xffffffffull));
    if (c > a.tau) {
      tgt = pos;
      atomicAdd(&a.cnt[h * a.totalB + a.bud_off[s] + pos], 1);
    }
  }
  if (a.target) a.target[row] = tgt;
}

// Retained entries: bias += log(1 + merged).
__global__ __launch_bounds__(256) void mrg_bias(MergeArgs a) {
  const int h = blockIdx.y, s = blockIdx.z;
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int B = a.bud_off[s + 1] - a.bud_off[s];
  if (r >= B) return;
  const int64_t i = h * a.totalB + a.bud_off[s] + r;
  const int c = a.cnt[i];
  if (c > 0) a.bias[i] += log1pf(static_cast<float>(c));
  if (a.merged) a.merged[i] = c;
}

hipError_t launch_merge(const MergeGeom& G, const void* k, const int32_t* seq_off, const int32_t* bud_off,
                        const int32_t* idx, float tau, float* bias, int32_t* merged, int32_t* target, void* ws,
                        hipStream_t st) {
  char* wsb = static_cast<char*>(ws);
  MergeArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.seq_off = seq_off;
  a.bud_off = bud_off;
  a.idx = idx;
  a.bias = bias;
  a.merged = merged;
  a.target = target;
  a.tau = tau;
  a.S = G.S;
  a.Hkv = G.Hkv;
  a.T = G.T;
  a.nkb = (G.maxB + MRG_KB - 1) / MRG_KB;
  a.ntc = (G.max_len + MRG_TCH - 1) / MRG_TCH;
  a.totalB = G.totalB;
  a.invn = reinterpret_cast<float*>(wsb + G.off_invn);
  a.flag = reinterpret_cast<int*>(wsb + G.off_flag);
  a.best = reinterpret_cast<unsigned long long*>(wsb + G.off_best);
  a.cnt = reinterpret_cast<int*>(wsb + G.off_cnt);
  const int64_t rows = static_cast<int64_t>(G.Hkv) * G.T;
  hipLaunchKernelGGL(mrg_prep, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(MRG_THREADS), 0, st, a, rows);
  const int64_t ncnt = static_cast<int64_t>(G.Hkv) * G.totalB;
  if (ncnt > 0)
    hipLaunchKernelGGL(mrg_zero, dim3(static_cast<unsigned>((ncnt + 255) / 256 < 4096 ? (ncnt + 255) / 256 : 4096)),
                       dim3(256), 0, st, a.cnt, ncnt);
  if (G.maxB > 0) {
    hipLaunchKernelGGL(mrg_mark, dim3((G.maxB + 255) / 256, G.Hkv, G.S), dim3(256), 0, st, a);
    hipLaunchKernelGGL(mrg_sim, dim3(a.nkb * a.ntc, G.Hkv, G.S), dim3(MRG_THREADS), 0, st, a);
  }
  hipLaunchKernelGGL(mrg_apply, dim3((G.max_len + 255) / 256, G.Hkv, G.S), dim3(256), 0, st, a);
  if (G.maxB > 0) hipLaunchKernelGGL(mrg_bias, dim3((G.maxB + 255) / 256, G.Hkv, G.S), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kve
