// Partition-conserving merge ("Information-Theoretic Token Eviction and
// KV-Cache Compression for Memory-Bounded Long-Context LLM Inference", §4.1):
// every evicted entry goes to the retained entry of its (sequence, KV head)
// with the largest key cosine similarity (lowest kept position on ties) when
// that similarity exceeds tau_merge, and each retained entry's bias grows by
// log(1 + number merged into it), so exact duplicates leave the softmax
// normaliser unchanged.
//
// The similarity search is a dense contraction (evicted keys x retained
// keys x d), done on bf16 MFMAs with fp32 accumulation: a workgroup holds 512
// retained keys in registers (the A operands, 128 per wave) and streams 2048
// tokens of the sequence through a 3-stage LDS ring of 32-token tiles (the B
// operand); per token it keeps the best similarity over its 512 keys and
// folds it into the token's running best with one 64-bit atomic max of
// (ordered similarity, inverted position), which makes the result
// independent of workgroup order.
#include "common.h"
#include "launch.h"

namespace kve {

constexpr int MRG_THREADS = 256;
constexpr int MRG_KB = 512;      // retained keys per workgroup (128 per wave)
constexpr int MRG_TCH = 2048;    // tokens per workgroup
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

// ------------------------------------------------------------ LDS ring
// Token tiles reach LDS through direct global->LDS loads issued from inline
// assembly, with explicit waits, so the compiler's in-order wait counting
// does not drain the ring before every read.  Row k of a tile stores its
// 16-byte chunk c at c ^ (k & 15): the 16 rows a group of lanes reads at one
// chunk land on distinct banks.
__device__ __forceinline__ void mrg_dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(gptr), "s"(lds_base) : "memory");
}
template <int N>
__device__ __forceinline__ void mrg_wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }
__device__ __forceinline__ void mrg_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ uint32_t mrg_lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}
template <typename T>
__device__ __forceinline__ void mrg_settle(const T& x) { asm volatile("" :: "v"(x)); }

constexpr int MRG_NST = 3;                      // ring stages
constexpr int MRG_GRP = 4;                      // tiles per cross-wave combine
constexpr int MRG_TILE_BYTES = MRG_TT * MRG_D * 2;

// Best retained key per token: a workgroup holds MRG_KB retained keys (each
// wave 4 blocks of 32 as MFMA A operands) and streams MRG_TCH tokens.
__global__ __launch_bounds__(MRG_THREADS, 2) void mrg_sim(MergeArgs a) {
  const int kb = blockIdx.x % a.nkb, tc = blockIdx.x / a.nkb;
  const int h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int B = a.bud_off[s + 1] - a.bud_off[s];
  if (kb * MRG_KB >= B || tc * MRG_TCH >= n || B >= n) return;
  __shared__ __align__(1024) char ring[MRG_NST * MRG_TILE_BYTES];
  __shared__ __align__(16) float kinv[MRG_KB];   // 1 / ||k_r||
  __shared__ float wbest[4][MRG_GRP * MRG_TT];   // per wave, the last MRG_GRP tiles
  __shared__ int wrow[4][MRG_GRP * MRG_TT];
  __shared__ float cbest[MRG_TCH];
  __shared__ int crow[MRG_TCH];
  __shared__ float tinvs[MRG_TCH];   // 1 / ||k|| of the range's tokens (no global loads in the loop)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, col = lane & 31;
  const size_t hrow = static_cast<size_t>(h) * a.T + base;
  const int32_t* kid = a.idx + h * a.totalB + a.bud_off[s];
  // A operands: retained keys kb*MRG_KB + 128*wave + 32*rb + col; rows past
  // the kept count repeat the last kept key (equal values, higher row: they
  // never win)
  auto kept_pos = [&](int r) {
    const int j = kid[min(r, B - 1)];
    return min(max(j, 0), n - 1);
  };
  bf16x8 qa[4][MRG_D / 16];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int jr = kept_pos(kb * MRG_KB + 128 * wave + 32 * rb + col);
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk)
      qa[rb][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(a.k + (hrow + jr) * MRG_D + 16 * kk + 8 * hl));
  }
  for (int i = tid; i < MRG_KB; i += MRG_THREADS) kinv[i] = a.invn[hrow + kept_pos(kb * MRG_KB + i)];
  const int t_begin = tc * MRG_TCH;
  const int t_end = min(n, t_begin + MRG_TCH);
  for (int i = tid; i < MRG_TCH; i += MRG_THREADS) tinvs[i] = (t_begin + i < t_end) ? a.invn[hrow + t_begin + i] : 0.f;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk) mrg_settle(qa[rb][kk]);
  __syncthreads();

  // ring fill: tile rows 8*wave .. 8*wave+7 (two 1 KiB blocks per wave)
  const int ntile = (t_end - t_begin + MRG_TT - 1) / MRG_TT;
  const uint32_t ring0 = mrg_lds_addr(ring);
  auto issue = [&](int t) {   // tile t of the range into stage t % MRG_NST (rows past the end repeat the last)
    const uint32_t sb = ring0 + static_cast<uint32_t>((t % MRG_NST) * MRG_TILE_BYTES);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = 2 * wave + i;                  // rows 4*blk .. 4*blk+3
      const int row = 4 * blk + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);        // logical chunk for this physical slot
      const int tok = min(t_begin + t * MRG_TT + row, n - 1);
      mrg_dma16(a.k + (hrow + tok) * MRG_D + 8 * c, __builtin_amdgcn_readfirstlane(sb + blk * 1024));
    }
  };
  issue(0);
  issue(1);
  for (int t = 0; t < ntile; ++t) {
    mrg_wait_vm<2>();          // this wave's part of tile t has landed (tile t+1 may be in flight)
    mrg_lds_barrier();         // every wave's part; stage (t+2) % 3 is free
    issue(t + 2);
    const char* tl = ring + (t % MRG_NST) * MRG_TILE_BYTES;
    bf16x8 kop[MRG_D / 16];
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk)
      kop[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(tl + col * (MRG_D * 2) + (((2 * kk + hl) ^ (col & 15)) << 4)));
    // c = k_r.k_t / ||k_r|| + 2 ||k_t|| lies in [||k_t||, 3 ||k_t||] (a zero
    // token key: 1), so its fp32 bits order like unsigned integers; the low
    // 6 bits are replaced by 63 - e (e = 16 rb + r, increasing row order) and
    // one unsigned maximum keeps the best value and, on ties, the lowest row
    const float tinv = tinvs[t * MRG_TT + col];
    const float sh = tinv > 0.f ? 2.f / tinv : 1.f;
    uint32_t best = 0u;
    auto post = [&](const f32x16& acc, int rb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&kinv[128 * wave + 32 * rb + 8 * q4 + 4 * hl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = fmaf(acc[4 * q4 + e], kv[e], sh);
          const uint32_t key = (__float_as_uint(c) & 0xffffffc0u) | static_cast<uint32_t>(63 - (16 * rb + 4 * q4 + e));
          best = max(best, key);
        }
      }
    };
    // the MFMA chain of block rb runs while block rb - 1 is post-processed
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk) acc0 = mfma32(qa[0][kk], kop[kk], acc0);
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk) acc1 = mfma32(qa[1][kk], kop[kk], acc1);
    post(acc0, 0);
    acc0 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk) acc0 = mfma32(qa[2][kk], kop[kk], acc0);
    post(acc1, 1);
    acc1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < MRG_D / 16; ++kk) acc1 = mfma32(qa[3][kk], kop[kk], acc1);
    post(acc0, 2);
    post(acc1, 3);
    const int eb = 63 - static_cast<int>(best & 63u);
    float bv = (__uint_as_float(best & 0xffffffc0u) - sh) * tinv;   // the cosine, to about 2^-16
    int br = 128 * wave + 32 * (eb >> 4) + 8 * ((eb >> 2) & 3) + 4 * hl + (eb & 3);
    const float ov = __shfl_xor(bv, 32, 64);
    const int orow = __shfl_xor(br, 32, 64);
    if (ov > bv || (ov == bv && orow < br)) { bv = ov; br = orow; }
    const int gs = (t % MRG_GRP) * MRG_TT;
    if (hl == 0) {
      wbest[wave][gs + col] = bv;
      wrow[wave][gs + col] = br;
    }
    if (t % MRG_GRP == MRG_GRP - 1 || t == ntile - 1) {   // combine the waves over the group's tiles
      mrg_lds_barrier();
      const int g0 = t - t % MRG_GRP;
      if (tid < (t - g0 + 1) * MRG_TT) {
        float v = wbest[0][tid];
        int rw = wrow[0][tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float v2 = wbest[w][tid];
          if (v2 > v) { v = v2; rw = wrow[w][tid]; }   // later waves hold higher rows: ties stay
        }
        cbest[g0 * MRG_TT + tid] = v;
        crow[g0 * MRG_TT + tid] = rw;
      }
    }
  }
  mrg_wait_vm<0>();
  __syncthreads();
  // fold the range into the tokens' running bests (one 64-bit atomic max per
  // evicted token); kept tokens and tokens past the end take no part
  for (int i = tid; i < t_end - t_begin; i += MRG_THREADS) {
    const float v = cbest[i];
    if (v > -INFINITY && a.flag[hrow + t_begin + i] == 0) {
      const uint32_t pos = static_cast<uint32_t>(min(kb * MRG_KB + crow[i], B - 1));
      const unsigned long long key =
          (static_cast<unsigned long long>(mrg_order(v)) << 32) | static_cast<unsigned long long>(0xffffffffu - pos);
      atomicMax(&a.best[hrow + t_begin + i], key);
    }
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
