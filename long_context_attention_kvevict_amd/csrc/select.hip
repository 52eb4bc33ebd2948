// Budgeted per-head selection.
//
// Top-k ("DropKV" page, §3.3: evict the smallest scores, i.e. keep the B
// largest; "A Probabilistic Interpretation of KV Cache Eviction", §4: top-k
// as a zero-variance estimator): the B largest scores of each (sequence, KV
// head), ties to the lower index, NaN below every number.
//
// Sampling ("A Probabilistic Interpretation ...", §4 proposals with full
// support, App. D.1 tempering, App. F Problem 5 / Algorithm 2 and Eq. 24-25,
// §6 Eq. 10): fp64 proposal log pi~ = log(max(s, 2^-126)) / tau, a number of
// with-replacement draws m whose expected distinct count
// E(m) = sum_j 1 - (1 - pi_j)^m lies within 0.5 of B, Gumbel keys from
// Philox-4x64-10 (the B largest are kept), bias -log(q_j) / tau_w with
// q_j = 1 - (1 - pi_j)^m.  Optionally (App. D.1) the normalised proposal is
// mixed with the uniform, pi' = alpha pi + (1 - alpha) / n, before all of it.
//
// Work is spread over workgroups of SEL_CHUNK keys of one (sequence, head),
// one launch per pass; no launch waits on another workgroup of the same
// launch.  Selection is a radix select over the order-preserving integer
// image of the keys (11-bit digits, most significant first): histogram
// launches count one digit each (integer atomics) and the next launch reads
// the finished histograms and fixes the digits of the B-th largest key.  The
// last digit's launch also leaves, per chunk, the count of keys above the
// threshold's leading digits and the last digits of those that share them,
// from which the write launch places each chunk's kept indices after those
// of earlier chunks, so the output is ascending (under a soft budget a count
// launch tallies the keys above / equal to the threshold per chunk instead).
// With a per-head budget the sampling passes carry the digit levels of the
// Gumbel keys, which do not depend on m.  Cross-chunk sums of the sampling
// passes (the proposal's normaliser, E(m) and its derivative) are per-chunk
// partials that the next launch adds up in chunk order: results are
// bit-reproducible.
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

constexpr int SEL_THREADS = 256;
constexpr int SEL_PER = 4;
constexpr int SEL_CHUNK = SEL_THREADS * SEL_PER;
constexpr int SEL_BINS = 2048;
static_assert(SEL_CHUNK == kSelChunk && SEL_BINS == kSelBins, "host and device select geometry disagree");

// ------------------------------------------------------------ block helpers
// Inclusive prefix sum over a 256-thread block; *total gets the block sum.
// lds: 4 ints.  Two barriers.
__device__ __forceinline__ int block_incl_scan256(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) lds[wave] = v;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int wv = 0; wv < 4; ++wv) {
    const int c = lds[wv];
    if (wv < wave) off += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return v + off;
}

// Block sum / max of fp64 in a fixed order (lanes, then waves 0..3).
__device__ __forceinline__ double block_sum_d(double v, double* lds) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  const double t = (lds[0] + lds[1]) + (lds[2] + lds[3]);
  __syncthreads();
  return t;
}
// Block sums of three fp64 values at once (same order as block_sum_d);
// lds: 12 doubles.  Two barriers.
__device__ __forceinline__ void block_sum3_d(double* a, double* b, double* c, double* lds) {
  double x = wave_sum_d(*a), y = wave_sum_d(*b), z = wave_sum_d(*c);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    lds[wave] = x;
    lds[4 + wave] = y;
    lds[8 + wave] = z;
  }
  __syncthreads();
  *a = (lds[0] + lds[1]) + (lds[2] + lds[3]);
  *b = (lds[4] + lds[5]) + (lds[6] + lds[7]);
  *c = (lds[8] + lds[9]) + (lds[10] + lds[11]);
  __syncthreads();
}

// Workgroup sums (256 threads) of 32 values per thread.  Within a wave,
// five exchange steps each hand half of the lane's remaining values to the
// partner lane (xor 32, 16, 8, 4, 2) and add the half it keeps, and a sixth
// adds the neighbour's (xor 1): lanes 2k and 2k+1 then hold value k's wave
// sum.  The four waves' sums are added in wave order.  On return every
// thread reads value k's total in red[128 + k] (red: 160 floats of LDS).
constexpr int kRed32 = 160;
template <int N>
__device__ __forceinline__ void fold_half(const float (&v)[2 * N], float (&o)[N], int mask) {
  const bool hi = (threadIdx.x & mask) != 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float keep = hi ? v[N + i] : v[i];
    const float give = hi ? v[i] : v[N + i];
    o[i] = keep + __shfl_xor(give, mask);
  }
}
__device__ __forceinline__ void block_sum32(const float (&v)[32], float* red) {
  float a[16], b[8], c[4], d[2], e[1];
  fold_half<16>(v, a, 32);
  fold_half<8>(a, b, 16);
  fold_half<4>(b, c, 8);
  fold_half<2>(c, d, 4);
  fold_half<1>(d, e, 2);
  const float t = e[0] + __shfl_xor(e[0], 1);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((lane & 1) == 0) red[wave * 32 + (lane >> 1)] = t;
  __syncthreads();
  if (threadIdx.x < 32)
    red[128 + threadIdx.x] = ((red[threadIdx.x] + red[32 + threadIdx.x]) + red[64 + threadIdx.x]) + red[96 + threadIdx.x];
  __syncthreads();
}

__device__ __forceinline__ double block_max_d(double v, double* lds) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  const double t = fmax(fmax(lds[0], lds[1]), fmax(lds[2], lds[3]));
  __syncthreads();
  return t;
}

// --------------------------------------------------------------- key types
template <typename K>
struct Radix;
template <>
struct Radix<uint32_t> {   // digits of 11 + 11 + 10 bits
  static constexpr int LEVELS = 3;
  static constexpr int LAST_BINS = 1024;
  __device__ static int shift(int lv) { return lv == 0 ? 21 : (lv == 1 ? 10 : 0); }
  __device__ static uint32_t wmask(int lv) { return lv == 2 ? 0x3ffu : 0x7ffu; }
};
template <>
struct Radix<uint64_t> {   // digits of 5 x 11 + 9 bits
  static constexpr int LEVELS = 6;
  static constexpr int LAST_BINS = 512;
  __device__ static int shift(int lv) { return lv < 5 ? 53 - 11 * lv : 0; }
  __device__ static uint64_t wmask(int lv) { return lv < 5 ? 0x7ffull : 0x1ffull; }
};
static_assert(Radix<uint32_t>::LEVELS == kSelLevels32 && Radix<uint64_t>::LEVELS == kSelLevels64,
              "host and device digit counts disagree");

// Keys of a [Hkv][T] plane: fp32 scores (top-k) or fp64 Gumbel keys.
struct ScoreKeys {
  typedef uint32_t K;
  const float* p;
  __device__ K key(size_t i) const { return f32_order_key(p[i]); }
};
struct GumbelKeys {
  typedef uint64_t K;
  const double* p;
  __device__ K key(size_t i) const { return f64_order_key(p[i]); }
};

// Geometry shared by the selection kernels.
struct SelArgs {
  const int32_t* seq_off;
  const int32_t* bud_off;   // per-sequence budget B_s (the target under a soft budget)
  const int32_t* out_off;   // output slots of each sequence (bud_off, or the capacities)
  const int32_t* bsh;       // soft budget: kept count of each (sequence, head), else NULL
  int S, Hkv, T, nchunk;
  int64_t totalB;           // out_off[S]
  struct RCache* rcache;    // [S*Hkv][kSelLevels64] threshold digits resolved so far
};

// Threshold digits resolved so far for one (sequence, head): the key prefix
// of levels 0 .. L and the count still needed among keys carrying it.
struct RCache {
  uint64_t prefix;
  int32_t need, pad;
};
static_assert(sizeof(RCache) == kSelRCacheBytes, "host and device cache entry size disagree");

// Kept count of (sequence s, head h).
__device__ __forceinline__ int sel_budget(const SelArgs& a, int s, int sh) {
  return a.bsh ? a.bsh[sh] : a.bud_off[s + 1] - a.bud_off[s];
}

// Scans the 8 bins a thread holds (thread t owns bins 2047-8t .. 2040-8t, in
// that order) across the block from the top bin down; returns the bin at
// which the running count first reaches `need` and the count strictly above
// it.  lds: 6 ints.
__device__ void pick_bin(const int (&c)[8], int need, int* lds, int* digit, int* above) {
  const int t = threadIdx.x;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += c[i];
  if (t == 0) { lds[4] = 0; lds[5] = 0; }
  int total;
  const int incl = block_incl_scan256(sum, lds, &total);   // its barriers order the init above
  const int excl = incl - sum;
  if (excl < need && need <= incl) {
    int cum = excl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (cum + c[i] >= need) {
        lds[4] = SEL_BINS - 1 - 8 * t - i;
        lds[5] = cum;
        break;
      }
      cum += c[i];
    }
  }
  __syncthreads();
  *digit = lds[4];
  *above = lds[5];
  __syncthreads();
}

// Resolves digit levels 0 .. NLV-1 from the finished histograms: key prefix,
// its mask and the count still needed among the keys carrying that prefix.
// Levels 0 .. NLV-2 come from the per-head cache the previous launch of the
// chain left (the launches resolve one more level each), so only level
// NLV-1 is picked from its histogram here; the first chunk's workgroup of
// the head then caches levels 0 .. NLV-1 for the next launch.
template <typename K, int NLV>
__device__ void resolve(const int* __restrict__ hist, int SH, int sh, int B, int* lds, K* prefix, K* mask, int* need,
                        RCache* cache) {
  K p = 0, m = 0;
  int nd = B;
  if (NLV > 0) {
    constexpr int lv = NLV - 1;
    int c[8];
    const int* gh = hist + (static_cast<size_t>(lv) * SH + sh) * SEL_BINS;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = gh[SEL_BINS - 1 - 8 * threadIdx.x - i];
    if (NLV > 1) {
      const RCache r = cache[static_cast<size_t>(sh) * kSelLevels64 + (NLV - 2)];
      p = static_cast<K>(r.prefix);
      nd = r.need;
#pragma unroll
      for (int l = 0; l < NLV - 1; ++l) m |= Radix<K>::wmask(l) << Radix<K>::shift(l);
    }
    int dg, ab;
    pick_bin(c, nd, lds, &dg, &ab);
    p |= static_cast<K>(dg) << Radix<K>::shift(lv);
    m |= Radix<K>::wmask(lv) << Radix<K>::shift(lv);
    nd -= ab;
    if (blockIdx.x == 0 && threadIdx.x == 0)
      cache[static_cast<size_t>(sh) * kSelLevels64 + (NLV - 1)] = RCache{static_cast<uint64_t>(p), nd, 0};
  }
  *prefix = p;
  *mask = m;
  *need = nd;
}

// One digit level: histogram of the keys matching the prefix resolved so far.
// lh: SEL_BINS ints of LDS, lds: 8 ints of LDS (the caller's, so that fused
// kernels can share one allocation between their parts).
template <class Src, int LV>
__device__ __forceinline__ void sel_hist_body(Src src, const SelArgs& a, int* __restrict__ hist, int* lh, int* lds) {
  typedef typename Src::K K;
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int sh = s * a.Hkv + h;
  const int B = sel_budget(a, s, sh);
  const int j0 = ch * SEL_CHUNK;
  if (B <= 0 || B >= n || j0 >= n) return;
  const int SH = a.S * a.Hkv;
  const size_t row = static_cast<size_t>(h) * a.T + base;
  K u[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {   // all key loads in flight at once
    const int j = j0 + i * SEL_THREADS + threadIdx.x;
    u[i] = (j < n) ? src.key(row + j) : K(0);
  }
  K prefix, mask;
  int need;
  resolve<K, LV>(hist, SH, sh, B, lds, &prefix, &mask, &need, a.rcache);   // its loads overlap the keys'
  for (int i = threadIdx.x; i < SEL_BINS; i += SEL_THREADS) lh[i] = 0;
  __syncthreads();   // lh cleared
  const int sft = Radix<K>::shift(LV);
  const K dm = Radix<K>::wmask(LV);
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const int j = j0 + i * SEL_THREADS + threadIdx.x;
    if (j < n && (u[i] & mask) == prefix) atomicAdd(&lh[static_cast<int>((u[i] >> sft) & dm)], 1);
  }
  __syncthreads();
  int* gh = hist + (static_cast<size_t>(LV) * SH + sh) * SEL_BINS;
  for (int i = threadIdx.x; i < SEL_BINS; i += SEL_THREADS) {
    const int c = lh[i];
    if (c) atomicAdd(&gh[i], c);
  }
}
template <class Src, int LV>
__global__ __launch_bounds__(SEL_THREADS) void sel_hist(Src src, SelArgs a, int* __restrict__ hist) {
  __shared__ int lh[SEL_BINS];
  __shared__ int lds[8];
  sel_hist_body<Src, LV>(src, a, hist, lh, lds);
}

// Key-axis max pooling folded into a selection's first pass (one-call
// eviction; the pooling kernel's values bit for bit): the workgroup sums
// the raw planes of its chunk and a halo of `radius` keys, in plane order,
// into LDS (-inf outside the sequence), and each key takes the maximum over
// its window.  v: SEL_CHUNK + 2 * kPoolMaxRadius floats of LDS; keys
// j0 - r .. j0 + SEL_CHUNK + r - 1 of the sequence at `base` (n keys).
__device__ void pool_stage(const PoolSrc& P, int Hkv, int T, int h, int base, int n, int j0, float* v) {
  const int r = P.radius;
  for (int i = threadIdx.x; i < SEL_CHUNK + 2 * r; i += SEL_THREADS) {
    const int j = j0 - r + i;
    float x = -INFINITY;
    if (j >= 0 && j < n) {
      x = 0.f;
      for (int p = 0; p < P.planes; ++p) x += P.sraw[(static_cast<size_t>(p) * Hkv + h) * T + base + j];
    }
    v[i] = x;
  }
  __syncthreads();
}
// The pooled score of key j0 + jl (window v[jl .. jl + 2r]).
__device__ __forceinline__ float pool_at(const PoolSrc& P, const float* v, int jl) {
  float m = -INFINITY;
  for (int d = 0; d <= 2 * P.radius; ++d) m = fmaxf(m, v[jl + d]);
  return m;
}

// Top-k level 0 on the pooled scores, which it also writes (for every
// chunk of every head, selected or not).  The histograms are already clear.
__global__ __launch_bounds__(SEL_THREADS) void sel_hist0_pool(PoolSrc P, SelArgs a, int* __restrict__ hist) {
  typedef uint32_t K;
  __shared__ int lh[SEL_BINS];
  __shared__ float v[SEL_CHUNK + 2 * kPoolMaxRadius];
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int j0 = ch * SEL_CHUNK;
  if (j0 >= n) return;
  pool_stage(P, a.Hkv, a.T, h, base, n, j0, v);
  const size_t row = static_cast<size_t>(h) * a.T + base;
  K u[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const int jl = i * SEL_THREADS + threadIdx.x;
    u[i] = K(0);
    if (j0 + jl < n) {
      const float m = pool_at(P, v, jl);
      P.out[row + j0 + jl] = m;
      u[i] = f32_order_key(m);
    }
  }
  const int sh = s * a.Hkv + h;
  const int B = sel_budget(a, s, sh);
  if (B <= 0 || B >= n) return;
  for (int i = threadIdx.x; i < SEL_BINS; i += SEL_THREADS) lh[i] = 0;
  __syncthreads();
  const int sft = Radix<K>::shift(0);
  const K dm = Radix<K>::wmask(0);
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i)
    if (j0 + i * SEL_THREADS + static_cast<int>(threadIdx.x) < n) atomicAdd(&lh[static_cast<int>((u[i] >> sft) & dm)], 1);
  __syncthreads();
  int* gh = hist + static_cast<size_t>(sh) * SEL_BINS;   // level 0
  for (int i = threadIdx.x; i < SEL_BINS; i += SEL_THREADS) {
    const int c = lh[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Last digit level of the radix select, which also leaves the ordered write
// what a separate count launch would.  Per chunk: the number of keys whose
// leading digits (levels 0 .. LEVELS-2) exceed those of the threshold, and,
// for the keys that share them, their last digits in the chunk's own region
// of `cand` (kSelChunk ints) -- listed when at most kSelListMax, otherwise as
// suffix sums S[d] = (keys with a last digit >= d), so that the write reads
// a bounded amount per earlier chunk however many keys tie.  cnt[.][1] holds
// the listed count, or -1 for suffix sums.
// lh: SEL_BINS ints of LDS, lds: 8 ints of LDS.
template <class Src>
__device__ __forceinline__ void sel_hist_last_body(Src src, const SelArgs& a, int* __restrict__ hist,
                                                   int* __restrict__ cand, int* __restrict__ cnt, int* lh, int* lds) {
  typedef typename Src::K K;
  constexpr int LV = Radix<K>::LEVELS - 1;
  constexpr int NB = Radix<K>::LAST_BINS;
  static_assert(NB % SEL_THREADS == 0 && NB <= SEL_CHUNK, "a chunk's region holds the suffix sums");
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int sh = s * a.Hkv + h;
  const int B = sel_budget(a, s, sh);
  const int j0 = ch * SEL_CHUNK;
  if (B <= 0 || B >= n || j0 >= n) return;
  const int SH = a.S * a.Hkv;
  const size_t row = static_cast<size_t>(h) * a.T + base;
  K u[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const int j = j0 + i * SEL_THREADS + threadIdx.x;
    u[i] = (j < n) ? src.key(row + j) : K(0);
  }
  K prefix, mask;
  int need;
  resolve<K, LV>(hist, SH, sh, B, lds, &prefix, &mask, &need, a.rcache);   // its loads overlap the keys'
  for (int i = threadIdx.x; i < SEL_BINS; i += SEL_THREADS) lh[i] = 0;
  __syncthreads();   // lh cleared
  const int sft = Radix<K>::shift(LV);
  const K dm = Radix<K>::wmask(LV);
  int above = 0, nmine = 0;
  int dg[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const int j = j0 + i * SEL_THREADS + threadIdx.x;
    dg[i] = -1;
    if (j >= n) continue;
    const K lead = u[i] & mask;
    if (lead > prefix) {
      ++above;
    } else if (lead == prefix) {
      dg[i] = static_cast<int>((u[i] >> sft) & dm);
      atomicAdd(&lh[dg[i]], 1);
      ++nmine;
    }
  }
  // both counts in one scan (each field stays below 2^16)
  const int packed = (above << 16) | nmine;
  int tot;
  const int incl = block_incl_scan256(packed, lds, &tot);   // its barriers also complete lh
  const int nl = tot & 0xffff;
  const size_t ci = static_cast<size_t>(sh) * a.nchunk + ch;
  int* reg = cand + ci * SEL_CHUNK;
  if (nl <= kSelListMax) {
    int pos = (incl - packed) & 0xffff;
#pragma unroll
    for (int i = 0; i < SEL_PER; ++i)
      if (dg[i] >= 0) reg[pos++] = dg[i];
  } else {
    // thread t holds bins NB-1-Q t .. NB-Q(t+1), top down
    constexpr int Q = NB / SEL_THREADS;
    int v[Q], sum = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      v[q] = lh[NB - 1 - (threadIdx.x * Q + q)];
      sum += v[q];
    }
    int t2;
    int run = block_incl_scan256(sum, lds, &t2) - sum;   // keys in the bins above this thread's
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      run += v[q];
      reg[NB - 1 - (threadIdx.x * Q + q)] = run;
    }
  }
  if (threadIdx.x == 0) {
    cnt[ci * 2] = tot >> 16;
    cnt[ci * 2 + 1] = (nl <= kSelListMax) ? nl : -1;
  }
  int* gh = hist + (static_cast<size_t>(LV) * SH + sh) * SEL_BINS;
  for (int i = threadIdx.x; i < SEL_BINS; i += SEL_THREADS) {
    const int c = lh[i];
    if (c) atomicAdd(&gh[i], c);
  }
}
template <class Src>
__global__ __launch_bounds__(SEL_THREADS) void sel_hist_last(Src src, SelArgs a, int* __restrict__ hist,
                                                             int* __restrict__ cand, int* __restrict__ cnt) {
  __shared__ int lh[SEL_BINS];
  __shared__ int lds[8];
  sel_hist_last_body<Src>(src, a, hist, cand, cnt, lh, lds);
}

// Threshold (the B-th largest key) and the number of keys equal to it that
// are kept, per (sequence, head).
struct RState {
  uint64_t thr;
  int32_t need, pad;
};

// Per chunk: keys above the threshold and keys equal to it.  Chunk 0 also
// stores the threshold and the number of equal keys to keep.
template <class Src>
__global__ __launch_bounds__(SEL_THREADS) void sel_count(Src src, SelArgs a, const int* __restrict__ hist,
                                                         int* __restrict__ cnt, RState* __restrict__ rs) {
  typedef typename Src::K K;
  constexpr int NLV = Radix<K>::LEVELS;
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int sh = s * a.Hkv + h;
  const int B = sel_budget(a, s, sh);
  const int j0 = ch * SEL_CHUNK;
  if (B <= 0 || B >= n || j0 >= n) return;
  const int SH = a.S * a.Hkv;
  __shared__ int lds[8];
  const size_t row = static_cast<size_t>(h) * a.T + base;
  K u[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const int j = j0 + i * SEL_THREADS + threadIdx.x;
    u[i] = (j < n) ? src.key(row + j) : K(0);
  }
  K thr, mask;
  int need;
  resolve<K, NLV>(hist, SH, sh, B, lds, &thr, &mask, &need, a.rcache);
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const int j = j0 + i * SEL_THREADS + threadIdx.x;
    gt += (j < n) && (u[i] > thr);
    eq += (j < n) && (u[i] == thr);
  }
  const int packed = (gt << 16) | eq;   // each count <= SEL_CHUNK < 2^16
  int tot;
  block_incl_scan256(packed, lds, &tot);
  if (threadIdx.x == 0) {
    cnt[(static_cast<size_t>(sh) * a.nchunk + ch) * 2 + 0] = tot >> 16;
    cnt[(static_cast<size_t>(sh) * a.nchunk + ch) * 2 + 1] = tot & 0xffff;
    if (ch == 0) {
      RState r;
      r.thr = static_cast<uint64_t>(thr);
      r.need = need;
      r.pad = 0;
      rs[sh] = r;
    }
  }
}

// Bias of a kept entry: 0 (top-k) or -log(q_j) / tau_w (sampling).
struct ZeroBias {
  __device__ float operator()(int, size_t) const { return 0.f; }
};
struct SnisBias {
  const double* L;        // log1p(-pi), [Hkv][T]
  const double* mvals;    // final m per (sequence, head)
  double inv_tau_w;
  __device__ float operator()(int sh, size_t i) const {
    const double q = -expm1(mvals[sh] * L[i]);
    return static_cast<float>(-log(q) * inv_tau_w);
  }
};

// Ordered write: thread t owns keys j0 + 16t .. j0 + 16t + 15.
template <class Src, class Bias>
__global__ __launch_bounds__(SEL_THREADS) void sel_write(Src src, Bias bias_of, SelArgs a, const int* __restrict__ cnt,
                                                         const RState* __restrict__ rs, int32_t* __restrict__ idx,
                                                         float* __restrict__ bias) {
  typedef typename Src::K K;
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int j0 = ch * SEL_CHUNK;
  const int sh = s * a.Hkv + h;
  const int B = sel_budget(a, s, sh);
  if (j0 >= n) return;   // the chunks cover [0, n), which holds every output slot
  int32_t* out = idx + h * a.totalB + a.out_off[s];
  float* bout = bias + h * a.totalB + a.out_off[s];
  if (a.bsh) {   // soft budget: slots past this head's count are empty
    const int cap = a.out_off[s + 1] - a.out_off[s];
    for (int p = max(B, j0) + threadIdx.x; p < min(cap, j0 + SEL_CHUNK); p += SEL_THREADS) {
      out[p] = -1;
      bout[p] = -INFINITY;
    }
  }
  if (B <= 0) return;
  if (B >= n) {   // everything kept, weight 1
    for (int i = threadIdx.x; i < SEL_CHUNK; i += SEL_THREADS) {
      const int j = j0 + i;
      if (j < n) { out[j] = j; bout[j] = 0.f; }
    }
    return;
  }
  __shared__ int lds[8];
  const size_t row = static_cast<size_t>(h) * a.T + base;
  const int jt = j0 + SEL_PER * threadIdx.x;
  K u[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) u[i] = (jt + i < n) ? src.key(row + jt + i) : K(0);
  const K thr = static_cast<K>(rs[sh].thr);
  const int need = rs[sh].need;
  // keys above / equal to the threshold in earlier chunks
  int gt_b = 0, eq_b = 0;
  for (int c = threadIdx.x; c < ch; c += SEL_THREADS) {
    gt_b += cnt[(static_cast<size_t>(sh) * a.nchunk + c) * 2 + 0];
    eq_b += cnt[(static_cast<size_t>(sh) * a.nchunk + c) * 2 + 1];
  }
  int tot;
  block_incl_scan256(gt_b, lds, &tot);
  gt_b = tot;
  block_incl_scan256(eq_b, lds, &tot);
  eq_b = tot;
  int neq = 0;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) neq += (jt + i < n) && (u[i] == thr);
  int eq_tot;
  int eq_rank = eq_b + block_incl_scan256(neq, lds, &eq_tot) - neq;
  int ntake = 0;
  uint32_t take_bits = 0;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const bool in = jt + i < n;
    const bool gt = in && u[i] > thr;
    const bool eq = in && u[i] == thr;
    const bool take = gt || (eq && eq_rank < need);
    eq_rank += eq;
    take_bits |= static_cast<uint32_t>(take) << i;
    ntake += take;
  }
  int take_tot;
  int pos = gt_b + min(eq_b, need) + block_incl_scan256(ntake, lds, &take_tot) - ntake;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    if ((take_bits >> i) & 1u) {
      if (pos < B) {   // bounded even if the counts were inconsistent
        out[pos] = jt + i;
        bout[pos] = bias_of(sh, row + jt + i);
      }
      ++pos;
    }
  }
}

// The gather of a workgroup's kept rows into the compact cache (one-call
// eviction, [PI] §2 Eq. 3): rows ckey[r] (chunk-relative; r itself when
// ckey is NULL) of the sequence's K and V go to slots slot0 + r of KV head
// h, with their bias (0 when cbias is NULL), eight 16-byte pieces in flight
// per thread.
__device__ __forceinline__ void gather_kept(const CompactDst& cd, const int* ckey, const float* cbias, int nrow,
                                            int slot0, size_t src_row0, int h, int s) {
  const int chunks = cd.row_bytes >> 4;
  const int64_t dst0 = h * cd.totalC + cd.cap_off[s] + slot0;
  constexpr int U = 8;   // items in flight per thread
  for (int it0 = threadIdx.x; it0 < nrow * chunks; it0 += U * SEL_THREADS) {
    u32x4 kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * SEL_THREADS;
      if (it < nrow * chunks) {
        const int r = it / chunks, q = it - r * chunks;
        const size_t src = (src_row0 + static_cast<size_t>(ckey ? ckey[r] : r)) * cd.row_bytes + 16 * q;
        kv[u] = *reinterpret_cast<const u32x4*>(cd.k + src);
        vv[u] = *reinterpret_cast<const u32x4*>(cd.v + src);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * SEL_THREADS;
      if (it < nrow * chunks) {
        const int r = it / chunks, q = it - r * chunks;
        const size_t dst = static_cast<size_t>(dst0 + r) * cd.row_bytes + 16 * q;
        *reinterpret_cast<u32x4*>(cd.k_c + dst) = kv[u];
        *reinterpret_cast<u32x4*>(cd.v_c + dst) = vv[u];
        if (q == 0) cd.bias_c[dst0 + r] = cbias ? cbias[r] : 0.f;
      }
    }
  }
}

// Ordered write from sel_hist_last's counts: the threshold is resolved here
// from the finished histograms (as sel_count does); the keys above it in an
// earlier chunk are that chunk's count of larger leading digits plus its
// keys with the same leading digits and a larger last digit, and the keys
// equal to it are those with the same last digit (from the chunk's list or
// suffix sums).  The rest is sel_write's; the output is the same.
//
// With CP the workgroup also gathers the rows of the keys it keeps (listed
// in LDS, so no re-read of idx) into the compact cache: it owns the
// consecutive output slots from the count of kept keys in earlier chunks on.
template <class Src, class Bias, bool CP>
__global__ __launch_bounds__(SEL_THREADS) void sel_write_listed(Src src, Bias bias_of, SelArgs a,
                                                                const int* __restrict__ hist,
                                                                const int* __restrict__ cnt,
                                                                const int* __restrict__ cand,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ bias, CompactDst cd) {
  typedef typename Src::K K;
  constexpr int NLV = Radix<K>::LEVELS;
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int j0 = ch * SEL_CHUNK;
  const int sh = s * a.Hkv + h;
  const int B = sel_budget(a, s, sh);
  if (j0 >= n) return;   // the chunks cover [0, n), which holds every output slot
  int32_t* out = idx + h * a.totalB + a.out_off[s];
  float* bout = bias + h * a.totalB + a.out_off[s];
  if (B <= 0) return;
  const size_t row = static_cast<size_t>(h) * a.T + base;
  if (B >= n) {   // everything kept, weight 1
    for (int i = threadIdx.x; i < SEL_CHUNK; i += SEL_THREADS) {
      const int j = j0 + i;
      if (j < n) { out[j] = j; bout[j] = 0.f; }
    }
    if constexpr (CP) gather_kept(cd, nullptr, nullptr, min(SEL_CHUNK, n - j0), j0, row + j0, h, s);
    return;
  }
  __shared__ int lds[8];
  const int jt = j0 + SEL_PER * threadIdx.x;
  K u[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) u[i] = (jt + i < n) ? src.key(row + jt + i) : K(0);
  K thr, mask;
  int need;
  resolve<K, NLV>(hist, a.S * a.Hkv, sh, B, lds, &thr, &mask, &need, a.rcache);
  const int dlast = static_cast<int>((thr >> Radix<K>::shift(NLV - 1)) & Radix<K>::wmask(NLV - 1));
  constexpr int NB = Radix<K>::LAST_BINS;
  int gt_b = 0, eq_b = 0;
  for (int c = threadIdx.x; c < ch; c += SEL_THREADS) {
    const size_t ci = static_cast<size_t>(sh) * a.nchunk + c;
    const int* reg = cand + ci * SEL_CHUNK;
    const int m = cnt[ci * 2 + 1];
    gt_b += cnt[ci * 2];
    if (m >= 0) {
      for (int i = 0; i < m; ++i) {
        const int d = reg[i];
        gt_b += d > dlast;
        eq_b += d == dlast;
      }
    } else {
      const int ge = reg[dlast], gt = (dlast + 1 < NB) ? reg[dlast + 1] : 0;
      gt_b += gt;
      eq_b += ge - gt;
    }
  }
  int tot;
  block_incl_scan256(gt_b, lds, &tot);
  gt_b = tot;
  block_incl_scan256(eq_b, lds, &tot);
  eq_b = tot;
  int neq = 0;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) neq += (jt + i < n) && (u[i] == thr);
  int eq_tot;
  int eq_rank = eq_b + block_incl_scan256(neq, lds, &eq_tot) - neq;
  int ntake = 0;
  uint32_t take_bits = 0;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const bool in = jt + i < n;
    const bool gt = in && u[i] > thr;
    const bool eq = in && u[i] == thr;
    const bool take = gt || (eq && eq_rank < need);
    eq_rank += eq;
    take_bits |= static_cast<uint32_t>(take) << i;
    ntake += take;
  }
  int take_tot;
  const int wbase = gt_b + min(eq_b, need);   // slots of earlier chunks' kept keys
  int lpos = block_incl_scan256(ntake, lds, &take_tot) - ntake;
  __shared__ int ckey[CP ? SEL_CHUNK : 1];
  __shared__ float cbias[CP ? SEL_CHUNK : 1];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    if ((take_bits >> i) & 1u) {
      if (wbase + lpos < B) {   // bounded even if the counts were inconsistent
        const float b = bias_of(sh, row + jt + i);
        out[wbase + lpos] = jt + i;
        bout[wbase + lpos] = b;
        if constexpr (CP) {
          ckey[lpos] = jt + i - j0;
          cbias[lpos] = b;
        }
      }
      ++lpos;
    }
  }
  if constexpr (CP) {
    __syncthreads();
    gather_kept(cd, ckey, cbias, max(0, min(take_tot, B - wbase)), wbase, row + j0, h, s);
  }
}

// ----------------------------------------------------------------- sampling
// The sampling passes are arithmetic-heavy (fp64 transcendentals, Philox, the
// fp32 grid) and use smaller chunks than the radix passes, so that a head's
// keys spread over four times as many workgroups.
constexpr int SMP_PER = 4;
constexpr int SMP_CHUNK = SEL_THREADS * SMP_PER;
static_assert(SMP_CHUNK == kSmpChunk, "host and device sampling chunk disagree");
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  *lo = a * b;
  *hi = __umul64hi(a, b);
}

// Philox-4x64 with 10 rounds (Salmon et al., SC'11): the block of counter
// c[0..3] under key (k0, k1), in place (c[i] becomes output word i).
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(M0, c[0], &hi0, &lo0);
    mulhilo64(M1, c[2], &hi1, &lo1);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}
// Output word 0 of the block of counter (c0, c1, c2, c3).
__device__ uint64_t philox4x64_10_w0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                     uint64_t k1) {
  uint64_t c[4] = {c0, c1, c2, c3};
  philox4x64_10(c, k0, k1);
  return c[0];
}

constexpr double kAlphaMax = 1e12;   // upper end of the search range for m

// Search state of one (sequence, head): current log m, bracket in log m,
// and whether the search has stopped (1: converged, 2: target out of reach).
struct Search {
  double u, lo, hi, done;
};
static_assert(sizeof(Search) == kSelSearchBytes, "host and device state size disagree");

struct SmpArgs {
  SelArgs g;
  const float* scores;
  double* lp;         // [Hkv][T]: log pi~, then the Gumbel keys
  double* L;          // [Hkv][T]: log1p(-pi)
  int nsmp;           // chunks of SMP_CHUNK keys per (sequence, head)
  double* part;       // [2][S*Hkv][nsmp][3] per-chunk partials (ping-pong)
  float* grid;        // [S*Hkv][nsmp][kSelGrid] per-chunk E(m) on the start grid
  Search* state;      // [2][S*Hkv] search state (ping-pong)
  double* mvals;      // [S*Hkv] final m
  double inv_tau;
  double mix;         // weight of the proposal against the uniform (1: unmixed)
  uint64_t seed;
  int global;         // soft budget: one m per sequence for all its heads (Eq. 33)
  int32_t* bsh;       // soft budget: [S*Hkv] kept count per head (written by smp_decide)
  int32_t* kept_out;  // [S*Hkv] kept counts for the caller, or NULL
};

__device__ __forceinline__ double* part_of(const SmpArgs& A, int buf, int sh, int ch) {
  const size_t SH = static_cast<size_t>(A.g.S) * A.g.Hkv;
  return A.part + ((buf * SH + sh) * A.nsmp + ch) * 3;
}

// Fixed-order sums of components c of the head's nch partials in buffer buf
// (every workgroup of the head gets the same value).
__device__ double sum_part(const SmpArgs& A, int buf, int sh, int nch, int c, double* dl) {
  double v = 0.0;
  for (int i = threadIdx.x; i < nch; i += SEL_THREADS) v += part_of(A, buf, sh, i)[c];
  return block_sum_d(v, dl);
}
// The search's view of the chunk sums: the head's own, or under a soft
// budget the mean over the sequence's heads (heads in order, then chunks).
__device__ double search_sum(const SmpArgs& A, int buf, int sh, int nch, int c, double* dl) {
  if (!A.global) return sum_part(A, buf, sh, nch, c, dl);
  const int s0 = (sh / A.g.Hkv) * A.g.Hkv;
  double v = 0.0;
  for (int h = 0; h < A.g.Hkv; ++h)
    for (int i = threadIdx.x; i < nch; i += SEL_THREADS) v += part_of(A, buf, s0 + h, i)[c];
  return block_sum_d(v, dl) / A.g.Hkv;
}
// The three components of search_sum at once (one block reduction).
__device__ void search_sum3(const SmpArgs& A, int buf, int sh, int nch, double* e, double* de, double* eh,
                            double* dl) {
  const int h0 = A.global ? (sh / A.g.Hkv) * A.g.Hkv : sh;
  const int nh = A.global ? A.g.Hkv : 1;
  double a = 0.0, b = 0.0, c = 0.0;
  for (int h = 0; h < nh; ++h)
    for (int i = threadIdx.x; i < nch; i += SEL_THREADS) {
      const double* p = part_of(A, buf, h0 + h, i);
      a += p[0];
      b += p[1];
      c += p[2];
    }
  block_sum3_d(&a, &b, &c, dl);
  *e = a / nh;
  *de = b / nh;
  *eh = c / nh;
}
__device__ double max_part(const SmpArgs& A, int buf, int sh, int nch, int c, double* dl) {
  double v = -INFINITY;
  for (int i = threadIdx.x; i < nch; i += SEL_THREADS) v = fmax(v, part_of(A, buf, sh, i)[c]);
  return block_max_d(v, dl);
}

// Whether (sequence s, chunk ch) takes part in the sampling search.
__device__ __forceinline__ bool smp_active(const SmpArgs& A, int s, int ch, int* n_out, int* B_out, int* base_out) {
  const int base = A.g.seq_off[s];
  const int n = A.g.seq_off[s + 1] - base;
  const int B = A.g.bud_off[s + 1] - A.g.bud_off[s];
  *n_out = n;
  *B_out = B;
  *base_out = base;
  return B > 0 && B < n && ch * SMP_CHUNK < n;
}

// log pi~ of key j of a row: log(max(s, 2^-126)) / tau.
__device__ __forceinline__ double smp_logpt(const SmpArgs& A, size_t i) {
  return log(static_cast<double>(fmaxf(A.scores[i], 1.17549435e-38f))) * A.inv_tau;
}
// Gumbel key with log-proposal x from Philox word w:
// x - log(-log u), u = ((w >> 11) + 0.5) 2^-53.  Key j of (sequence s,
// head h) takes word j mod 4 of the block of counter (j / 4, h, s, 0), so
// one block serves four consecutive keys.
__device__ __forceinline__ double gumbel_of(double x, uint64_t w) {
  const double uu = (static_cast<double>(w >> 11) + 0.5) * 0x1.0p-53;
  return x - log(-log(uu));
}
__device__ __forceinline__ void smp_block(const SmpArgs& A, int j4, int h, int s, uint64_t c[4]) {
  c[0] = static_cast<uint64_t>(j4);
  c[1] = static_cast<uint64_t>(h);
  c[2] = static_cast<uint64_t>(s);
  c[3] = 0ull;
  philox4x64_10(c, A.seed, 0ull);
}
// One key on its own (a whole block for one of its words).
__device__ __forceinline__ double smp_gumbel(const SmpArgs& A, double x, int j, int h, int s) {
  uint64_t c[4];
  smp_block(A, j >> 2, h, s, c);
  const int r = j & 3;
  const uint64_t w = r == 0 ? c[0] : r == 1 ? c[1] : r == 2 ? c[2] : c[3];
  return gumbel_of(x, w);
}

// Pass A: log pi~ = log(max(s, 2^-126)) / tau, its per-chunk maximum and
// the chunk's sum of exp(log pi~ - maximum) (the normaliser in parts).
// KEYS (unmixed proposal): the Gumbel keys need no normaliser, so this pass
// writes them in place of log pi~, and it also clears the selection's
// histograms ([0, nzero) of `zero`: every digit level's), which no
// workgroup of this launch touches otherwise.
// POOL (one-call eviction, KEYS only): the scores are max-pooled from the
// scorer's raw planes here (and written to P.out for every chunk of every
// head) instead of read from A.scores.
template <bool KEYS, bool POOL = false>
__global__ __launch_bounds__(SEL_THREADS) void smp_logp(SmpArgs A, int* __restrict__ zero, int nzero, PoolSrc P) {
  static_assert(KEYS || !POOL, "pooling rides on the key pass");
  if constexpr (KEYS) {
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int wg = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    for (int i = wg * SEL_THREADS + threadIdx.x; i < nzero; i += nwg * SEL_THREADS) zero[i] = 0;
  }
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  float pooled[SMP_PER];
  if constexpr (POOL) {
    static_assert(SMP_CHUNK == SEL_CHUNK, "the pooling stage covers one selection chunk");
    __shared__ float v[SEL_CHUNK + 2 * kPoolMaxRadius];
    const int pbase = A.g.seq_off[s];
    const int pn = A.g.seq_off[s + 1] - pbase;
    const int pj0 = ch * SMP_CHUNK;
    if (pj0 >= pn) return;
    pool_stage(P, A.g.Hkv, A.g.T, h, pbase, pn, pj0, v);
    const size_t prow = static_cast<size_t>(h) * A.g.T + pbase;
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) {
      const int jl = SMP_PER * threadIdx.x + i;
      pooled[i] = 0.f;
      if (pj0 + jl < pn) {
        pooled[i] = pool_at(P, v, jl);
        P.out[prow + pj0 + jl] = pooled[i];
      }
    }
  }
  int n, B, base;
  if (!smp_active(A, s, ch, &n, &B, &base)) return;
  const int sh = s * A.g.Hkv + h;
  const size_t row = static_cast<size_t>(h) * A.g.T + base;
  __shared__ double dl[4];
  double x[SMP_PER];
  double mx = -INFINITY;
  if constexpr (KEYS) {
    // four consecutive keys per thread: one Philox block gives their words;
    // log pi~ waits in the log1p(-pi) plane for the next pass
    static_assert(SMP_PER == 4, "one Philox block per thread");
    const int j0 = ch * SMP_CHUNK + SMP_PER * threadIdx.x;
    uint64_t c[4] = {0ull, 0ull, 0ull, 0ull};
    if (j0 < n) smp_block(A, j0 >> 2, h, s, c);
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) {
      const int j = j0 + i;
      x[i] = -INFINITY;
      if (j < n) {
        x[i] = POOL ? log(static_cast<double>(fmaxf(pooled[i], 1.17549435e-38f))) * A.inv_tau : smp_logpt(A, row + j);
        A.lp[row + j] = gumbel_of(x[i], c[i]);
        A.L[row + j] = x[i];
        mx = fmax(mx, x[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) {
      const int j = ch * SMP_CHUNK + i * SEL_THREADS + threadIdx.x;
      x[i] = -INFINITY;
      if (j < n) {
        x[i] = smp_logpt(A, row + j);
        A.lp[row + j] = x[i];
        mx = fmax(mx, x[i]);
      }
    }
  }
  mx = block_max_d(mx, dl);
  double z = 0.0;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) z += exp(x[i] - mx);   // exp(-inf) = 0 past the end
  z = block_sum_d(z, dl);
  if (threadIdx.x == 0) {
    double* p = part_of(A, 0, sh, ch);
    p[0] = mx;
    p[1] = z;
  }
}

// Grid of the expected-samples start: m_k = B 2^k, k = 0 .. kSelGrid - 1
// (u_k = log m_k).  A key's term d_k = 1 - (1 - pi)^(m_k) then follows
// d_(k+1) = d_k (2 - d_k) (the square of 1 - d_k), which keeps full
// relative precision when d_k is tiny, so the grid costs one expm1 per key.
// Points beyond 10^12 are clamped there (E >= B is then out of the search's
// range).
__device__ __forceinline__ double grid_u(int k, int B) {
  return fmin(log(static_cast<double>(B)) + k * 0.69314718055994531, log(kAlphaMax));
}

// log(1 - p) for 0 <= p <= 1: below 2^-10 the series -p (1 + p/2 + p^2/3 +
// ... + p^5/6), whose first omitted term is under 2^-60 p; log1p(-p) above.
__device__ __forceinline__ double log1m(double p) {
  if (p < 0x1.0p-10) {
    double t = fma(p, 1.0 / 6.0, 0.2);
    t = fma(p, t, 0.25);
    t = fma(p, t, 1.0 / 3.0);
    t = fma(p, t, 0.5);
    t = fma(p, t, 1.0);
    return -p * t;
  }
  return log1p(-p);
}

// Pass B: log1p(-pi_j) and (KEYS) the Gumbel keys of the proposal's
// logarithm, mixed or not (smp_gumbel); without KEYS pass A already wrote
// them and left log pi~ in the log1p(-pi) plane, which this pass overwrites.  Also the chunk's
// E(m) = sum 1 - (1 - pi_j)^m on the start grid, in fp32 (it only brackets
// the search; every value the search accepts is fp64).
// eg: kSelGrid x 257 floats of LDS.
template <bool KEYS>
__device__ void smp_keys_body(const SmpArgs& A, float* red) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  int n, B, base;
  if (!smp_active(A, s, ch, &n, &B, &base)) return;
  const int sh = s * A.g.Hkv + h;
  const int nch = (n + SMP_CHUNK - 1) / SMP_CHUNK;
  const size_t row = static_cast<size_t>(h) * A.g.T + base;
  __shared__ double dl[4];
  // every load first (their latencies overlap): this thread's log pi~ and,
  // with at most one chunk per thread, its chunk's part of the normaliser
  double xin[SMP_PER];
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + i * SEL_THREADS + threadIdx.x;
    xin[i] = (j < n) ? (KEYS ? A.lp[row + j] : A.L[row + j]) : 0.0;
  }
  const bool one = nch <= SEL_THREADS;
  double pm0 = -INFINITY, pz0 = 0.0;
  if (one && threadIdx.x < nch) {
    const double* p = part_of(A, 0, sh, threadIdx.x);
    pm0 = fmax(pm0, p[0]);   // as max_part folds it
    pz0 = p[1];
  }
  // log-sum-exp of the whole row from the chunk parts, in chunk order
  const double M = one ? block_max_d(pm0, dl) : max_part(A, 0, sh, nch, 0, dl);
  double zp = 0.0;
  if (one) {
    if (threadIdx.x < nch) zp = pz0 * exp(pm0 - M);
  } else {
    for (int i = threadIdx.x; i < nch; i += SEL_THREADS) {
      const double* p = part_of(A, 0, sh, i);
      zp += p[1] * exp(p[0] - M);
    }
  }
  const double lse = M + log(block_sum_d(zp, dl));
  // the keys' fp64 terms first, then (with those temporaries dead) each
  // key's run over the grid points: this thread's share of the chunk's
  // E(m_k), accumulated key by key
  float d0[SMP_PER];
#pragma unroll 2
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + i * SEL_THREADS + threadIdx.x;
    d0[i] = 0.f;
    if (j < n) {
      double x = xin[i];
      double l;
      if (KEYS && A.mix < 1.0) {   // pi' = alpha pi + (1 - alpha) / n; the keys use log pi'
        const double pm = A.mix * exp(x - lse) + (1.0 - A.mix) / n;
        l = log1p(-pm);
        x = log(pm);
      } else {
        l = log1m(exp(x - lse));
      }
      A.L[row + j] = l;
      if (KEYS) A.lp[row + j] = smp_gumbel(A, x, j, h, s);
      d0[i] = -expm1f(static_cast<float>(static_cast<double>(B) * l));
    }
  }
  float e[kSelGrid];
#pragma unroll
  for (int k = 0; k < kSelGrid; ++k) e[k] = 0.f;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    if (ch * SMP_CHUNK + i * SEL_THREADS + static_cast<int>(threadIdx.x) < n) {
      float dk = d0[i];
#pragma unroll
      for (int k = 0; k < kSelGrid; ++k) {
        e[k] += dk;
        dk *= 2.f - dk;
      }
    }
  }
  // per grid point, the chunk sum in a fixed order
  static_assert(kSelGrid == 32, "the grid sums fold 32 values");
  block_sum32(e, red);
  if (threadIdx.x < kSelGrid) A.grid[(static_cast<size_t>(sh) * A.nsmp + ch) * kSelGrid + threadIdx.x] = red[128 + threadIdx.x];
}
__global__ __launch_bounds__(SEL_THREADS) void smp_keys(SmpArgs A) {
  __shared__ float red[kRed32];
  smp_keys_body<true>(A, red);
}

// What a search step (or the finish) reads, loaded at the start of its
// launch so that the latencies overlap each other and the histogram's.  With
// a head-local search and at most one chunk per thread (`one`), thread t
// holds chunk t's grid values (step 0) or partials (later steps); otherwise
// the state update reads them itself.
struct SearchIn {
  double l[SMP_PER];   // log1p(-pi) of this thread's keys (0 past the end)
  float g[kSelGrid];   // step 0: chunk threadIdx.x's E(m) on the start grid
  double p[3];         // later steps: chunk threadIdx.x's partials of the previous step
  Search st;           // later steps: the state the previous step left
  bool one;
};
__device__ __forceinline__ void search_load(const SmpArgs& A, int step, int sh, int nch, int n, size_t row,
                                            SearchIn* in) {
  const int ch = blockIdx.x;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + i * SEL_THREADS + threadIdx.x;
    in->l[i] = (j < n) ? A.L[row + j] : 0.0;
  }
  in->one = !A.global && nch <= SEL_THREADS;
  const bool mine = in->one && static_cast<int>(threadIdx.x) < nch;
#pragma unroll
  for (int k = 0; k < kSelGrid; ++k) in->g[k] = 0.f;
  in->p[0] = in->p[1] = in->p[2] = 0.0;
  if (step == 0) {
    if (mine) {
      const float* gp = A.grid + (static_cast<size_t>(sh) * A.nsmp + threadIdx.x) * kSelGrid;
#pragma unroll
      for (int k = 0; k < kSelGrid; ++k) in->g[k] = gp[k];
    }
  } else {
    const size_t SH = static_cast<size_t>(A.g.S) * A.g.Hkv;
    in->st = A.state[(step & 1) * SH + sh];
    if (mine) {
      const double* q = part_of(A, (step - 1) & 1, sh, threadIdx.x);
      in->p[0] = q[0];
      in->p[1] = q[1];
      in->p[2] = q[2];
    }
  }
}

// The search state after step `step`: step 0 starts from the grid the keys
// pass wrote; later steps apply the update of the previous step's partials (every
// workgroup computes the same update, in the same order).  The update is a
// safeguarded Newton step in log m on E(e^u) - B (bisection of the bracket
// when the step leaves it), or stop once |E - B| <= 0.5, or -- on step 1,
// from E(10^12) -- stop with the target out of reach.
__device__ Search search_state(const SmpArgs& A, int step, int sh, int nch, int B, double* dl,
                               float* red, const SearchIn& in) {
  if (step == 0) {
    // start from the grid: the first point whose E reaches B, and a bracket
    // one grid cell wider on each side than the crossing (the grid sums are
    // fp32); log B is a true lower bound since E(m) <= m
    const double target = static_cast<double>(B);
    const int h0 = A.global ? (sh / A.g.Hkv) * A.g.Hkv : sh;
    const int nh = A.global ? A.g.Hkv : 1;
    // every grid point's head (or heads') total in one block reduction
    float v[kSelGrid];
    if (in.one) {   // one chunk per thread: its fp32 values as they are
#pragma unroll
      for (int k = 0; k < kSelGrid; ++k) v[k] = in.g[k];
    } else {
      double acc[kSelGrid];
#pragma unroll
      for (int k = 0; k < kSelGrid; ++k) acc[k] = 0.0;
      for (int hh = 0; hh < nh; ++hh)
        for (int i = threadIdx.x; i < nch; i += SEL_THREADS) {
          const float* gp = A.grid + (static_cast<size_t>(h0 + hh) * A.nsmp + i) * kSelGrid;
#pragma unroll
          for (int k = 0; k < kSelGrid; ++k) acc[k] += static_cast<double>(gp[k]);
        }
#pragma unroll
      for (int k = 0; k < kSelGrid; ++k) v[k] = static_cast<float>(acc[k]);
    }
    block_sum32(v, red);
    int kx = kSelGrid;   // first grid point with E >= B
    double Ek = 0.0, Ep = 0.0;
    for (int k = 0; k < kSelGrid; ++k) {
      const double e = static_cast<double>(red[128 + k]) / nh;
      if (e >= target) { kx = k; Ek = e; break; }
      Ep = e;
    }
    __syncthreads();
    Search st;
    // -1: still searching, and a grid point below 10^12 already exceeds the
    // target by more than the fp32 grid's error, so E(10^12) reaches the
    // band (E is increasing) and need not be evaluated
    st.done = (kx < kSelGrid && grid_u(kx, B) < log(kAlphaMax) && Ek >= target * (1.0 + 1e-5) + 1.0) ? -1.0 : 0.0;
    if (kx == 0) {
      st.u = grid_u(0, B);
    } else if (kx == kSelGrid) {
      st.u = log(kAlphaMax);
    } else {
      const double u0 = grid_u(kx - 1, B), u1 = grid_u(kx, B);
      st.u = (Ek > Ep) ? u0 + (target - Ep) / (Ek - Ep) * (u1 - u0) : u1;
    }
    st.lo = grid_u(max(kx - 2, 0), B);
    st.hi = (kx + 1 < kSelGrid) ? grid_u(kx + 1, B) : log(kAlphaMax);
    return st;
  }
  Search st = in.st;
  if (st.done > 0.0) return st;
  const int pb = (step - 1) & 1;
  double E, dE, Eh;
  if (in.one) {   // the same sums as search_sum3's for one chunk per thread
    E = in.p[0];
    dE = in.p[1];
    Eh = in.p[2];
    block_sum3_d(&E, &dE, &Eh, dl);
  } else {
    search_sum3(A, pb, sh, nch, &E, &dE, &Eh, dl);
  }
  const double target = static_cast<double>(B);
  if (step == 1 && st.done == 0.0) {
    if (Eh < target - 0.5) {   // no m in [0, 10^12] reaches the band
      st.done = 2.0;
      return st;
    }
  }
  const double g = E - target;
  if (fabs(g) <= 0.5) {
    st.done = 1.0;
    return st;
  }
  if (g < 0.0) st.lo = st.u; else st.hi = st.u;
  const double dg = exp(st.u) * dE;   // dE / dlog m
  double un = (dg > 0.0) ? st.u - g / dg : 0.5 * (st.lo + st.hi);
  if (!(un > st.lo && un < st.hi)) un = 0.5 * (st.lo + st.hi);
  st.u = un;
  return st;
}

// One step of the expected-samples search: brings the state up to date,
// then (if still searching) writes the chunk's E(m), dE/dm at m = e^u, and
// on the first step also E(10^12).
// red: kRed32 floats of LDS, used on step 0 only (may be NULL after);
// in: search_load's values for this workgroup.
__device__ void smp_search_body(const SmpArgs& A, int step, float* red, const SearchIn& in) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  int n, B, base;
  if (!smp_active(A, s, ch, &n, &B, &base)) return;
  const int sh = s * A.g.Hkv + h;
  const int nch = (n + SMP_CHUNK - 1) / SMP_CHUNK;
  const size_t SH = static_cast<size_t>(A.g.S) * A.g.Hkv;
  __shared__ double dl[12];
  const Search st = search_state(A, step, sh, nch, B, dl, red, in);
  if (ch == 0 && threadIdx.x == 0) A.state[((step + 1) & 1) * SH + sh] = st;
  if (st.done > 0.0) return;
  const bool want_eh = step == 0 && st.done == 0.0;
  const double m = exp(st.u);
  double e = 0.0, de = 0.0, eh = 0.0;
#pragma unroll 4
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + i * SEL_THREADS + threadIdx.x;
    if (j < n) {
      const double l = in.l[i];
      const double x = expm1(m * l);
      e -= x;
      de -= l * (x + 1.0);
      if (want_eh) eh -= expm1(kAlphaMax * l);
    }
  }
  block_sum3_d(&e, &de, &eh, dl);
  if (threadIdx.x == 0) {
    double* p = part_of(A, step & 1, sh, ch);
    p[0] = e;
    p[1] = de;
    p[2] = eh;
  }
}

// Brings the state up to date after the last step, then writes the chunk's
// E at m0 = floor(e^u) and m0 + 1 (one of them lies in the band when the
// search converged: E rises by at most 1 per unit step).
__device__ void smp_finish_body(const SmpArgs& A, int steps, const SearchIn& in) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  int n, B, base;
  if (!smp_active(A, s, ch, &n, &B, &base)) return;
  const int sh = s * A.g.Hkv + h;
  const int nch = (n + SMP_CHUNK - 1) / SMP_CHUNK;
  const size_t SH = static_cast<size_t>(A.g.S) * A.g.Hkv;
  __shared__ double dl[12];
  const Search st = search_state(A, steps, sh, nch, B, dl, nullptr, in);   // steps >= 1: no grid
  if (ch == 0 && threadIdx.x == 0) A.state[((steps + 1) & 1) * SH + sh] = st;
  // out of reach: E at 10^12 (the second value), which sets a head's count
  // under a soft budget
  const double m0 = (st.done == 2.0) ? kAlphaMax - 1.0 : fmin(floor(exp(st.u)), kAlphaMax - 1.0);
  double e0 = 0.0, e1 = 0.0;
#pragma unroll 4
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + i * SEL_THREADS + threadIdx.x;
    if (j < n) {
      const double l = in.l[i];
      e0 -= expm1(m0 * l);
      e1 -= expm1((m0 + 1.0) * l);
    }
  }
  e0 = block_sum_d(e0, dl);
  e1 = block_sum_d(e1, dl);
  if (threadIdx.x == 0) {
    double* p = part_of(A, steps & 1, sh, ch);
    p[0] = e0;
    p[1] = e1;
    p[2] = 0.0;
  }
}

// E(m) = sum_j -expm1(m log1p(-pi_j)) of the head (fp64, fixed order), or
// with `mean` the mean over the sequence's heads (the soft budget, Eq. 33).
__device__ double expected_at(const SmpArgs& A, bool mean, int s, int sh, int n, int base, double m, double* dl) {
  const int h0 = mean ? 0 : sh - s * A.g.Hkv;
  const int nh = mean ? A.g.Hkv : 1;
  double v = 0.0;
  for (int hh = 0; hh < nh; ++hh) {
    const double* L = A.L + static_cast<size_t>(h0 + hh) * A.g.T + base;
    for (int j = threadIdx.x; j < n; j += SEL_THREADS) v -= expm1(m * L[j]);
  }
  return block_sum_d(v, dl) / nh;
}

// Final m and status per (sequence, head): the first of m0, m0 + 1 in the
// band; 10^12 and KVE_ENOCONV if the target is out of reach.  If neither
// integer is in the band (the Newton steps ran out), the pages' integer
// binary search ("A Probabilistic Interpretation of KV Cache Eviction",
// App. F, Algorithm 2) continues on the search's bracket, widened to [0,
// 10^12] if its ends do not straddle the target; since E rises by at most 1
// per unit step and E(10^12) reaches the band, it ends in the band (at most
// about 40 evaluations, in this workgroup).  Under a soft budget the band is
// on the heads' mean (every head of a sequence decides the same m) and each
// head keeps floor(E_h(m) + 0.5) entries, clamped to its sequence length and
// capacity.  One workgroup per head.
__device__ void smp_decide_body(const SmpArgs& A, int steps, double* m_out, int32_t* status_out, int h, int s) {
  const int sh = s * A.g.Hkv + h;
  int n, B, base;
  const bool active = smp_active(A, s, 0, &n, &B, &base);
  double m = 0.0;
  int status = KVE_OK;
  int kept = (B >= n) ? n : max(B, 0);
  if (active) {
    const size_t SH = static_cast<size_t>(A.g.S) * A.g.Hkv;
    const int nch = (n + SMP_CHUNK - 1) / SMP_CHUNK;
    __shared__ double dl[12];
    const Search st = A.state[((steps + 1) & 1) * SH + sh];
    double E0, E1, unused;
    search_sum3(A, steps & 1, sh, nch, &E0, &E1, &unused, dl);
    int which;   // 0: m0, 1: m0 + 1 (or 10^12), 2: found by the binary search
    if (st.done == 2.0) {
      m = kAlphaMax;
      which = 1;
      status = KVE_ENOCONV;
    } else {
      const double target = static_cast<double>(B);
      const double m0 = fmin(floor(exp(st.u)), kAlphaMax - 1.0);
      if (fabs(E0 - target) <= 0.5) {
        which = 0;
        m = m0;
      } else if (fabs(E1 - target) <= 0.5) {
        which = 1;
        m = m0 + 1.0;
      } else {
        which = 2;
        double lo = fmax(floor(exp(st.lo)), 0.0), hi = fmin(ceil(exp(st.hi)), kAlphaMax);
        if (expected_at(A, A.global, s, sh, n, base, lo, dl) > target + 0.5) lo = 0.0;
        if (expected_at(A, A.global, s, sh, n, base, hi, dl) < target - 0.5) hi = kAlphaMax;
        m = -1.0;
        while (lo <= hi) {
          const double mid = floor(0.5 * (lo + hi));
          const double e = expected_at(A, A.global, s, sh, n, base, mid, dl);
          if (fabs(e - target) <= 0.5) {
            m = mid;
            break;
          }
          if (e < target) lo = mid + 1.0;
          else hi = mid - 1.0;
        }
        if (m < 0.0) {   // unreachable when E(10^12) reaches the band
          m = kAlphaMax;
          status = KVE_ENOCONV;
        }
      }
    }
    if (A.global) {
      const double Eh = (which == 2) ? expected_at(A, false, s, sh, n, base, m, dl)
                                     : sum_part(A, steps & 1, sh, nch, which, dl);
      const int cap = A.g.out_off[s + 1] - A.g.out_off[s];
      kept = static_cast<int>(fmin(fmax(floor(Eh + 0.5), 0.0), static_cast<double>(min(n, cap))));
    }
  } else if (A.global) {
    kept = min(kept, A.g.out_off[s + 1] - A.g.out_off[s]);
  }
  if (threadIdx.x == 0) {
    A.mvals[sh] = m;
    if (m_out) m_out[sh] = m;
    if (status_out) status_out[sh] = status;
    if (A.bsh) A.bsh[sh] = kept;
    if (A.kept_out) A.kept_out[sh] = kept;
  }
}

// search_load for this workgroup's chunk; false if the chunk takes no part.
__device__ __forceinline__ bool search_load_wg(const SmpArgs& A, int step, SearchIn* in) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  int n, B, base;
  if (!smp_active(A, s, ch, &n, &B, &base)) return false;
  search_load(A, step, s * A.g.Hkv + h, (n + SMP_CHUNK - 1) / SMP_CHUNK, n, static_cast<size_t>(h) * A.g.T + base,
              in);
  return true;
}

__global__ __launch_bounds__(SEL_THREADS) void smp_search(SmpArgs A, int step) {
  __shared__ float red[kRed32];
  SearchIn in;
  if (!search_load_wg(A, step, &in)) return;
  smp_search_body(A, step, red, in);
}
__global__ __launch_bounds__(SEL_THREADS) void smp_finish(SmpArgs A, int steps) {
  SearchIn in;
  if (!search_load_wg(A, steps, &in)) return;
  smp_finish_body(A, steps, in);
}
__global__ __launch_bounds__(SEL_THREADS) void smp_decide(SmpArgs A, int steps, double* m_out, int32_t* status_out) {
  smp_decide_body(A, steps, m_out, status_out, blockIdx.x, blockIdx.y);
}

// The Gumbel keys' radix digit levels do not depend on m (the kept set is
// the top B of the keys whatever m the search returns), so with a per-head
// budget each search launch also makes one histogram level of the keys over
// the same chunk (the sampling and radix chunks are both 1024 keys):
// search steps with levels 0 .. steps-1, the finish with level steps, and
// the decision (in the first chunk's workgroup of each head) with the next.
// Step 0 (which sums the start grid) shares one LDS block between its two
// parts; the others hold only the histogram's.
// The search's loads go out first, then the histogram runs (its own loads
// overlap them), then the search step; a chunk outside the search (budget
// 0, at least n, or past the end) is outside the histograms too.
template <int LV, bool FIRST>
__global__ __launch_bounds__(SEL_THREADS) void smp_search_hist(SmpArgs A, int step, int* __restrict__ hist) {
  // per-head budgets only (never the soft budget's shared m); step 0 is
  // the FIRST launch's, so each instance compiles only its own state update
  __builtin_assume(A.global == 0);
  __builtin_assume(FIRST ? step == 0 : step > 0);
  __shared__ int lds[8];
  SearchIn in;
  if (!search_load_wg(A, step, &in)) return;
  if constexpr (FIRST) {
    __shared__ int lh[SEL_BINS];
    __shared__ float red[kRed32];
    sel_hist_body<GumbelKeys, LV>(GumbelKeys{A.lp}, A.g, hist, lh, lds);
    smp_search_body(A, step, red, in);
  } else {
    __shared__ int lh[SEL_BINS];
    sel_hist_body<GumbelKeys, LV>(GumbelKeys{A.lp}, A.g, hist, lh, lds);
    smp_search_body(A, step, nullptr, in);
  }
}
template <int LV>
__global__ __launch_bounds__(SEL_THREADS) void smp_finish_hist(SmpArgs A, int steps, int* __restrict__ hist) {
  __builtin_assume(A.global == 0);
  __builtin_assume(steps > 0);
  __shared__ int lh[SEL_BINS];
  __shared__ int lds[8];
  SearchIn in;
  if (!search_load_wg(A, steps, &in)) return;
  sel_hist_body<GumbelKeys, LV>(GumbelKeys{A.lp}, A.g, hist, lh, lds);
  smp_finish_body(A, steps, in);
}
template <int LV>
__global__ __launch_bounds__(SEL_THREADS) void smp_decide_hist(SmpArgs A, int steps, double* m_out,
                                                               int32_t* status_out, int* __restrict__ hist) {
  __builtin_assume(A.global == 0);
  __shared__ int lh[SEL_BINS];
  __shared__ int lds[8];
  if (blockIdx.x == 0) smp_decide_body(A, steps, m_out, status_out, blockIdx.y, blockIdx.z);
  sel_hist_body<GumbelKeys, LV>(GumbelKeys{A.lp}, A.g, hist, lh, lds);
}
// Pass B without the keys (pass A wrote them), with the keys' level 0.
__global__ __launch_bounds__(SEL_THREADS) void smp_grid_hist(SmpArgs A, int* __restrict__ hist) {
  __shared__ int lds[8];
  __shared__ int lh[SEL_BINS];
  __shared__ float red[kRed32];
  smp_keys_body<false>(A, red);
  sel_hist_body<GumbelKeys, 0>(GumbelKeys{A.lp}, A.g, hist, lh, lds);
}
// The decision with the keys' last level (its candidate list and counts).
__global__ __launch_bounds__(SEL_THREADS) void smp_decide_last(SmpArgs A, int steps, double* m_out,
                                                               int32_t* status_out, int* __restrict__ hist,
                                                               int* __restrict__ cand, int* __restrict__ cnt) {
  __builtin_assume(A.global == 0);
  __shared__ int lh[SEL_BINS];
  __shared__ int lds[8];
  if (blockIdx.x == 0) smp_decide_body(A, steps, m_out, status_out, blockIdx.y, blockIdx.z);
  sel_hist_last_body<GumbelKeys>(GumbelKeys{A.lp}, A.g, hist, cand, cnt, lh, lds);
}

// ------------------------------------------------------- literal estimator
// "A Probabilistic Interpretation of KV Cache Eviction", §4 (keep the
// entries drawn at least once in m draws with replacement from pi),
// Algorithm 1 step 4 and Eq. 10 (weight c_j / (m pi_j), tempered): draw k
// takes u_k from Philox-4x64-10 on counter (k, h, s, 1) and lands on the
// first entry whose cumulative probability exceeds u_k times the total.
// The cumulative sums are chunk-local fp64 scans plus chunk offsets summed
// in chunk order; counts are integer atomics, so results are reproducible.
struct LitArgs {
  const int32_t* seq_off;
  const int32_t* cap_off;
  const float* scores;
  const double* m_in;     // [S*Hkv] draws per head
  int S, Hkv, T, nch;     // nch: chunks of SMP_CHUNK keys per (sequence, head), maximum
  int64_t total_cap;
  double inv_tau, mix, inv_tau_w;
  uint64_t seed;
  double* part;           // [S*Hkv][nch][2] chunk max and sum of exp, then [.][.][0] chunk mass
  double* pi;             // [Hkv][T] proposal
  double* cdf;            // [Hkv][T] chunk-local inclusive cumulative proposal
  int* cnt;               // [Hkv][T] draw counts (cleared first)
  int* nz;                // [S*Hkv][nch] drawn entries per chunk
  int32_t* idx;
  float* bias;
  int32_t* kept;          // [S*Hkv] or NULL
  int32_t* status;        // [S*Hkv] or NULL
};

// Draws of one head: m when it is a whole number in [0, kLitMaxDraws], else -1.
__device__ __forceinline__ int64_t lit_draws(const LitArgs& A, int sh) {
  const double m = A.m_in[sh];
  if (!(m >= 0.0 && m <= static_cast<double>(kLitMaxDraws)) || m != floor(m)) return -1;
  return static_cast<int64_t>(m);
}

// Inclusive scan of doubles over a 256-thread block in a fixed order; lds: 4.
__device__ __forceinline__ double block_incl_scan256_d(double v, double* lds, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) lds[wave] = v;
  __syncthreads();
  double off = 0.0;
  for (int wv = 0; wv < wave; ++wv) off += lds[wv];
  *total = ((lds[0] + lds[1]) + lds[2]) + lds[3];
  __syncthreads();
  return v + off;
}

// Pass 1: log pi~ and the chunk's max and sum of exp (the normaliser in parts).
__global__ __launch_bounds__(SEL_THREADS) void lit_logp(LitArgs A) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = A.seq_off[s], n = A.seq_off[s + 1] - base;
  if (ch * SMP_CHUNK >= n) return;
  const int sh = s * A.Hkv + h;
  const size_t row = static_cast<size_t>(h) * A.T + base;
  __shared__ double dl[4];
  double x[SMP_PER];
  double mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + SMP_PER * threadIdx.x + i;
    x[i] = -INFINITY;
    if (j < n) {
      x[i] = log(static_cast<double>(fmaxf(A.scores[row + j], 1.17549435e-38f))) * A.inv_tau;
      A.pi[row + j] = x[i];
      mx = fmax(mx, x[i]);
    }
  }
  mx = block_max_d(mx, dl);
  double z = 0.0;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) z += exp(x[i] - mx);
  z = block_sum_d(z, dl);
  if (threadIdx.x == 0) {
    double* p = A.part + (static_cast<size_t>(sh) * A.nch + ch) * 2;
    p[0] = mx;
    p[1] = z;
  }
}

// Pass 2: pi (mixed with the uniform when mix < 1), its chunk-local
// cumulative sums and the chunk's mass.
__global__ __launch_bounds__(SEL_THREADS) void lit_cdf(LitArgs A) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = A.seq_off[s], n = A.seq_off[s + 1] - base;
  if (ch * SMP_CHUNK >= n) return;
  const int sh = s * A.Hkv + h;
  const int nc = (n + SMP_CHUNK - 1) / SMP_CHUNK;
  const size_t row = static_cast<size_t>(h) * A.T + base;
  __shared__ double dl[4];
  const double* pp = A.part + static_cast<size_t>(sh) * A.nch * 2;
  double M = -INFINITY;
  for (int i = threadIdx.x; i < nc; i += SEL_THREADS) M = fmax(M, pp[2 * i]);
  M = block_max_d(M, dl);
  double zp = 0.0;
  for (int i = threadIdx.x; i < nc; i += SEL_THREADS) zp += pp[2 * i + 1] * exp(pp[2 * i] - M);
  const double lse = M + log(block_sum_d(zp, dl));
  double v[SMP_PER], acc = 0.0;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + SMP_PER * threadIdx.x + i;
    double p = 0.0;
    if (j < n) {
      p = exp(A.pi[row + j] - lse);
      if (A.mix < 1.0) p = A.mix * p + (1.0 - A.mix) / n;
    }
    v[i] = p;
    acc += p;
  }
  double tot;
  double run = block_incl_scan256_d(acc, dl, &tot) - acc;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + SMP_PER * threadIdx.x + i;
    run += v[i];
    if (j < n) {
      A.pi[row + j] = v[i];
      A.cdf[row + j] = run;
    }
  }
}

// Pass 3: the draws.  Every workgroup of a head forms the chunk offsets
// (masses summed in chunk order, from each chunk's last cumulative value),
// then its threads take draws k = t, t + stride, ... below m.
constexpr int LIT_DRAW_WGS = 256;    // workgroups per head
constexpr int LIT_MAX_CHUNKS = 4096; // chunk offsets held in LDS (n <= 4M)
__global__ __launch_bounds__(SEL_THREADS) void lit_draw(LitArgs A) {
  const int h = blockIdx.y, s = blockIdx.z;
  const int base = A.seq_off[s], n = A.seq_off[s + 1] - base;
  const int sh = s * A.Hkv + h;
  const int64_t m = lit_draws(A, sh);
  if (n <= 0 || m <= 0) return;
  const int nc = (n + SMP_CHUNK - 1) / SMP_CHUNK;
  const size_t row = static_cast<size_t>(h) * A.T + base;
  __shared__ double off[LIT_MAX_CHUNKS + 1];
  __shared__ double dl[4];
  // exclusive offsets of the chunks: a block scan per 256 chunks, carried in order
  double carry = 0.0;
  for (int c0 = 0; c0 < nc; c0 += SEL_THREADS) {
    const int c = c0 + threadIdx.x;
    const double mass = (c < nc) ? A.cdf[row + min(n, (c + 1) * SMP_CHUNK) - 1] : 0.0;
    double tot;
    const double incl = block_incl_scan256_d(mass, dl, &tot);
    if (c < nc) off[c] = carry + (incl - mass);
    carry += tot;
  }
  if (threadIdx.x == 0) off[nc] = carry;
  __syncthreads();
  const double total = off[nc];
  const int64_t stride = static_cast<int64_t>(LIT_DRAW_WGS) * SEL_THREADS;
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * SEL_THREADS + threadIdx.x; k < m; k += stride) {
    const uint64_t w = philox4x64_10_w0(static_cast<uint64_t>(k), static_cast<uint64_t>(h),
                                        static_cast<uint64_t>(s), 1ull, A.seed, 0ull);
    const double t = ((static_cast<double>(w >> 11) + 0.5) * 0x1.0p-53) * total;
    // first chunk whose end exceeds t
    int lo = 0, hi = nc - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (off[mid + 1] > t) hi = mid; else lo = mid + 1;
    }
    // first entry of that chunk whose cumulative value exceeds t
    const int j0 = lo * SMP_CHUNK;
    int a = j0, b = min(n, j0 + SMP_CHUNK) - 1;
    while (a < b) {
      const int mid = (a + b) >> 1;
      if (off[lo] + A.cdf[row + mid] > t) b = mid; else a = mid + 1;
    }
    atomicAdd(&A.cnt[row + a], 1);
  }
}

// Pass 4: entries drawn at least once, per chunk.
__global__ __launch_bounds__(SEL_THREADS) void lit_count(LitArgs A) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = A.seq_off[s], n = A.seq_off[s + 1] - base;
  if (ch * SMP_CHUNK >= n) return;
  const int sh = s * A.Hkv + h;
  const size_t row = static_cast<size_t>(h) * A.T + base;
  __shared__ int lds[8];
  int c = 0;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + SMP_PER * threadIdx.x + i;
    c += (j < n) && A.cnt[row + j] > 0;
  }
  int tot;
  block_incl_scan256(c, lds, &tot);
  if (threadIdx.x == 0) A.nz[static_cast<size_t>(sh) * A.nch + ch] = tot;
}

// Pass 5: ordered write of the drawn entries into the head's capacity slots,
// bias log(c_j / (m pi_j)) / tau_w; slots past the drawn count get -1 and
// -inf; the chunk that holds the last entry reports the count and status.
__global__ __launch_bounds__(SEL_THREADS) void lit_write(LitArgs A) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = A.seq_off[s], n = A.seq_off[s + 1] - base;
  if (ch * SMP_CHUNK >= n) return;
  const int sh = s * A.Hkv + h;
  const int nc = (n + SMP_CHUNK - 1) / SMP_CHUNK;
  const int cap = A.cap_off[s + 1] - A.cap_off[s];
  const int64_t m = lit_draws(A, sh);
  const size_t row = static_cast<size_t>(h) * A.T + base;
  int32_t* out = A.idx + h * A.total_cap + A.cap_off[s];
  float* bout = A.bias + h * A.total_cap + A.cap_off[s];
  __shared__ int lds[8];
  int before = 0, all = 0;
  for (int c = threadIdx.x; c < nc; c += SEL_THREADS) {
    const int v = A.nz[static_cast<size_t>(sh) * A.nch + c];
    before += (c < ch) ? v : 0;
    all += v;
  }
  int tot;
  block_incl_scan256(before, lds, &tot);
  before = tot;
  block_incl_scan256(all, lds, &tot);
  const int J = (m > 0) ? tot : 0;
  int take = 0;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = ch * SMP_CHUNK + SMP_PER * threadIdx.x + i;
    take += (m > 0) && (j < n) && A.cnt[row + j] > 0;
  }
  int pos = before + block_incl_scan256(take, lds, &tot) - take;
  if (m > 0) {
    const double lm = log(static_cast<double>(m));
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) {
      const int j = ch * SMP_CHUNK + SMP_PER * threadIdx.x + i;
      if (j < n && A.cnt[row + j] > 0) {
        if (pos < cap) {
          out[pos] = j;
          bout[pos] = static_cast<float>((log(static_cast<double>(A.cnt[row + j])) - lm - log(A.pi[row + j])) *
                                         A.inv_tau_w);
        }
        ++pos;
      }
    }
  }
  for (int p = max(J, ch * SMP_CHUNK) + threadIdx.x; p < min(cap, (ch + 1) * SMP_CHUNK); p += SEL_THREADS) {
    out[p] = -1;
    bout[p] = -INFINITY;
  }
  if (ch == nc - 1 && threadIdx.x == 0) {
    if (A.kept) A.kept[sh] = J;
    if (A.status) A.status[sh] = (m < 0) ? KVE_ENOTSUP : KVE_OK;
  }
}

__global__ __launch_bounds__(256) void lit_clear(int* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0;
}

hipError_t launch_literal(const LiteralGeom& G, const int32_t* seq_off, const float* scores, const double* m_in,
                          const int32_t* cap_off, int64_t total_cap, float tau, float tau_w, float mix,
                          uint64_t seed, int32_t* idx, float* bias, int32_t* kept, int32_t* status, void* ws,
                          hipStream_t st) {
  char* wsb = static_cast<char*>(ws);
  LitArgs A;
  A.seq_off = seq_off;
  A.cap_off = cap_off;
  A.scores = scores;
  A.m_in = m_in;
  A.S = G.S;
  A.Hkv = G.Hkv;
  A.T = G.T;
  A.nch = G.nch;
  A.total_cap = total_cap;
  A.inv_tau = 1.0 / static_cast<double>(tau);
  A.mix = static_cast<double>(mix);
  A.inv_tau_w = 1.0 / static_cast<double>(tau_w);
  A.seed = seed;
  A.part = reinterpret_cast<double*>(wsb + G.off_part);
  A.pi = reinterpret_cast<double*>(wsb + G.off_pi);
  A.cdf = reinterpret_cast<double*>(wsb + G.off_cdf);
  A.cnt = reinterpret_cast<int*>(wsb + G.off_cnt);
  A.nz = reinterpret_cast<int*>(wsb + G.off_nz);
  A.idx = idx;
  A.bias = bias;
  A.kept = kept;
  A.status = status;
  const int64_t ncnt = static_cast<int64_t>(G.Hkv) * G.T;
  const dim3 grid(G.nch, G.Hkv, G.S);
  stage_begin(ST_SELECT, st);
  hipLaunchKernelGGL(lit_clear, dim3(static_cast<unsigned>((ncnt + 255) / 256 < 4096 ? (ncnt + 255) / 256 : 4096)), dim3(256), 0, st,
                     A.cnt, ncnt);
  hipLaunchKernelGGL(lit_logp, grid, dim3(SEL_THREADS), 0, st, A);
  hipLaunchKernelGGL(lit_cdf, grid, dim3(SEL_THREADS), 0, st, A);
  hipLaunchKernelGGL(lit_draw, dim3(LIT_DRAW_WGS, G.Hkv, G.S), dim3(SEL_THREADS), 0, st, A);
  hipLaunchKernelGGL(lit_count, grid, dim3(SEL_THREADS), 0, st, A);
  hipLaunchKernelGGL(lit_write, grid, dim3(SEL_THREADS), 0, st, A);
  stage_end(ST_SELECT, st);
  return hipGetLastError();
}

// ----------------------------------------------------------------- launch
template <class Src, class Bias>
static void launch_radix(const SelectGeom& G, const SelArgs& a, Src src, Bias bias_of, int* hist, int* cnt,
                         RState* rs, int32_t* idx, float* bias, hipStream_t st, int* cand,
                         const PoolSrc* pool = nullptr, const CompactDst* compact = nullptr) {
  typedef typename Src::K K;
  const dim3 grid(G.nchunk, G.Hkv, G.S);
  if (a.bsh == nullptr) {   // no count launch (not under a soft budget)
    if (pool)   // level 0 on the scores it pools (and writes)
      hipLaunchKernelGGL(sel_hist0_pool, grid, dim3(SEL_THREADS), 0, st, *pool, a, hist);
    else
      hipLaunchKernelGGL((sel_hist<Src, 0>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
    hipLaunchKernelGGL((sel_hist<Src, 1>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
    if (Radix<K>::LEVELS > 3) {
      hipLaunchKernelGGL((sel_hist<Src, 2>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
      hipLaunchKernelGGL((sel_hist<Src, 3>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
      hipLaunchKernelGGL((sel_hist<Src, 4>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
    }
    hipLaunchKernelGGL((sel_hist_last<Src>), grid, dim3(SEL_THREADS), 0, st, src, a, hist, cand, cnt);
    if (compact)
      hipLaunchKernelGGL((sel_write_listed<Src, Bias, true>), grid, dim3(SEL_THREADS), 0, st, src, bias_of, a, hist,
                         cnt, cand, idx, bias, *compact);
    else
      hipLaunchKernelGGL((sel_write_listed<Src, Bias, false>), grid, dim3(SEL_THREADS), 0, st, src, bias_of, a, hist,
                         cnt, cand, idx, bias, CompactDst{});
    return;
  }
  hipLaunchKernelGGL((sel_hist<Src, 0>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
  hipLaunchKernelGGL((sel_hist<Src, 1>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
  hipLaunchKernelGGL((sel_hist<Src, 2>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
  if (Radix<K>::LEVELS > 3) {
    hipLaunchKernelGGL((sel_hist<Src, 3>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
    hipLaunchKernelGGL((sel_hist<Src, 4>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
    hipLaunchKernelGGL((sel_hist<Src, 5>), grid, dim3(SEL_THREADS), 0, st, src, a, hist);
  }
  hipLaunchKernelGGL((sel_count<Src>), grid, dim3(SEL_THREADS), 0, st, src, a, hist, cnt, rs);
  hipLaunchKernelGGL((sel_write<Src, Bias>), grid, dim3(SEL_THREADS), 0, st, src, bias_of, a, cnt, rs, idx, bias);
}

// Top-k when every sequence fits one selection chunk (at most SEL_CHUNK
// keys): one workgroup per (sequence, head) resolves the three digit levels
// in LDS and writes the ordered output itself, in one launch (the same
// selection as the multi-workgroup path: the B largest keys, ties to the
// lower index, NaN below every number).  Also writes m = 0 and status OK.
__global__ __launch_bounds__(SEL_THREADS) void sel_topk_one(const float* __restrict__ scores, SelArgs a,
                                                            int32_t* __restrict__ idx, float* __restrict__ bias,
                                                            double* m_out, int32_t* status_out) {
  typedef uint32_t K;
  const int h = blockIdx.y, s = blockIdx.z;
  const int sh = s * a.Hkv + h;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int B = a.bud_off[s + 1] - a.bud_off[s];
  if (threadIdx.x == 0) {
    if (m_out) m_out[sh] = 0.0;
    if (status_out) status_out[sh] = KVE_OK;
  }
  int32_t* out = idx + h * a.totalB + a.out_off[s];
  float* bout = bias + h * a.totalB + a.out_off[s];
  if (B <= 0) return;
  if (B >= n) {   // everything kept, weight 0
    for (int j = threadIdx.x; j < n; j += SEL_THREADS) {
      out[j] = j;
      bout[j] = 0.f;
    }
    return;
  }
  __shared__ int lh[SEL_BINS];
  __shared__ int lds[8];
  const size_t row = static_cast<size_t>(h) * a.T + base;
  // thread t holds keys 4t .. 4t+3 (the ordered write's layout)
  const int jt = SEL_PER * threadIdx.x;
  K u[SEL_PER];
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) u[i] = (jt + i < n) ? f32_order_key(scores[row + jt + i]) : K(0);
  K prefix = 0, mask = 0;
  int need = B;
#pragma unroll 1
  for (int lv = 0; lv < Radix<K>::LEVELS; ++lv) {
    for (int i = threadIdx.x; i < SEL_BINS; i += SEL_THREADS) lh[i] = 0;
    __syncthreads();
    const int sft = Radix<K>::shift(lv);
    const K dm = Radix<K>::wmask(lv);
#pragma unroll
    for (int i = 0; i < SEL_PER; ++i)
      if (jt + i < n && (u[i] & mask) == prefix) atomicAdd(&lh[static_cast<int>((u[i] >> sft) & dm)], 1);
    __syncthreads();
    int c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = lh[SEL_BINS - 1 - 8 * threadIdx.x - i];
    int dg, ab;
    pick_bin(c, need, lds, &dg, &ab);   // its barriers also end this level's reads of lh
    prefix |= static_cast<K>(dg) << sft;
    mask |= dm << sft;
    need -= ab;
  }
  const K thr = prefix;   // the B-th largest key; `need` of the keys equal to it are kept
  int neq = 0;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) neq += (jt + i < n) && (u[i] == thr);
  int tot;
  int eq_rank = block_incl_scan256(neq, lds, &tot) - neq;
  int ntake = 0;
  uint32_t take_bits = 0;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const bool in = jt + i < n;
    const bool eq = in && u[i] == thr;
    const bool take = (in && u[i] > thr) || (eq && eq_rank < need);
    eq_rank += eq;
    take_bits |= static_cast<uint32_t>(take) << i;
    ntake += take;
  }
  int pos = block_incl_scan256(ntake, lds, &tot) - ntake;
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    if ((take_bits >> i) & 1u) {
      if (pos < B) {
        out[pos] = jt + i;
        bout[pos] = 0.f;
      }
      ++pos;
    }
  }
}

// Clears the histograms and, in top-k mode, writes m = 0 and status OK.
__global__ __launch_bounds__(256) void sel_init(int* __restrict__ p, int n, double* m_out, int32_t* status_out,
                                                int SH) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
  if (i < SH) {
    if (m_out) m_out[i] = 0.0;
    if (status_out) status_out[i] = KVE_OK;
  }
}

hipError_t launch_select(const SelectGeom& G, const float* scores, const int32_t* seq_off,
                         const int32_t* bud_off, float tau, float tau_w, float mix, uint64_t seed,
                         int32_t* idx, float* bias, double* m_out, int32_t* status_out, void* ws,
                         hipStream_t st, const SoftBudget* soft, const PoolSrc* pool,
                         const CompactDst* compact) {
  char* wsb = static_cast<char*>(ws);
  int* hist = reinterpret_cast<int*>(wsb + G.off_hist);
  int* cnt = reinterpret_cast<int*>(wsb + G.off_cnt);
  RState* rs = reinterpret_cast<RState*>(wsb + G.off_rstate);
  static_assert(sizeof(RState) == kSelRStateBytes, "host and device state size disagree");
  const int SH = G.S * G.Hkv;
  SelArgs a;
  a.seq_off = seq_off;
  a.bud_off = bud_off;
  a.out_off = soft ? soft->cap_off : bud_off;
  a.bsh = soft ? reinterpret_cast<int32_t*>(wsb + G.off_bsh) : nullptr;
  a.S = G.S;
  a.Hkv = G.Hkv;
  a.T = G.T;
  a.nchunk = G.nchunk;
  a.totalB = soft ? soft->total_cap : G.total_B;
  a.rcache = reinterpret_cast<RCache*>(wsb + G.off_rcache);
  const dim3 grid(G.nchunk, G.Hkv, G.S);
  // histograms start at zero; cleared by a kernel, so that a captured graph
  // holds no memset node
  const int nzero = static_cast<int>((G.zero_end - G.off_hist) / sizeof(int));
  const bool topk = G.mode == KVE_TOPK;
  // sampling with a per-head budget and the unmixed proposal: the first
  // pass also writes the Gumbel keys and clears the histograms
  const bool chain = !topk && !soft && mix >= 1.0f;
  // with pooling folded in: top-k over several chunks or the unmixed chain
  // only, the counters already clear
  if (pool && (soft || (topk && G.max_len <= SEL_CHUNK) || (!topk && !chain))) return hipErrorInvalidValue;
  // the gather rides on the listed ordered write: no soft budget, no
  // single-chunk top-k
  if (compact && (soft || (topk && G.max_len <= SEL_CHUNK))) return hipErrorInvalidValue;
  stage_begin(ST_SELECT, st);
  if (topk && !soft && G.max_len <= SEL_CHUNK) {   // every head in one workgroup
    hipLaunchKernelGGL(sel_topk_one, dim3(1, G.Hkv, G.S), dim3(SEL_THREADS), 0, st, scores, a, idx, bias, m_out,
                       status_out);
    stage_end(ST_SELECT, st);
    return hipGetLastError();
  }
  if (!chain && !pool)
    hipLaunchKernelGGL(sel_init, dim3((max(nzero, SH) + 255) / 256), dim3(256), 0, st, hist, nzero,
                       topk ? m_out : nullptr, topk ? status_out : nullptr, topk ? SH : 0);
  if (topk) {
    launch_radix(G, a, ScoreKeys{pool ? pool->out : scores}, ZeroBias{}, hist, cnt, rs, idx, bias, st,
                 reinterpret_cast<int*>(wsb + G.off_cand), pool, compact);
  } else {
    SmpArgs A;
    A.g = a;
    A.scores = scores;
    A.lp = reinterpret_cast<double*>(wsb + G.off_a);
    A.L = reinterpret_cast<double*>(wsb + G.off_b);
    A.nsmp = G.nsmp;
    A.part = reinterpret_cast<double*>(wsb + G.off_part);
    A.grid = reinterpret_cast<float*>(wsb + G.off_grid);
    A.state = reinterpret_cast<Search*>(wsb + G.off_state);
    A.mvals = reinterpret_cast<double*>(wsb + G.off_mvals);
    A.inv_tau = 1.0 / static_cast<double>(tau);
    A.mix = static_cast<double>(mix);
    A.seed = seed;
    A.global = soft ? 1 : 0;
    A.bsh = soft ? reinterpret_cast<int32_t*>(wsb + G.off_bsh) : nullptr;
    A.kept_out = soft ? soft->kept : nullptr;
    const dim3 sgrid(G.nsmp, G.Hkv, G.S);
    const SnisBias bias_of{A.L, A.mvals, 1.0 / static_cast<double>(tau_w)};
    int* cand = reinterpret_cast<int*>(wsb + G.off_cand);
    // the search launches carry the keys' histogram levels
    static_assert(kSelSearchSteps == 3 && Radix<uint64_t>::LEVELS == 6 && kSmpChunk == kSelChunk,
                  "the fused launches pair 3 search steps, the finish and the decision with the 6 levels");
    if (chain) {
      // keys first: levels 0 .. 5 ride on the grid pass, the 3 search steps,
      // the finish and the decision
      if (pool) {
        A.scores = pool->out;
        hipLaunchKernelGGL((smp_logp<true, true>), sgrid, dim3(SEL_THREADS), 0, st, A, hist, nzero, *pool);
      } else {
        hipLaunchKernelGGL((smp_logp<true>), sgrid, dim3(SEL_THREADS), 0, st, A, hist, nzero, PoolSrc{});
      }
      hipLaunchKernelGGL(smp_grid_hist, sgrid, dim3(SEL_THREADS), 0, st, A, hist);
      hipLaunchKernelGGL((smp_search_hist<1, true>), sgrid, dim3(SEL_THREADS), 0, st, A, 0, hist);
      hipLaunchKernelGGL((smp_search_hist<2, false>), sgrid, dim3(SEL_THREADS), 0, st, A, 1, hist);
      hipLaunchKernelGGL((smp_search_hist<3, false>), sgrid, dim3(SEL_THREADS), 0, st, A, 2, hist);
      hipLaunchKernelGGL((smp_finish_hist<4>), sgrid, dim3(SEL_THREADS), 0, st, A, kSelSearchSteps, hist);
      hipLaunchKernelGGL(smp_decide_last, sgrid, dim3(SEL_THREADS), 0, st, A, kSelSearchSteps, m_out, status_out,
                         hist, cand, cnt);
      if (compact)
        hipLaunchKernelGGL((sel_write_listed<GumbelKeys, SnisBias, true>), sgrid, dim3(SEL_THREADS), 0, st,
                           GumbelKeys{A.lp}, bias_of, a, hist, cnt, cand, idx, bias, *compact);
      else
        hipLaunchKernelGGL((sel_write_listed<GumbelKeys, SnisBias, false>), sgrid, dim3(SEL_THREADS), 0, st,
                           GumbelKeys{A.lp}, bias_of, a, hist, cnt, cand, idx, bias, CompactDst{});
      stage_end(ST_SELECT, st);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((smp_logp<false>), sgrid, dim3(SEL_THREADS), 0, st, A, nullptr, 0, PoolSrc{});
    hipLaunchKernelGGL(smp_keys, sgrid, dim3(SEL_THREADS), 0, st, A);
    if (!soft) {
      // (mixed proposal) the keys need the normaliser: levels 0 .. 4 ride
      // on the search steps, the finish and the decision
      hipLaunchKernelGGL((smp_search_hist<0, true>), sgrid, dim3(SEL_THREADS), 0, st, A, 0, hist);
      hipLaunchKernelGGL((smp_search_hist<1, false>), sgrid, dim3(SEL_THREADS), 0, st, A, 1, hist);
      hipLaunchKernelGGL((smp_search_hist<2, false>), sgrid, dim3(SEL_THREADS), 0, st, A, 2, hist);
      hipLaunchKernelGGL((smp_finish_hist<3>), sgrid, dim3(SEL_THREADS), 0, st, A, kSelSearchSteps, hist);
      hipLaunchKernelGGL((smp_decide_hist<4>), sgrid, dim3(SEL_THREADS), 0, st, A, kSelSearchSteps, m_out,
                         status_out, hist);
      const dim3 grid(G.nchunk, G.Hkv, G.S);
      hipLaunchKernelGGL((sel_hist_last<GumbelKeys>), grid, dim3(SEL_THREADS), 0, st, GumbelKeys{A.lp}, a, hist,
                         cand, cnt);
      if (compact)
        hipLaunchKernelGGL((sel_write_listed<GumbelKeys, SnisBias, true>), grid, dim3(SEL_THREADS), 0, st,
                           GumbelKeys{A.lp}, bias_of, a, hist, cnt, cand, idx, bias, *compact);
      else
        hipLaunchKernelGGL((sel_write_listed<GumbelKeys, SnisBias, false>), grid, dim3(SEL_THREADS), 0, st,
                           GumbelKeys{A.lp}, bias_of, a, hist, cnt, cand, idx, bias, CompactDst{});
    } else {
      // a soft budget decides each head's kept count first (its radix
      // levels need it)
      for (int it = 0; it < kSelSearchSteps; ++it)
        hipLaunchKernelGGL(smp_search, sgrid, dim3(SEL_THREADS), 0, st, A, it);
      hipLaunchKernelGGL(smp_finish, sgrid, dim3(SEL_THREADS), 0, st, A, kSelSearchSteps);
      hipLaunchKernelGGL(smp_decide, dim3(G.Hkv, G.S), dim3(SEL_THREADS), 0, st, A, kSelSearchSteps, m_out,
                         status_out);
      launch_radix(G, a, GumbelKeys{A.lp}, bias_of, hist, cnt, rs, idx, bias, st, cand);
    }
  }
  stage_end(ST_SELECT, st);
  return hipGetLastError();
}

}  // namespace kve
