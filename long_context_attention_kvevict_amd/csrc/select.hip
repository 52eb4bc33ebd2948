// Budgeted per-head selection.
//
// Top-k ("DropKV" page, §3.3: evict the smallest scores, keep the B largest;
// "A Probabilistic Interpretation of KV Cache Eviction", §4: top-k as a
// zero-variance estimator).  Radix select over the order-preserving uint32
// image of the fp32 scores (four 8-bit digit passes, most significant first)
// finds the B-th largest key; an ordered stream compaction (wave ballot +
// mbcnt prefix + per-wave totals in LDS) then writes the kept indices in
// ascending order: every key above the threshold plus the lowest-indexed
// keys equal to it.
//
// Sampling ("A Probabilistic Interpretation ...", §4 proposals, App. D.1
// temperature, App. F Problem 5 / Algorithm 2, §6 Eq. 10): fp64 proposal,
// expected-samples search for m (Newton iterations on the concave
// E[J(m)] = sum 1 - (1-pi)^m, then an integer check of the +-0.5 band),
// Gumbel keys from Philox-4x64-10, radix select on the fp64 keys, bias
// -log(q_j)/tau_w with q_j = 1 - (1-pi_j)^m.
//
// One workgroup of 1024 threads per (sequence, KV head).
#include "common.h"
#include "launch.h"
#include "timing.h"

namespace kve {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;

// Block-wide exclusive prefix of two predicates at once.  Returns the prefix
// of each and writes the block totals.  Contains two barriers.
__device__ __forceinline__ void block_scan2(bool p0, bool p1, int* pre0, int* pre1, int* tot0, int* tot1,
                                            int* lds /* [2][SEL_WAVES] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t b0 = __ballot(p0), b1 = __ballot(p1);
  const int in0 = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b0 >> 32),
                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b0), 0));
  const int in1 = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b1 >> 32),
                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b1), 0));
  if (lane == 0) {
    lds[wave] = __popcll(b0);
    lds[SEL_WAVES + wave] = __popcll(b1);
  }
  __syncthreads();
  int o0 = 0, o1 = 0, t0 = 0, t1 = 0;
  for (int wv = 0; wv < SEL_WAVES; ++wv) {
    const int c0 = lds[wv], c1 = lds[SEL_WAVES + wv];
    if (wv < wave) { o0 += c0; o1 += c1; }
    t0 += c0;
    t1 += c1;
  }
  __syncthreads();
  *pre0 = o0 + in0;
  *pre1 = o1 + in1;
  *tot0 = t0;
  *tot1 = t1;
}

// Finds the digit d (scanning from 255 down) where the running count of
// candidates with a larger digit first reaches `need`; returns d and the
// count strictly above it.  hist has 256 entries; executed by thread 0.
__device__ __forceinline__ void pick_digit(const int* hist, int need, int* digit, int* above) {
  int cum = 0;
  for (int dg = 255; dg >= 0; --dg) {
    const int c = hist[dg];
    if (cum + c >= need) {
      *digit = dg;
      *above = cum;
      return;
    }
    cum += c;
  }
  *digit = 0;
  *above = cum;
}

// ------------------------------------------------------------------ top-k
// Multi-workgroup radix select.  Every (sequence, KV head) is cut into chunks
// of TK_CHUNK keys, one workgroup each.  Three histogram launches resolve the
// B-th largest key digit by digit (bits 31..21, 20..10, 9..0); a count launch
// tallies keys above / equal to that threshold per chunk; the write launch
// places each chunk's kept indices after those of all earlier chunks, so the
// output is ascending.  Integer atomics only: the result is deterministic.
constexpr int TK_THREADS = 256;
constexpr int TK_PER = 16;
constexpr int TK_CHUNK = TK_THREADS * TK_PER;
constexpr int TK_BINS = 2048;
constexpr int TK_LEVELS = 3;
static_assert(TK_CHUNK == kSelChunk && TK_BINS == kSelBins && TK_LEVELS == kSelLevels32,
              "host and device select geometry disagree");

__device__ __forceinline__ int tk_shift(int lv) { return lv == 0 ? 21 : (lv == 1 ? 10 : 0); }

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

// Scans a TK_BINS histogram from the top bin down; returns the bin at which
// the running count first reaches `need` and the count strictly above it.
// Thread t owns bins 2047-8t .. 2040-8t.  lds: 6 ints.
__device__ void tk_pick(const int* __restrict__ gh, int need, int* lds, int* digit, int* above) {
  const int t = threadIdx.x;
  int c[8];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[i] = gh[TK_BINS - 1 - 8 * t - i];
    sum += c[i];
  }
  if (t == 0) { lds[4] = 0; lds[5] = 0; }
  int total;
  const int incl = block_incl_scan256(sum, lds, &total);   // barriers order the init above
  const int excl = incl - sum;
  if (excl < need && need <= incl) {
    int cum = excl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (cum + c[i] >= need) {
        lds[4] = TK_BINS - 1 - 8 * t - i;
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

// Resolves levels 0 .. nlv-1: key prefix, its mask and the count still
// needed among keys carrying that prefix.
__device__ void tk_resolve(const int* __restrict__ hist, int SH, int sh, int nlv, int B, int* lds,
                           uint32_t* prefix, uint32_t* mask, int* need) {
  uint32_t p = 0, m = 0;
  int nd = B;
  for (int lv = 0; lv < nlv; ++lv) {
    int dg, ab;
    tk_pick(hist + (static_cast<size_t>(lv) * SH + sh) * TK_BINS, nd, lds, &dg, &ab);
    const int sft = tk_shift(lv);
    const uint32_t width_mask = (lv == 2) ? 0x3ffu : 0x7ffu;
    p |= static_cast<uint32_t>(dg) << sft;
    m |= width_mask << sft;
    nd -= ab;
  }
  *prefix = p;
  *mask = m;
  *need = nd;
}

__global__ __launch_bounds__(256) void topk_zero(int* __restrict__ hist, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) hist[i] = 0;
}

template <int LV>
__global__ __launch_bounds__(TK_THREADS) void topk_hist(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ seq_off,
                                                        const int32_t* __restrict__ bud_off, int T, int Hkv,
                                                        int SH, int* __restrict__ hist) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = seq_off[s];
  const int n = seq_off[s + 1] - base;
  const int B = bud_off[s + 1] - bud_off[s];
  const int j0 = ch * TK_CHUNK;
  if (B <= 0 || B >= n || j0 >= n) return;
  const int sh = s * Hkv + h;
  __shared__ int lh[TK_BINS];
  __shared__ int lds[8];
  for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) lh[i] = 0;
  uint32_t prefix = 0, mask = 0;
  int need = B;
  if (LV > 0) tk_resolve(hist, SH, sh, LV, B, lds, &prefix, &mask, &need);
  __syncthreads();
  const float* sc = scores + static_cast<size_t>(h) * T + base;
  const int sft = tk_shift(LV);
  const uint32_t dmask = (LV == 2) ? 0x3ffu : 0x7ffu;
#pragma unroll 4
  for (int i = 0; i < TK_PER; ++i) {
    const int j = j0 + i * TK_THREADS + threadIdx.x;
    if (j < n) {
      const uint32_t u = f32_order_key(sc[j]);
      if ((u & mask) == prefix) atomicAdd(&lh[(u >> sft) & dmask], 1);
    }
  }
  __syncthreads();
  int* gh = hist + (static_cast<size_t>(LV) * SH + sh) * TK_BINS;
  for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) {
    const int c = lh[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Per chunk: keys above the threshold and keys equal to it.  Chunk 0 also
// stores the threshold and the number of equal keys to keep.
__global__ __launch_bounds__(TK_THREADS) void topk_count(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ seq_off,
                                                         const int32_t* __restrict__ bud_off, int T, int Hkv,
                                                         int SH, int nchunk, const int* __restrict__ hist,
                                                         int* __restrict__ cnt, uint32_t* __restrict__ state) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = seq_off[s];
  const int n = seq_off[s + 1] - base;
  const int B = bud_off[s + 1] - bud_off[s];
  const int j0 = ch * TK_CHUNK;
  if (B <= 0 || B >= n || j0 >= n) return;
  const int sh = s * Hkv + h;
  __shared__ int lds[8];
  uint32_t thr, mask;
  int need;
  tk_resolve(hist, SH, sh, TK_LEVELS, B, lds, &thr, &mask, &need);
  const float* sc = scores + static_cast<size_t>(h) * T + base;
  int gt = 0, eq = 0;
#pragma unroll 4
  for (int i = 0; i < TK_PER; ++i) {
    const int j = j0 + i * TK_THREADS + threadIdx.x;
    if (j < n) {
      const uint32_t u = f32_order_key(sc[j]);
      gt += (u > thr);
      eq += (u == thr);
    }
  }
  const int packed = (gt << 16) | eq;   // each count <= TK_CHUNK < 2^16
  int tot;
  block_incl_scan256(packed, lds, &tot);
  if (threadIdx.x == 0) {
    cnt[(static_cast<size_t>(sh) * nchunk + ch) * 2 + 0] = tot >> 16;
    cnt[(static_cast<size_t>(sh) * nchunk + ch) * 2 + 1] = tot & 0xffff;
    if (ch == 0) {
      state[sh * 2 + 0] = thr;
      state[sh * 2 + 1] = static_cast<uint32_t>(need);
    }
  }
}

// Ordered write: thread t owns keys j0 + 16t .. j0 + 16t + 15.
__global__ __launch_bounds__(TK_THREADS) void topk_write(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ seq_off,
                                                         const int32_t* __restrict__ bud_off, int T, int Hkv,
                                                         int64_t totalB, int nchunk, const int* __restrict__ cnt,
                                                         const uint32_t* __restrict__ state,
                                                         int32_t* __restrict__ idx, float* __restrict__ bias,
                                                         double* __restrict__ m_out,
                                                         int32_t* __restrict__ status_out) {
  const int ch = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int base = seq_off[s];
  const int n = seq_off[s + 1] - base;
  const int B = bud_off[s + 1] - bud_off[s];
  const int j0 = ch * TK_CHUNK;
  const int sh = s * Hkv + h;
  if (ch == 0 && threadIdx.x == 0) {
    if (m_out) m_out[sh] = 0.0;
    if (status_out) status_out[sh] = KVE_OK;
  }
  if (B <= 0 || j0 >= n) return;
  int32_t* out = idx + h * totalB + bud_off[s];
  float* bout = bias + h * totalB + bud_off[s];
  if (B >= n) {
    for (int i = threadIdx.x; i < TK_CHUNK; i += TK_THREADS) {
      const int j = j0 + i;
      if (j < n) { out[j] = j; bout[j] = 0.f; }
    }
    return;
  }
  __shared__ int lds[8];
  const uint32_t thr = state[sh * 2 + 0];
  const int need = static_cast<int>(state[sh * 2 + 1]);
  // keys above / equal to the threshold in earlier chunks
  int gt_b = 0, eq_b = 0;
  for (int c = threadIdx.x; c < ch; c += TK_THREADS) {
    gt_b += cnt[(static_cast<size_t>(sh) * nchunk + c) * 2 + 0];
    eq_b += cnt[(static_cast<size_t>(sh) * nchunk + c) * 2 + 1];
  }
  int tot;
  block_incl_scan256(gt_b, lds, &tot);
  gt_b = tot;
  block_incl_scan256(eq_b, lds, &tot);
  eq_b = tot;
  const float* sc = scores + static_cast<size_t>(h) * T + base;
  const int jt = j0 + TK_PER * threadIdx.x;
  uint32_t u[TK_PER];
  int neq = 0;
#pragma unroll
  for (int i = 0; i < TK_PER; ++i) {
    u[i] = (jt + i < n) ? f32_order_key(sc[jt + i]) : 0u;
    neq += (jt + i < n) && (u[i] == thr);
  }
  int eq_tot;
  int eq_rank = eq_b + block_incl_scan256(neq, lds, &eq_tot) - neq;
  int ntake = 0;
  uint32_t take_bits = 0;
#pragma unroll
  for (int i = 0; i < TK_PER; ++i) {
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
  for (int i = 0; i < TK_PER; ++i) {
    if ((take_bits >> i) & 1u) {
      if (pos < B) {   // bounded even if the counts were inconsistent
        out[pos] = jt + i;
        bout[pos] = 0.f;
      }
      ++pos;
    }
  }
}

// ------------------------------------------------------------------ sampling
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  *lo = a * b;
  *hi = __umul64hi(a, b);
}

// Philox-4x64 with 10 rounds (Salmon et al., SC'11); returns output word 0.
__device__ uint64_t philox4x64_10_w0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                     uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(M0, c0, &hi0, &lo0);
    mulhilo64(M1, c2, &hi1, &lo1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}

__device__ double block_sum_d(double v, double* lds /* [SEL_WAVES] */) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < SEL_WAVES; ++i) t += lds[i];
  __syncthreads();
  return t;
}

__device__ double block_max_d(double v, double* lds) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  double t = -INFINITY;
  for (int i = 0; i < SEL_WAVES; ++i) t = fmax(t, lds[i]);
  __syncthreads();
  return t;
}

// E[J(m)] - target and its derivative over the head's log1p(-pi) plane.
__device__ void eval_E(const double* L, int n, double m, double target, double* f, double* fp,
                       double* lds) {
  double e = 0.0, de = 0.0;
  for (int j = threadIdx.x; j < n; j += SEL_THREADS) {
    const double x = m * L[j];
    const double ex = exp(x);
    e += -expm1(x);
    de += -L[j] * ex;
  }
  const double se = block_sum_d(e, lds);
  const double sde = block_sum_d(de, lds);
  *f = se - target;
  *fp = sde;
}

__device__ double eval_E_only(const double* L, int n, double m, double* lds) {
  double e = 0.0;
  for (int j = threadIdx.x; j < n; j += SEL_THREADS) e += -expm1(m * L[j]);
  return block_sum_d(e, lds);
}

__global__ __launch_bounds__(SEL_THREADS) void select_sample(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ seq_off,
                                                            const int32_t* __restrict__ bud_off, int Hkv,
                                                            int T, int64_t totalB, double inv_tau,
                                                            double inv_tau_w, uint64_t seed,
                                                            double* __restrict__ planeA,
                                                            double* __restrict__ planeB,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ bias,
                                                            double* __restrict__ m_out,
                                                            int32_t* __restrict__ status_out) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int base = seq_off[s];
  const int n = seq_off[s + 1] - base;
  const int B = bud_off[s + 1] - bud_off[s];
  int32_t* out = idx + h * totalB + bud_off[s];
  float* bout = bias + h * totalB + bud_off[s];
  const float* sc = scores + static_cast<size_t>(h) * T + base;
  double* lp = planeA + static_cast<size_t>(h) * T + base;   // log proposal, then Gumbel keys
  double* L = planeB + static_cast<size_t>(h) * T + base;    // log1p(-pi)
  const int tid = threadIdx.x;
  __shared__ double dl[SEL_WAVES];
  __shared__ int hist[256];
  __shared__ int scan_lds[2 * SEL_WAVES];
  __shared__ int sh_digit, sh_above;

  if (B <= 0 || B >= n) {
    if (B >= n)
      for (int j = tid; j < n; j += SEL_THREADS) { out[j] = j; bout[j] = 0.f; }
    if (tid == 0) {
      if (m_out) m_out[s * Hkv + h] = 0.0;
      if (status_out) status_out[s * Hkv + h] = KVE_OK;
    }
    return;
  }
  // proposal: log pi~ = log(max(s, 2^-126)) / tau ; pi = softmax(log pi~)
  double mx = -INFINITY;
  for (int j = tid; j < n; j += SEL_THREADS) {
    const double x = log(static_cast<double>(fmaxf(sc[j], 1.17549435e-38f))) * inv_tau;
    lp[j] = x;
    mx = fmax(mx, x);
  }
  mx = block_max_d(mx, dl);
  double z = 0.0;
  for (int j = tid; j < n; j += SEL_THREADS) z += exp(lp[j] - mx);
  z = block_sum_d(z, dl);
  const double lse = mx + log(z);
  for (int j = tid; j < n; j += SEL_THREADS) L[j] = log1p(-exp(lp[j] - lse));
  __syncthreads();

  // expected-samples search
  const double target = static_cast<double>(B);
  const double ALPHA = 1e12;
  double m;
  int status = KVE_OK;
  double f, fp;
  eval_E(L, n, ALPHA, target, &f, &fp, dl);
  if (f < -0.5) {
    m = ALPHA;
    status = KVE_ENOCONV;
  } else {
    // Newton from the left on the concave increasing f: iterates increase
    // monotonically towards the root (E[J(m)] <= m, so m = B is left of it)
    m = target;
    for (int it = 0; it < 200; ++it) {
      eval_E(L, n, m, target, &f, &fp, dl);
      if (f >= -1e-3 || !(fp > 0.0)) break;
      const double step = -f / fp;
      m = fmin(m + step, ALPHA);
      if (step < 1e-9 * m) break;
    }
    // integer in the band |E - B| <= 0.5: bracket search around round(m)
    double lo = fmax(0.0, floor(m) - 2.0), hi = fmin(ALPHA, ceil(m) + 2.0);
    for (int grow = 0; grow < 64; ++grow) {
      const double elo = eval_E_only(L, n, lo, dl) - target;
      const double ehi = eval_E_only(L, n, hi, dl) - target;
      if (elo <= 0.5 && ehi >= -0.5) break;
      const double wdt = hi - lo + 1.0;
      if (elo > 0.5) lo = fmax(0.0, lo - wdt);
      if (ehi < -0.5) hi = fmin(ALPHA, hi + wdt);
    }
    // integer binary search (the steps of Algorithm 2) inside [lo, hi]
    m = -1.0;
    for (int it = 0; it < 128 && lo <= hi; ++it) {
      const double mid = floor((lo + hi) * 0.5);
      const double e = eval_E_only(L, n, mid, dl) - target;
      if (fabs(e) <= 0.5) { m = mid; break; }
      if (e < 0.0) lo = mid + 1.0; else hi = mid - 1.0;
    }
    if (m < 0.0) { m = ALPHA; status = KVE_ENOCONV; }
  }
  if (tid == 0) {
    if (m_out) m_out[s * Hkv + h] = m;
    if (status_out) status_out[s * Hkv + h] = status;
  }

  // Gumbel keys kappa = log pi~ - log(-log u), stored over the log-proposal
  for (int j = tid; j < n; j += SEL_THREADS) {
    const uint64_t x = philox4x64_10_w0(static_cast<uint64_t>(j), static_cast<uint64_t>(h),
                                        static_cast<uint64_t>(s), 0ull, seed, 0ull);
    const double u = (static_cast<double>(x >> 11) + 0.5) * 0x1.0p-53;
    lp[j] = lp[j] - log(-log(u));
  }
  __syncthreads();

  // radix select of the B-th largest 64-bit key
  uint64_t prefix = 0, mask = 0;
  int need = B;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += SEL_THREADS) {
      const uint64_t u = f64_order_key(lp[j]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255ull], 1);
    }
    __syncthreads();
    if (tid == 0) pick_digit(hist, need, &sh_digit, &sh_above);
    __syncthreads();
    prefix |= static_cast<uint64_t>(sh_digit) << shift;
    mask |= 255ull << shift;
    need -= sh_above;
    __syncthreads();
  }
  const uint64_t thr = prefix;
  int run_eq = 0, run_sel = 0;
  for (int j0 = 0; j0 < n; j0 += SEL_THREADS) {
    const int j = j0 + tid;
    uint64_t u = 0;
    if (j < n) u = f64_order_key(lp[j]);
    const bool gt = j < n && u > thr;
    const bool eq = j < n && u == thr;
    int pe, dummy, te, td;
    block_scan2(eq, false, &pe, &dummy, &te, &td, scan_lds);
    const bool take = gt || (eq && run_eq + pe < need);
    int ps, tsel;
    block_scan2(take, false, &ps, &dummy, &tsel, &td, scan_lds);
    if (take && run_sel + ps < B) {   // bounded even if the threshold logic were off
      const double q = -expm1(m * L[j]);
      out[run_sel + ps] = j;
      bout[run_sel + ps] = static_cast<float>(-log(q) * inv_tau_w);
    }
    run_eq += te;
    run_sel += tsel;
  }
}

hipError_t launch_select(const SelectGeom& G, const float* scores, const int32_t* seq_off,
                         const int32_t* bud_off, float tau, float tau_w, uint64_t seed, int32_t* idx,
                         float* bias, double* m_out, int32_t* status_out, void* ws, hipStream_t st) {
  dim3 grid(G.Hkv, G.S);
  if (G.mode == KVE_TOPK) {
    char* wsb = static_cast<char*>(ws);
    int* hist = reinterpret_cast<int*>(wsb + G.off_hist);
    int* cnt = reinterpret_cast<int*>(wsb + G.off_cnt);
    uint32_t* state = reinterpret_cast<uint32_t*>(wsb + G.off_state);
    const int SH = G.S * G.Hkv;
    const int nhist = TK_LEVELS * SH * TK_BINS;
    dim3 cgrid(G.nchunk, G.Hkv, G.S);
    stage_begin(ST_SELECT, st);
    hipLaunchKernelGGL(topk_zero, dim3((nhist + 255) / 256), dim3(256), 0, st, hist, nhist);
    hipLaunchKernelGGL(topk_hist<0>, cgrid, dim3(TK_THREADS), 0, st, scores, seq_off, bud_off, G.T, G.Hkv, SH, hist);
    hipLaunchKernelGGL(topk_hist<1>, cgrid, dim3(TK_THREADS), 0, st, scores, seq_off, bud_off, G.T, G.Hkv, SH, hist);
    hipLaunchKernelGGL(topk_hist<2>, cgrid, dim3(TK_THREADS), 0, st, scores, seq_off, bud_off, G.T, G.Hkv, SH, hist);
    hipLaunchKernelGGL(topk_count, cgrid, dim3(TK_THREADS), 0, st, scores, seq_off, bud_off, G.T, G.Hkv, SH,
                       G.nchunk, hist, cnt, state);
    hipLaunchKernelGGL(topk_write, cgrid, dim3(TK_THREADS), 0, st, scores, seq_off, bud_off, G.T, G.Hkv,
                       G.total_B, G.nchunk, cnt, state, idx, bias, m_out, status_out);
    stage_end(ST_SELECT, st);
    return hipGetLastError();
  }
  char* base = static_cast<char*>(ws);
  stage_begin(ST_SELECT, st);
  hipLaunchKernelGGL(select_sample, grid, dim3(SEL_THREADS), 0, st, scores, seq_off, bud_off, G.Hkv, G.T,
                     G.total_B, 1.0 / static_cast<double>(tau), 1.0 / static_cast<double>(tau_w), seed,
                     reinterpret_cast<double*>(base + G.off_a), reinterpret_cast<double*>(base + G.off_b),
                     idx, bias, m_out, status_out);
  stage_end(ST_SELECT, st);
  return hipGetLastError();
}

}  // namespace kve
