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

__global__ __launch_bounds__(SEL_THREADS) void select_topk(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ seq_off,
                                                          const int32_t* __restrict__ bud_off, int T,
                                                          int64_t totalB, int Hkv, int32_t* __restrict__ idx,
                                                          float* __restrict__ bias,
                                                          double* __restrict__ m_out,
                                                          int32_t* __restrict__ status_out) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  if (threadIdx.x == 0) {
    if (m_out) m_out[s * Hkv + h] = 0.0;
    if (status_out) status_out[s * Hkv + h] = KVE_OK;
  }
  const int base = seq_off[s];
  const int n = seq_off[s + 1] - base;
  const int B = bud_off[s + 1] - bud_off[s];
  int32_t* out = idx + h * totalB + bud_off[s];
  float* bout = bias + h * totalB + bud_off[s];
  const float* sc = scores + static_cast<size_t>(h) * T + base;
  const int tid = threadIdx.x;
  if (B <= 0) return;
  if (B >= n) {
    for (int j = tid; j < n; j += SEL_THREADS) { out[j] = j; bout[j] = 0.f; }
    return;
  }
  __shared__ int hist[256];
  __shared__ int scan_lds[2 * SEL_WAVES];
  __shared__ int sh_digit, sh_above;

  uint32_t prefix = 0, mask = 0;
  int need = B;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += SEL_THREADS) {
      const uint32_t u = f32_order_key(sc[j]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) pick_digit(hist, need, &sh_digit, &sh_above);
    __syncthreads();
    prefix |= static_cast<uint32_t>(sh_digit) << shift;
    mask |= 255u << shift;
    need -= sh_above;
    __syncthreads();
  }
  const uint32_t thr = prefix;   // key of the B-th largest; `need` equal keys are taken
  int run_eq = 0, run_sel = 0;
  for (int j0 = 0; j0 < n; j0 += SEL_THREADS) {
    const int j = j0 + tid;
    uint32_t u = 0;
    if (j < n) u = f32_order_key(sc[j]);
    const bool gt = j < n && u > thr;
    const bool eq = j < n && u == thr;
    int pe, dummy, te, td;
    block_scan2(eq, false, &pe, &dummy, &te, &td, scan_lds);
    const bool take = gt || (eq && run_eq + pe < need);
    int ps, tsel;
    block_scan2(take, false, &ps, &dummy, &tsel, &td, scan_lds);
    if (take && run_sel + ps < B) {   // bounded even if the threshold logic were off
      out[run_sel + ps] = j;
      bout[run_sel + ps] = 0.f;
    }
    run_eq += te;
    run_sel += tsel;
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
    stage_begin(ST_SELECT, st);
    hipLaunchKernelGGL(select_topk, grid, dim3(SEL_THREADS), 0, st, scores, seq_off, bud_off, G.T,
                       G.total_B, G.Hkv, idx, bias, m_out, status_out);
    stage_end(ST_SELECT, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipSuccess;
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
