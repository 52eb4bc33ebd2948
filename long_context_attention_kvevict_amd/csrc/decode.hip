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

#include <mutex>
#include <type_traits>

namespace kve {

// Device scratch of the allocation-free decode entry point: the split
// partials live here instead of in a caller workspace.  Every GPU the
// library runs on holds its own copy for the life of the process; calls on
// one GPU share it.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  // The array's name is a host-side stand-in; its device address is looked
  // up once per device, with that device current, and kept.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }

// The step's own token, appended by the decode itself (kvevict_decode_snis_append):
// the split kernels attend to it from k_new / v_new (bias 0) at slot
// cache_len[s], and the merge kernel, which runs after every split has read
// the cache, stores it there and advances cache_len[s].  All NULL for the
// plain decode.
struct DecAppend {
  const void* k_new;    // [Hkv][S][d]
  const void* v_new;
  void* k_c;            // the cache, written at the appended slot
  void* v_c;
  float* bias_c;
  int32_t* cache_len;   // advanced by one where the token was stored
  int32_t* app;         // [S][2] workspace: entries attended, appended slot or -1
};

// Entries the split kernels attend to for sequence s, and the slot of the
// appended token (-1: none).  Never past the sequence's capacity, whatever
// cache_len holds; a full cache attends to its entries only.
__device__ __forceinline__ int dec_len(const int32_t* cache_len, const int32_t* cap_off, int s, bool append,
                                       int* app) {
  const int cap = cap_off[s + 1] - cap_off[s];
  const int c = cache_len[s];
  if (append && c >= 0 && c < cap) {
    *app = c;
    return c + 1;
  }
  *app = -1;
  return min(c, cap);
}

template <typename T, int DD, int GMAX>
__global__ __launch_bounds__(256) void decode_split(const T* __restrict__ q, const T* __restrict__ k_c,
                                                    const T* __restrict__ v_c, const float* __restrict__ bias_c,
                                                    const int32_t* __restrict__ cap_off,
                                                    const int32_t* __restrict__ cache_len, int Hq, int Hkv,
                                                    int64_t totalC, int split_len, int splits, float c2,
                                                    float* __restrict__ part_ml, float* __restrict__ part_o,
                                                    DecAppend ap) {
  constexpr int CPL = DD / 16;   // features per lane
  const int sp = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int g = Hq / Hkv;
  int app;
  const int len = dec_len(cache_len, cap_off, s, ap.k_new != nullptr, &app);
  if (ap.k_new && sp == 0 && h == 0 && threadIdx.x == 0) {
    ap.app[2 * s] = len;
    ap.app[2 * s + 1] = app;
  }
  const T* knew = ap.k_new ? static_cast<const T*>(ap.k_new) + (static_cast<size_t>(h) * gridDim.z + s) * DD : nullptr;
  const T* vnew = ap.k_new ? static_cast<const T*>(ap.v_new) + (static_cast<size_t>(h) * gridDim.z + s) * DD : nullptr;
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
    const bool isnew = e == app;   // the step's token: from k_new / v_new, bias 0
    const T* kp = isnew ? knew : k_c + (rowbase + e) * DD;
    const T* vp = isnew ? vnew : v_c + (rowbase + e) * DD;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      kr[c] = ld_elem<T>(kp + fl * CPL + c);
      vr[c] = ld_elem<T>(vp + fl * CPL + c);
    }
    const float bv = bias_c[rowbase + e];   // within the capacity in every case
    const float bl2 = isnew ? 0.f : bv * kLog2e;
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

// bf16 caches: both contractions on the matrix cores.  Workgroup = 256
// consecutive entries of one (sequence, KV head), 4 waves of two 32-entry
// blocks each.  Per block a wave forms the logits S = K . Q^T with
// 16x16x32 MFMAs (entries as M, the group's q-heads as N, padded to 16),
// updates an online softmax per q-head and accumulates O += P . V with P
// split into bf16 hi + lo parts (so the weights keep ~16 mantissa bits) and
// V read back transposed from LDS.  K and bias go straight to registers;
// all loads of the wave's two blocks are issued before any compute.
//
// Lane roles (l = lane, ln = l % 16, lq = l / 16):
//   K operand   entry 16*mb + ln of the block, 16-byte chunk 4*j + lq
//   Q operand   q-head ln of the group (zero past g), same chunk
//   logits      entries 16*mb + 4*lq + r (r < 4) of q-head ln
//   P operand   the same 8 values, k-slot 8*lq + i <-> entry 4*lq + i (i < 4)
//               or 16 + 4*lq + i - 4 (i >= 4)
//   V operand   two transposing LDS reads: entries 4*lq..+3 and
//               16 + 4*lq..+3 at feature 16*dt + ln
//   O           q-head 4*lq + r, feature 16*dt + ln
constexpr int kDecBlk = 32;
constexpr int kDecWaveBlocks = 2;
static_assert(4 * kDecWaveBlocks * kDecBlk == kDecodeChunkBf16, "decode chunk geometry");

template <int DD>
__device__ __forceinline__ int dec_swz(int row) {
  return (row & (DD / 16 - 1)) << 1;   // keeps 16-byte chunk pairs together
}

template <int DD, bool APPEND>
__global__ __launch_bounds__(256, 2) void decode_split_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_c, const uint16_t* __restrict__ v_c,
    const float* __restrict__ bias_c, const int32_t* __restrict__ cap_off,
    const int32_t* __restrict__ cache_len, int Hq, int Hkv, int64_t totalC, int splits, float c2,
    float* __restrict__ part_ml, float* __restrict__ part_o, DecAppend ap) {
  constexpr int KS = DD / 32;             // k-steps of S = K . Q^T
  constexpr int DT = DD / 16;             // 16-feature tiles of O
  constexpr int ROWB = DD * 2;            // bytes per cache row
  constexpr int CPR = DD / 8;             // 16-byte chunks per row
  constexpr int VPL = kDecBlk * CPR / 64; // 16-byte V pieces per lane per block
  constexpr int WAVE_LDS = kDecBlk * ROWB;
  __shared__ __align__(16) char lds[4 * WAVE_LDS + 512];

  const int sp = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int g = Hq / Hkv;
  int app;
  const int len = dec_len(cache_len, cap_off, s, APPEND, &app);
  if (APPEND && sp == 0 && h == 0 && threadIdx.x == 0) {
    ap.app[2 * s] = len;
    ap.app[2 * s + 1] = app;
  }
  const char* knew =
      APPEND ? static_cast<const char*>(ap.k_new) + (static_cast<size_t>(h) * gridDim.z + s) * (DD * 2) : nullptr;
  const char* vnew =
      APPEND ? static_cast<const char*>(ap.v_new) + (static_cast<size_t>(h) * gridDim.z + s) * (DD * 2) : nullptr;
  const int e0 = sp * kDecodeChunkBf16;
  if (e0 >= len) return;                  // uniform over the workgroup
  const int e1 = min(e0 + kDecodeChunkBf16, len);
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, ln = l & 15, lq = l >> 4;
  const size_t rowbase = static_cast<size_t>(h) * totalC + cap_off[s];
  const char* kbase = reinterpret_cast<const char*>(k_c + rowbase * DD);
  const char* vbase = reinterpret_cast<const char*>(v_c + rowbase * DD);
  const float* bbase = bias_c + rowbase;
  const int we0 = e0 + wave * kDecWaveBlocks * kDecBlk;
  const int last = e1 - 1;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (we0 < e1) {                         // uniform over the wave
    bf16x8 qop[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (ln < g)
        z = *reinterpret_cast<const u32x4*>(q + (static_cast<size_t>(s) * Hq + h * g + ln) * DD + (4 * j + lq) * 8);
      qop[j] = as_bf16x8(z);
    }
    u32x4 kr[kDecWaveBlocks][2][KS], vr[kDecWaveBlocks][VPL];
    float bi[kDecWaveBlocks][2][4];
#pragma unroll
    for (int b = 0; b < kDecWaveBlocks; ++b) {
      const int eb = we0 + b * kDecBlk;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int er = min(eb + 16 * mb + ln, last);
        const char* kp = kbase + static_cast<size_t>(er) * ROWB;
        if constexpr (APPEND) kp = (er == app) ? knew : kp;   // the step's token
#pragma unroll
        for (int j = 0; j < KS; ++j) kr[b][mb][j] = *reinterpret_cast<const u32x4*>(kp + (4 * j + lq) * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int eb2 = min(eb + 16 * mb + 4 * lq + r, last);
          // loaded in every case (the slot lies within the capacity), so
          // that the selection below compiles to a select, not a branch
          const float bv = bbase[eb2];
          bi[b][mb][r] = (APPEND && eb2 == app) ? 0.f : bv;
        }
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int pc = i * 64 + l, ent = pc / CPR, ch = pc % CPR;
        const int er = min(eb + ent, last);
        const char* vp = vbase + static_cast<size_t>(er) * ROWB;
        if constexpr (APPEND) vp = (er == app) ? vnew : vp;
        vr[b][i] = *reinterpret_cast<const u32x4*>(vp + ch * 16);
      }
    }
    // keep every load of both blocks ahead of the compute
    __builtin_amdgcn_sched_barrier(0);
    char* vl = lds + wave * WAVE_LDS;
#pragma unroll
    for (int b = 0; b < kDecWaveBlocks; ++b) {
      const int eb = we0 + b * kDecBlk;
      f32x4 sacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j) sacc[mb] = mfma16(as_bf16x8(kr[b][mb][j]), qop[j], sacc[mb]);
      }
      // this block's V into the wave's LDS rows (the previous block's
      // transposing reads were issued earlier by this wave, LDS keeps order)
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int pc = i * 64 + l, ent = pc / CPR, ch = pc % CPR;
        *reinterpret_cast<u32x4*>(vl + ent * ROWB + ((ch ^ dec_swz<DD>(ent)) << 4)) = vr[b][i];
      }
      float x[2][4];
      float mloc = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xv = fmaf(sacc[mb][r], c2, bi[b][mb][r] * kLog2e);
          x[mb][r] = (eb + 16 * mb + 4 * lq + r < e1) ? xv : -INFINITY;
          mloc = fmaxf(mloc, x[mb][r]);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      // Raise the reference only when the block max exceeds it by 2^8, so
      // weights stay below 256 and O is rarely rescaled.
      if (__ballot(mloc > m_run + 8.f)) {
        const float mn = fmaxf(m_run, mloc);
        const float a = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= a;
        m_run = mn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(a, 4 * lq + r, 64);   // lane 4*lq + r holds q-head 4*lq + r
#pragma unroll
          for (int t = 0; t < DT; ++t) oacc[t][r] *= ar;
        }
      }
      const float mu = (m_run == -INFINITY) ? 0.f : m_run;
      bf16x8 phi, plo;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pf = __builtin_amdgcn_exp2f(x[mb][r] - mu);
          l_run += pf;
          const __bf16 hb = static_cast<__bf16>(pf);
          phi[4 * mb + r] = hb;
          plo[4 * mb + r] = static_cast<__bf16>(pf - static_cast<float>(hb));
        }
      }
      typedef short s16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int chp = 2 * t + ((ln >> 1) & 1);
        const int r0 = 4 * lq + (ln >> 2), r1 = 16 + 4 * lq + (ln >> 2);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vl + r0 * ROWB + ((chp ^ dec_swz<DD>(r0)) << 4) + 8 * (ln & 1)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vl + r1 * ROWB + ((chp ^ dec_swz<DD>(r1)) << 4) + 8 * (ln & 1)));
        const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[t] = mfma16(phi, vop, oacc[t]);
        oacc[t] = mfma16(plo, vop, oacc[t]);
      }
    }
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // merge the 4 waves through LDS
  __syncthreads();
  float* sm = reinterpret_cast<float*>(lds);          // [4][16]
  float* sl = sm + 64;                                // [4][16]
  float* so = sl + 64;                                // [4][g][DD]
  if (lq == 0 && ln < g) {
    sm[wave * 16 + ln] = m_run;
    sl[wave * 16 + ln] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * lq + r;
    if (row < g) {
#pragma unroll
      for (int t = 0; t < DT; ++t) so[(wave * g + row) * DD + 16 * t + ln] = oacc[t][r];
    }
  }
  __syncthreads();
  for (int t = tid; t < g * DD; t += 256) {
    const int i = t / DD, dcol = t % DD;
    float M = -INFINITY;
    for (int u = 0; u < 4; ++u) M = fmaxf(M, sm[u * 16 + i]);
    float L = 0.f, O = 0.f;
    for (int u = 0; u < 4; ++u) {
      const float f = (sm[u * 16 + i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm[u * 16 + i] - M);
      L += sl[u * 16 + i] * f;
      O += so[(u * g + i) * DD + dcol] * f;
    }
    const size_t row = (static_cast<size_t>(s) * Hq + h * g + i) * splits + sp;
    part_o[row * DD + dcol] = O;
    if (dcol == 0) {
      part_ml[row * 2] = M;
      part_ml[row * 2 + 1] = L;
    }
  }
}

// Merge of the split partials of one (sequence, q-head) row.  Each thread
// owns one feature; the partial outputs of up to PR splits per round are
// loaded together with the split maxima and sums (staged in LDS), so a
// round costs one memory round trip.
template <typename T, int DD>
__global__ __launch_bounds__(DD) void decode_merge(const float* __restrict__ part_ml, const float* __restrict__ part_o,
                                                   const int32_t* __restrict__ cache_len,
                                                   const int32_t* __restrict__ cap_off, int S, int Hq, int Hkv,
                                                   int64_t totalC, int splits, int split_len,
                                                   float* __restrict__ out, DecAppend ap) {
  constexpr int PR = 32;             // splits per round
  __shared__ float sml[PR][2];
  const int r = blockIdx.x;          // s * Hq + qh
  const int s = r / Hq;
  const int d = threadIdx.x;
  int len;
  if (ap.k_new) {   // the lengths the splits used (cache_len is advanced below)
    len = ap.app[2 * s];
    const int app = ap.app[2 * s + 1];
    const int qh = r % Hq, g = Hq / Hkv;
    if (app >= 0 && qh % g == 0) {   // one workgroup per (sequence, KV head) stores the token
      const int h = qh / g;
      const size_t src = (static_cast<size_t>(h) * S + s) * DD + d;
      const size_t dst = (static_cast<size_t>(h) * totalC + cap_off[s] + app) * DD + d;
      static_cast<T*>(ap.k_c)[dst] = static_cast<const T*>(ap.k_new)[src];
      static_cast<T*>(ap.v_c)[dst] = static_cast<const T*>(ap.v_new)[src];
      if (d == 0) ap.bias_c[static_cast<size_t>(h) * totalC + cap_off[s] + app] = 0.f;
      if (qh == 0 && d == 0) ap.cache_len[s] = app + 1;
    }
  } else {
    len = min(cache_len[s], cap_off[s + 1] - cap_off[s]);
  }
  const int ns = max(0, min(splits, (len + split_len - 1) / split_len));
  const float* ml = part_ml + static_cast<size_t>(r) * splits * 2;
  const float* po = part_o + static_cast<size_t>(r) * splits * DD;
  // running merge over rounds (the reference M only grows)
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int p0 = 0; p0 < ns; p0 += PR) {
    const int cnt = min(PR, ns - p0);
    if (d < 2 * cnt) sml[d >> 1][d & 1] = ml[2 * p0 + d];
    float v[PR];
#pragma unroll
    for (int u = 0; u < PR; ++u) v[u] = (u < cnt) ? po[static_cast<size_t>(p0 + u) * DD + d] : 0.f;
    __syncthreads();
    float Mr = M;
    for (int u = 0; u < cnt; ++u) Mr = fmaxf(Mr, sml[u][0]);
    if (Mr != -INFINITY) {
      const float a = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mr);
      L *= a;
      O *= a;
#pragma unroll
      for (int u = 0; u < PR; ++u) {
        if (u < cnt) {
          const float mm = sml[u][0];
          const float f = (mm == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mm - Mr);
          L = fmaf(sml[u][1], f, L);
          O = fmaf(v[u], f, O);
        }
      }
      M = Mr;
    }
    __syncthreads();
  }
  out[static_cast<size_t>(r) * DD + d] = (L > 0.f) ? O / L : 0.f;   // empty cache -> 0
}

template <typename T, int DD>
static hipError_t launch_decode_t(const DecodeGeom& G, int64_t totalC, const void* q, const void* k_c,
                                  const void* v_c, const float* bias_c, const int32_t* cap_off,
                                  const int32_t* cache_len, float sm_scale, float* out, void* ws,
                                  hipStream_t st, DecAppend ap) {
  char* base = static_cast<char*>(ws);
  float* pml = reinterpret_cast<float*>(base + G.off_ml);
  float* po = reinterpret_cast<float*>(base + G.off_o);
  if (ap.k_new) ap.app = reinterpret_cast<int32_t*>(base + G.off_app);
  dim3 grid(G.splits, G.Hkv, G.S);
  const int g = G.Hq / G.Hkv;
  const float c2 = sm_scale * kLog2e;
  stage_begin(ST_DECODE_SPLIT, st);
  if constexpr (std::is_same<T, uint16_t>::value) {
    (void)g;
    if (ap.k_new)
      hipLaunchKernelGGL((decode_split_mfma<DD, true>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(q),
                         static_cast<const uint16_t*>(k_c), static_cast<const uint16_t*>(v_c), bias_c, cap_off,
                         cache_len, G.Hq, G.Hkv, totalC, G.splits, c2, pml, po, ap);
    else
      hipLaunchKernelGGL((decode_split_mfma<DD, false>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(q),
                         static_cast<const uint16_t*>(k_c), static_cast<const uint16_t*>(v_c), bias_c, cap_off,
                         cache_len, G.Hq, G.Hkv, totalC, G.splits, c2, pml, po, ap);
  } else {
  if (g <= 4)
    hipLaunchKernelGGL((decode_split<T, DD, 4>), grid, dim3(256), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k_c), static_cast<const T*>(v_c), bias_c, cap_off, cache_len,
                       G.Hq, G.Hkv, totalC, G.split_len, G.splits, c2, pml, po, ap);
  else if (g <= 8)
    hipLaunchKernelGGL((decode_split<T, DD, 8>), grid, dim3(256), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k_c), static_cast<const T*>(v_c), bias_c, cap_off, cache_len,
                       G.Hq, G.Hkv, totalC, G.split_len, G.splits, c2, pml, po, ap);
  else
    hipLaunchKernelGGL((decode_split<T, DD, 16>), grid, dim3(256), 0, st, static_cast<const T*>(q),
                       static_cast<const T*>(k_c), static_cast<const T*>(v_c), bias_c, cap_off, cache_len,
                       G.Hq, G.Hkv, totalC, G.split_len, G.splits, c2, pml, po, ap);
  }
  stage_end(ST_DECODE_SPLIT, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(ST_DECODE_MERGE, st);
  hipLaunchKernelGGL((decode_merge<T, DD>), dim3(G.S * G.Hq), dim3(DD), 0, st, pml, po, cache_len, cap_off, G.S,
                     G.Hq, G.Hkv, totalC, G.splits, G.split_len, out, ap);
  stage_end(ST_DECODE_MERGE, st);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeGeom& G, int64_t totalC, const void* q, const void* k_c,
                         const void* v_c, const float* bias_c, const int32_t* cap_off,
                         const int32_t* cache_len, float sm_scale, float* out, void* ws,
                         hipStream_t st, const DecodeAppendArgs* append) {
  DecAppend ap{};
  if (append) {
    ap.k_new = append->k_new;
    ap.v_new = append->v_new;
    ap.k_c = append->k_c;
    ap.v_c = append->v_c;
    ap.bias_c = append->bias_c;
    ap.cache_len = append->cache_len;
  }
  if (G.dtype == KVE_BF16) {
    if (G.d == 64)
      return launch_decode_t<uint16_t, 64>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st,
                                           ap);
    return launch_decode_t<uint16_t, 128>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st,
                                          ap);
  }
  if (G.d == 64)
    return launch_decode_t<float, 64>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st, ap);
  return launch_decode_t<float, 128>(G, totalC, q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws, st, ap);
}

}  // namespace kve
