// C ABI of libkvevict: host validation, workspace sizing, kernel launches.
#include <hip/hip_runtime.h>

#include <string>

#include "../../include/kvevict.h"
#include "launch.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

kve_status set_err(kve_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

kve_status hip_err(hipError_t e, const char* where) {
  return set_err(KVE_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* kvevict_last_error(void) { return g_last_error.c_str(); }

int32_t kvevict_version(void) { return 100; }

size_t kvevict_score_workspace(const kve_layout* L) {
  kve::ScoreGeom G;
  std::string msg;
  if (kve::plan_score(L, &G, &msg) != KVE_OK) return 0;
  return G.bytes;
}

kve_status kvevict_score_ex(const kve_layout* L, const void* q_win, const void* k, const void* v,
                            float sm_scale, int32_t causal, int32_t pool_kernel, int32_t score_kind,
                            int32_t pool_mode, float* scores, void* ws, size_t ws_bytes, void* stream) {
  kve::ScoreGeom G;
  std::string msg;
  kve_status st = kve::plan_score(L, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_score: " + msg);
  if (!q_win || !k || !v || !scores) return set_err(KVE_EINVAL, "kvevict_score: null tensor pointer");
  if (!(sm_scale > 0.f) || sm_scale > 1e6f) return set_err(KVE_EINVAL, "kvevict_score: sm_scale must be in (0, 1e6]");
  if (pool_kernel < 1 || pool_kernel > 31 || pool_kernel % 2 == 0)
    return set_err(KVE_EINVAL, "kvevict_score: pool_kernel must be odd and in [1, 31]");
  if (score_kind < KVE_SCORE_PERTURB || score_kind > KVE_SCORE_KNORM)
    return set_err(KVE_EINVAL, "kvevict_score: unknown score kind");
  if (pool_mode != KVE_POOL_MAX && pool_mode != KVE_POOL_AVG)
    return set_err(KVE_EINVAL, "kvevict_score: unknown pool mode");
  if (score_kind != KVE_SCORE_PERTURB && score_kind != KVE_SCORE_KNORM && L->dtype != KVE_BF16)
    return set_err(KVE_ENOTSUP, "kvevict_score: attention-weight score kinds need bf16 inputs");
  if (!ws || ws_bytes < G.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_score: workspace smaller than kvevict_score_workspace()");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(q_win)) & 15)
    return set_err(KVE_EINVAL, "kvevict_score: q_win, k and v must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return set_err(KVE_EINVAL, "kvevict_score: workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  int planes = G.pool_rg;
  if (score_kind == KVE_SCORE_KNORM) {
    e = kve::launch_knorm(G, k, ws, s);
    planes = 1;
  } else if (L->dtype == KVE_BF16) {
    e = kve::launch_score_bf16(G, q_win, k, v, L->seq_off, sm_scale, causal ? 1 : 0, score_kind, ws, s);
  } else {
    e = kve::launch_score_f32(G, q_win, k, v, L->seq_off, sm_scale, causal ? 1 : 0, ws, s);
  }
  if (e != hipSuccess) return hip_err(e, "kvevict_score");
  e = kve::launch_pool(G, L->seq_off, pool_kernel, pool_mode, planes, ws, scores, s);
  if (e != hipSuccess) return hip_err(e, "kvevict_score (pool)");
  return KVE_OK;
}

kve_status kvevict_score(const kve_layout* L, const void* q_win, const void* k, const void* v,
                         float sm_scale, int32_t causal, int32_t pool_kernel, float* scores, void* ws,
                         size_t ws_bytes, void* stream) {
  return kvevict_score_ex(L, q_win, k, v, sm_scale, causal, pool_kernel, KVE_SCORE_PERTURB, KVE_POOL_MAX, scores,
                          ws, ws_bytes, stream);
}

size_t kvevict_select_workspace(const kve_layout* L, const int32_t* bud_off_host, int32_t mode) {
  kve::SelectGeom G;
  std::string msg;
  if (kve::plan_select(L, bud_off_host, mode, &G, &msg) != KVE_OK) return 0;
  return G.bytes;
}

kve_status kvevict_select_ex(const kve_layout* L, const float* scores, const int32_t* bud_off,
                             const int32_t* bud_off_host, int32_t mode, float tau, float tau_w, float mix,
                             uint64_t seed, int32_t* idx, float* bias, double* m_out, int32_t* status_out,
                             void* ws, size_t ws_bytes, void* stream) {
  kve::SelectGeom G;
  std::string msg;
  kve_status st = kve::plan_select(L, bud_off_host, mode, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_select: " + msg);
  if (!scores || !bud_off || !idx || !bias) return set_err(KVE_EINVAL, "kvevict_select: null tensor pointer");
  if (mode == KVE_SAMPLE && (!(tau > 0.f) || !(tau_w > 0.f)))
    return set_err(KVE_EINVAL, "kvevict_select: tau and tau_w must be > 0");
  if (!(mix >= 0.f && mix <= 1.f)) return set_err(KVE_EINVAL, "kvevict_select: mix must be in [0, 1]");
  if (!ws || ws_bytes < G.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_select: workspace smaller than kvevict_select_workspace()");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return set_err(KVE_EINVAL, "kvevict_select: workspace must be 256-byte aligned");
  hipError_t e = kve::launch_select(G, scores, L->seq_off, bud_off, tau, tau_w, mix, seed, idx, bias, m_out,
                                    status_out, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_err(e, "kvevict_select");
  return KVE_OK;
}

kve_status kvevict_select_soft(const kve_layout* L, const float* scores, const int32_t* bud_off,
                               const int32_t* bud_off_host, const int32_t* cap_off, const int32_t* cap_off_host,
                               float tau, float tau_w, float mix, uint64_t seed, int32_t* idx, float* bias,
                               int32_t* kept, double* m_out, int32_t* status_out, void* ws, size_t ws_bytes,
                               void* stream) {
  kve::SelectGeom G;
  std::string msg;
  kve_status st = kve::plan_select(L, bud_off_host, KVE_SAMPLE, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_select_soft: " + msg);
  if (!scores || !bud_off || !idx || !bias || !cap_off || !cap_off_host)
    return set_err(KVE_EINVAL, "kvevict_select_soft: null pointer");
  if (cap_off_host[0] != 0) return set_err(KVE_EINVAL, "kvevict_select_soft: cap_off[0] must be 0");
  for (int s = 0; s < L->S; ++s) {
    const int64_t C = static_cast<int64_t>(cap_off_host[s + 1]) - cap_off_host[s];
    const int64_t n = static_cast<int64_t>(L->seq_off_host[s + 1]) - L->seq_off_host[s];
    if (C < 0 || C > n) return set_err(KVE_EINVAL, "kvevict_select_soft: capacity cap_s must be in [0, n_s]");
    const int64_t B = static_cast<int64_t>(bud_off_host[s + 1]) - bud_off_host[s];
    if (B >= n && C != n) return set_err(KVE_EINVAL, "kvevict_select_soft: B_s = n_s needs cap_s = n_s");
  }
  if (!(tau > 0.f) || !(tau_w > 0.f)) return set_err(KVE_EINVAL, "kvevict_select_soft: tau and tau_w must be > 0");
  if (!(mix >= 0.f && mix <= 1.f)) return set_err(KVE_EINVAL, "kvevict_select_soft: mix must be in [0, 1]");
  if (!ws || ws_bytes < G.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_select_soft: workspace smaller than kvevict_select_workspace()");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return set_err(KVE_EINVAL, "kvevict_select_soft: workspace must be 256-byte aligned");
  const kve::SoftBudget soft{cap_off, cap_off_host[L->S], kept};
  hipError_t e = kve::launch_select(G, scores, L->seq_off, bud_off, tau, tau_w, mix, seed, idx, bias, m_out,
                                    status_out, ws, static_cast<hipStream_t>(stream), &soft);
  if (e != hipSuccess) return hip_err(e, "kvevict_select_soft");
  return KVE_OK;
}

size_t kvevict_merge_workspace(const kve_layout* L, const int32_t* bud_off_host) {
  kve::MergeGeom G;
  std::string msg;
  if (kve::plan_merge(L, bud_off_host, &G, &msg) != KVE_OK) return 0;
  return G.bytes;
}

kve_status kvevict_merge(const kve_layout* L, const void* k, const int32_t* bud_off, const int32_t* bud_off_host,
                         const int32_t* idx, float tau_merge, float* bias, int32_t* merged, int32_t* target,
                         void* ws, size_t ws_bytes, void* stream) {
  kve::MergeGeom G;
  std::string msg;
  kve_status st = kve::plan_merge(L, bud_off_host, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_merge: " + msg);
  if (!k || !bud_off || !idx || !bias) return set_err(KVE_EINVAL, "kvevict_merge: null pointer");
  if (!(tau_merge >= -1.f && tau_merge <= 1.f)) return set_err(KVE_EINVAL, "kvevict_merge: tau_merge must be in [-1, 1]");
  if (reinterpret_cast<uintptr_t>(k) & 15) return set_err(KVE_EINVAL, "kvevict_merge: k must be 16-byte aligned");
  if (!ws || ws_bytes < G.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_merge: workspace smaller than kvevict_merge_workspace()");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_err(KVE_EINVAL, "kvevict_merge: workspace must be 256-byte aligned");
  hipError_t e = kve::launch_merge(G, k, L->seq_off, bud_off, idx, tau_merge, bias, merged, target, ws,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_err(e, "kvevict_merge");
  return KVE_OK;
}

size_t kvevict_select_literal_workspace(const kve_layout* L) {
  kve::LiteralGeom G;
  std::string msg;
  if (kve::plan_literal(L, &G, &msg) != KVE_OK) return 0;
  return G.bytes;
}

kve_status kvevict_select_literal(const kve_layout* L, const float* scores, const double* m_in,
                                  const int32_t* cap_off, const int32_t* cap_off_host, float tau, float tau_w,
                                  float mix, uint64_t seed, int32_t* idx, float* bias, int32_t* kept,
                                  int32_t* status_out, void* ws, size_t ws_bytes, void* stream) {
  kve::LiteralGeom G;
  std::string msg;
  kve_status st = kve::plan_literal(L, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_select_literal: " + msg);
  if (!scores || !m_in || !idx || !bias || !cap_off || !cap_off_host)
    return set_err(KVE_EINVAL, "kvevict_select_literal: null pointer");
  if (cap_off_host[0] != 0) return set_err(KVE_EINVAL, "kvevict_select_literal: cap_off[0] must be 0");
  for (int s = 0; s < L->S; ++s) {
    const int64_t C = static_cast<int64_t>(cap_off_host[s + 1]) - cap_off_host[s];
    const int64_t n = static_cast<int64_t>(L->seq_off_host[s + 1]) - L->seq_off_host[s];
    if (C < 0 || C > n) return set_err(KVE_EINVAL, "kvevict_select_literal: capacity cap_s must be in [0, n_s]");
  }
  if (!(tau > 0.f) || !(tau_w > 0.f)) return set_err(KVE_EINVAL, "kvevict_select_literal: tau and tau_w must be > 0");
  if (!(mix >= 0.f && mix <= 1.f)) return set_err(KVE_EINVAL, "kvevict_select_literal: mix must be in [0, 1]");
  if (!ws || ws_bytes < G.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_select_literal: workspace smaller than kvevict_select_literal_workspace()");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return set_err(KVE_EINVAL, "kvevict_select_literal: workspace must be 256-byte aligned");
  hipError_t e = kve::launch_literal(G, L->seq_off, scores, m_in, cap_off, cap_off_host[L->S], tau, tau_w, mix, seed,
                                     idx, bias, kept, status_out, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_err(e, "kvevict_select_literal");
  return KVE_OK;
}

kve_status kvevict_select(const kve_layout* L, const float* scores, const int32_t* bud_off,
                          const int32_t* bud_off_host, int32_t mode, float tau, float tau_w, uint64_t seed,
                          int32_t* idx, float* bias, double* m_out, int32_t* status_out, void* ws,
                          size_t ws_bytes, void* stream) {
  return kvevict_select_ex(L, scores, bud_off, bud_off_host, mode, tau, tau_w, 1.f, seed, idx, bias, m_out,
                           status_out, ws, ws_bytes, stream);
}

kve_status kvevict_compact(const kve_layout* L, const void* k, const void* v, const int32_t* bud_off,
                           const int32_t* bud_off_host, const int32_t* idx, const float* bias,
                           const int32_t* cap_off, const int32_t* cap_off_host, void* k_c, void* v_c,
                           float* bias_c, void* stream) {
  std::string msg;
  kve_status st = kve::check_compact(L, bud_off_host, cap_off_host, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_compact: " + msg);
  if (!k || !v || !bud_off || !idx || !bias || !cap_off || !k_c || !v_c || !bias_c)
    return set_err(KVE_EINVAL, "kvevict_compact: null tensor pointer");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(k_c) |
       reinterpret_cast<uintptr_t>(v_c)) & 15)
    return set_err(KVE_EINVAL, "kvevict_compact: k, v, k_c, v_c must be 16-byte aligned");
  if (k_c == k || v_c == v || k_c == v || v_c == k)
    return set_err(KVE_EINVAL, "kvevict_compact: outputs must not alias inputs");
  int maxB = 0;
  for (int s = 0; s < L->S; ++s) maxB = std::max(maxB, bud_off_host[s + 1] - bud_off_host[s]);
  const int esize = (L->dtype == KVE_BF16) ? 2 : 4;
  hipError_t e = kve::launch_compact(L->S, L->Hkv, L->d, esize, L->seq_off_host[L->S], bud_off_host[L->S],
                                     cap_off_host[L->S], maxB, k, v, L->seq_off, bud_off, idx, bias, cap_off,
                                     k_c, v_c, bias_c, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_err(e, "kvevict_compact");
  return KVE_OK;
}

size_t kvevict_evict_workspace(const kve_layout* L, const int32_t* bud_off_host, int32_t mode) {
  const size_t a = kvevict_score_workspace(L);
  const size_t b = kvevict_select_workspace(L, bud_off_host, mode);
  if (a == 0 || b == 0) return 0;
  return ((a + 255) & ~static_cast<size_t>(255)) + b;
}

kve_status kvevict_evict(const kve_layout* L, const void* q_win, const void* k, const void* v, float sm_scale,
                         int32_t causal, int32_t pool_kernel, const int32_t* bud_off, const int32_t* bud_off_host,
                         int32_t mode, float tau, float tau_w, uint64_t seed, float* scores, int32_t* idx,
                         float* bias, double* m_out, int32_t* status_out, const int32_t* cap_off,
                         const int32_t* cap_off_host, void* k_c, void* v_c, float* bias_c, void* ws,
                         size_t ws_bytes, void* stream) {
  kve::ScoreGeom Gs;
  kve::SelectGeom Gl;
  std::string msg;
  kve_status st = kve::plan_score(L, &Gs, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_evict: " + msg);
  st = kve::plan_select(L, bud_off_host, mode, &Gl, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_evict: " + msg);
  st = kve::check_compact(L, bud_off_host, cap_off_host, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_evict: " + msg);
  if (!q_win || !k || !v || !scores || !bud_off || !idx || !bias || !cap_off || !k_c || !v_c || !bias_c)
    return set_err(KVE_EINVAL, "kvevict_evict: null tensor pointer");
  if (!(sm_scale > 0.f) || sm_scale > 1e6f) return set_err(KVE_EINVAL, "kvevict_evict: sm_scale must be in (0, 1e6]");
  if (pool_kernel < 1 || pool_kernel > 31 || pool_kernel % 2 == 0)
    return set_err(KVE_EINVAL, "kvevict_evict: pool_kernel must be odd and in [1, 31]");
  if (mode == KVE_SAMPLE && (!(tau > 0.f) || !(tau_w > 0.f)))
    return set_err(KVE_EINVAL, "kvevict_evict: tau and tau_w must be > 0");
  const size_t off_sel = (Gs.bytes + 255) & ~static_cast<size_t>(255);
  if (!ws || ws_bytes < off_sel + Gl.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_evict: workspace smaller than kvevict_evict_workspace()");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_err(KVE_EINVAL, "kvevict_evict: workspace must be 256-byte aligned");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(q_win) |
       reinterpret_cast<uintptr_t>(k_c) | reinterpret_cast<uintptr_t>(v_c)) & 15)
    return set_err(KVE_EINVAL, "kvevict_evict: q_win, k, v, k_c and v_c must be 16-byte aligned");
  if (k_c == k || v_c == v || k_c == v || v_c == k)
    return set_err(KVE_EINVAL, "kvevict_evict: outputs must not alias inputs");
  char* wsb = static_cast<char*>(ws);
  void* ws_sel = wsb + off_sel;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // bf16, and a selection whose first pass can pool and whose ordered write
  // can gather: top-k over several chunks or the sampling chain; otherwise
  // the three calls in turn
  const bool fuse = L->dtype == KVE_BF16 && (mode == KVE_SAMPLE || Gl.max_len > kve::kSelChunk);
  if (!fuse) {
    st = kvevict_score(L, q_win, k, v, sm_scale, causal, pool_kernel, scores, ws, off_sel, stream);
    if (st != KVE_OK) return st;
    st = kvevict_select(L, scores, bud_off, bud_off_host, mode, tau, tau_w, seed, idx, bias, m_out, status_out,
                        ws_sel, ws_bytes - off_sel, stream);
    if (st != KVE_OK) return st;
    return kvevict_compact(L, k, v, bud_off, bud_off_host, idx, bias, cap_off, cap_off_host, k_c, v_c, bias_c,
                           stream);
  }
  kve::ScoreZero z{};
  if (mode == KVE_TOPK) {   // what the selection's own clearing launch would clear
    z.p = reinterpret_cast<int*>(static_cast<char*>(ws_sel) + Gl.off_hist);
    z.n = static_cast<int>((Gl.zero_end - Gl.off_hist) / sizeof(int));
    z.m = m_out;
    z.st = status_out;
    z.nsh = L->S * L->Hkv;
  }
  hipError_t e = kve::launch_score_bf16(Gs, q_win, k, v, L->seq_off, sm_scale, causal ? 1 : 0, KVE_SCORE_PERTURB,
                                        ws, s, mode == KVE_TOPK ? &z : nullptr);
  if (e != hipSuccess) return hip_err(e, "kvevict_evict (score)");
  const kve::PoolSrc pool{reinterpret_cast<const float*>(wsb + Gs.off_sraw), scores, Gs.pool_rg, (pool_kernel - 1) / 2};
  // the ordered write gathers the kept rows itself (bf16 rows of d values)
  const kve::CompactDst cd{static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), static_cast<uint8_t*>(k_c),
                           static_cast<uint8_t*>(v_c), bias_c, cap_off, cap_off_host[L->S], L->d * 2};
  e = kve::launch_select(Gl, scores, L->seq_off, bud_off, tau, tau_w, 1.f, seed, idx, bias, m_out, status_out, ws_sel,
                         s, nullptr, &pool, &cd);
  if (e != hipSuccess) return hip_err(e, "kvevict_evict (select)");
  return KVE_OK;
}

size_t kvevict_decode_workspace(const kve_layout* L, int32_t max_cache_len) {
  kve::DecodeGeom G;
  std::string msg;
  // sizing depends on the shape and max_cache_len only (no capacity check)
  if (kve::plan_decode(L, nullptr, max_cache_len, &G, &msg) != KVE_OK) return 0;
  return G.bytes;
}

kve_status kvevict_decode_snis(const kve_layout* L, const void* q, const void* k_c, const void* v_c,
                               const float* bias_c, const int32_t* cap_off, const int32_t* cap_off_host,
                               const int32_t* cache_len, int32_t max_cache_len, float sm_scale, float* out,
                               void* ws, size_t ws_bytes, void* stream) {
  kve::DecodeGeom G;
  std::string msg;
  if (!cap_off_host) return set_err(KVE_EINVAL, "kvevict_decode_snis: cap_off_host is NULL");
  kve_status st = kve::plan_decode(L, cap_off_host, max_cache_len, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_decode_snis: " + msg);
  if (!q || !k_c || !v_c || !bias_c || !cap_off || !cache_len || !out)
    return set_err(KVE_EINVAL, "kvevict_decode_snis: null tensor pointer");
  if (!(sm_scale > 0.f)) return set_err(KVE_EINVAL, "kvevict_decode_snis: sm_scale must be > 0");
  if (!ws || ws_bytes < G.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_decode_snis: workspace smaller than kvevict_decode_workspace()");
  hipError_t e = kve::launch_decode(G, cap_off_host[L->S], q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale,
                                    out, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_err(e, "kvevict_decode_snis");
  return KVE_OK;
}

kve_status kvevict_decode_snis_append(const kve_layout* L, const void* q, const void* k_new, const void* v_new,
                                      void* k_c, void* v_c, float* bias_c, const int32_t* cap_off,
                                      const int32_t* cap_off_host, int32_t* cache_len, int32_t max_cache_len,
                                      float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  kve::DecodeGeom G;
  std::string msg;
  if (!cap_off_host) return set_err(KVE_EINVAL, "kvevict_decode_snis_append: cap_off_host is NULL");
  kve_status st = kve::plan_decode(L, cap_off_host, max_cache_len, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_decode_snis_append: " + msg);
  if (!q || !k_new || !v_new || !k_c || !v_c || !bias_c || !cap_off || !cache_len || !out)
    return set_err(KVE_EINVAL, "kvevict_decode_snis_append: null tensor pointer");
  if (!(sm_scale > 0.f)) return set_err(KVE_EINVAL, "kvevict_decode_snis_append: sm_scale must be > 0");
  if (!ws || ws_bytes < G.bytes)
    return set_err(KVE_EWORKSPACE, "kvevict_decode_snis_append: workspace smaller than kvevict_decode_workspace()");
  const kve::DecodeAppendArgs ap{k_new, v_new, k_c, v_c, bias_c, cache_len};
  hipError_t e = kve::launch_decode(G, cap_off_host[L->S], q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale,
                                    out, ws, static_cast<hipStream_t>(stream), &ap);
  if (e != hipSuccess) return hip_err(e, "kvevict_decode_snis_append");
  return KVE_OK;
}

size_t kvevict_decode_scratch_max(void) { return kve::kDecodeScratchBytes; }

kve_status kvevict_decode_snis_noalloc(const kve_layout* L, const void* q, const void* k_c, const void* v_c,
                                       const float* bias_c, const int32_t* cap_off, const int32_t* cap_off_host,
                                       const int32_t* cache_len, int32_t max_cache_len, float sm_scale,
                                       float* out, void* stream) {
  kve::DecodeGeom G;
  std::string msg;
  if (!cap_off_host) return set_err(KVE_EINVAL, "kvevict_decode_snis_noalloc: cap_off_host is NULL");
  kve_status st = kve::plan_decode(L, cap_off_host, max_cache_len, &G, &msg);
  if (st != KVE_OK) return set_err(st, "kvevict_decode_snis_noalloc: " + msg);
  if (!q || !k_c || !v_c || !bias_c || !cap_off || !cache_len || !out)
    return set_err(KVE_EINVAL, "kvevict_decode_snis_noalloc: null tensor pointer");
  if (!(sm_scale > 0.f)) return set_err(KVE_EINVAL, "kvevict_decode_snis_noalloc: sm_scale must be > 0");
  if (G.bytes > kve::kDecodeScratchBytes)
    return set_err(KVE_EWORKSPACE, "kvevict_decode_snis_noalloc: this batch needs " + std::to_string(G.bytes) +
                                       " bytes of decode scratch, more than the " +
                                       std::to_string(kve::kDecodeScratchBytes) +
                                       " the library holds per device (use kvevict_decode_snis)");
  void* ws = nullptr;
  hipError_t e = kve::decode_scratch(&ws);
  if (e != hipSuccess) return hip_err(e, "kvevict_decode_snis_noalloc: scratch address");
  e = kve::launch_decode(G, cap_off_host[L->S], q, k_c, v_c, bias_c, cap_off, cache_len, sm_scale, out, ws,
                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_err(e, "kvevict_decode_snis_noalloc");
  return KVE_OK;
}

}  // extern "C"
