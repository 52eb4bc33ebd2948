// Kernel launchers (one per translation unit), called by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace kve {

// Memory a later selection needs cleared, cleared by the scorer's merge
// launch instead of a launch of its own (one-call eviction): n ints at p, and
// m = 0, status = KVE_OK for nsh heads (m and st may be NULL).
struct ScoreZero {
  int* p;
  int n;
  double* m;
  int32_t* st;
  int nsh;
};
hipError_t launch_score_bf16(const ScoreGeom& G, const void* q_win, const void* k, const void* v,
                             const int32_t* seq_off, float sm_scale, int causal, int score_kind, void* ws,
                             hipStream_t st, const ScoreZero* zero = nullptr);
hipError_t launch_score_f32(const ScoreGeom& G, const void* q_win, const void* k, const void* v,
                            const int32_t* seq_off, float sm_scale, int causal, void* ws,
                            hipStream_t st);
hipError_t launch_merge_f32(const ScoreGeom& G, const int32_t* seq_off, void* ws, hipStream_t st);
hipError_t launch_knorm(const ScoreGeom& G, const void* k, void* ws, hipStream_t st);
hipError_t launch_pool(const ScoreGeom& G, const int32_t* seq_off, int pool_kernel, int pool_mode, int planes,
                       const void* ws, float* scores, hipStream_t st);

// Soft per-sequence budget of the sampling selection: output slots per
// sequence (capacities) and the per-head kept counts returned to the caller.
struct SoftBudget {
  const int32_t* cap_off;   // device [S+1]
  int64_t total_cap;        // cap_off[S]
  int32_t* kept;            // device [S*Hkv] out, or NULL
};
// Max pooling folded into the first selection pass (one-call eviction): the
// pass reads the scorer's raw planes, writes the pooled plane to `out` and
// selects on it; the selection's counters must already be clear (ScoreZero).
struct PoolSrc {
  const float* sraw;   // [planes][Hkv][T] raw score planes (summed in order)
  float* out;          // [Hkv][T] pooled scores
  int planes;
  int radius;          // (pool kernel - 1) / 2, at most kPoolMaxRadius
};
constexpr int kPoolMaxRadius = 15;
// The compaction folded into the selection's ordered write (one-call
// eviction): each workgroup gathers the K/V rows of the keys it keeps into
// the compact cache, row cap_off[s] + slot of KV head h, with their bias.
struct CompactDst {
  const uint8_t* k;        // [Hkv][T] rows of row_bytes
  const uint8_t* v;
  uint8_t* k_c;            // [Hkv][totalC] rows of row_bytes
  uint8_t* v_c;
  float* bias_c;           // [Hkv][totalC]
  const int32_t* cap_off;  // [S+1] device
  int64_t totalC;
  int row_bytes;           // a multiple of 16
};
hipError_t launch_select(const SelectGeom& G, const float* scores, const int32_t* seq_off,
                         const int32_t* bud_off, float tau, float tau_w, float mix, uint64_t seed,
                         int32_t* idx, float* bias, double* m_out, int32_t* status_out, void* ws,
                         hipStream_t st, const SoftBudget* soft = nullptr, const PoolSrc* pool = nullptr,
                         const CompactDst* compact = nullptr);

hipError_t launch_literal(const LiteralGeom& G, const int32_t* seq_off, const float* scores, const double* m_in,
                          const int32_t* cap_off, int64_t total_cap, float tau, float tau_w, float mix,
                          uint64_t seed, int32_t* idx, float* bias, int32_t* kept, int32_t* status, void* ws,
                          hipStream_t st);

hipError_t launch_merge(const MergeGeom& G, const void* k, const int32_t* seq_off, const int32_t* bud_off,
                        const int32_t* idx, float tau, float* bias, int32_t* merged, int32_t* target, void* ws,
                        hipStream_t st);

hipError_t launch_compact(int S, int Hkv, int d, int esize, int T, int64_t totalB, int64_t totalC,
                          int maxB, const void* k, const void* v, const int32_t* seq_off,
                          const int32_t* bud_off, const int32_t* idx, const float* bias,
                          const int32_t* cap_off, void* k_c, void* v_c, float* bias_c,
                          hipStream_t st);

// Device address of the decode scratch array on the current device.
hipError_t decode_scratch(void** ptr);

// The decode that appends the step's token itself (NULL: the plain decode).
struct DecodeAppendArgs {
  const void* k_new;   // [Hkv][S][d]
  const void* v_new;
  void* k_c;
  void* v_c;
  float* bias_c;
  int32_t* cache_len;
};
hipError_t launch_decode(const DecodeGeom& G, int64_t totalC, const void* q, const void* k_c,
                         const void* v_c, const float* bias_c, const int32_t* cap_off,
                         const int32_t* cache_len, float sm_scale, float* out, void* ws,
                         hipStream_t st, const DecodeAppendArgs* append = nullptr);

}  // namespace kve
