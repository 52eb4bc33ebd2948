// Host-side launch geometry and argument validation.  Pure C++ (no HIP),
// so it can be built and tested with g++ on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/kvevict.h"

namespace kve {

// Largest key chunk one scorer workgroup handles (its per-key LDS buffers
// are sized for it).
constexpr int kScoreChunkMax = 2048;

// Floats per (window row, key chunk) record of the scorer's first pass: the
// softmax reference m, the weight sum of every key but the row's candidate
// for a dominant key, and that candidate's weight and key (int bits).  The
// rounding error of the weight its P.V contraction used has a plane of its
// own (only the merge of a row with a dominant key reads it).
constexpr int kScoreRec = 4;

// Geometry of one kvevict_score call; the workspace is carved into the
// regions below (byte offsets, each 256-byte aligned).
struct ScoreGeom {
  int S, Hq, Hkv, d, w, T, dtype;
  int max_len;
  int R;        // rows per group = (Hq/Hkv) * w
  int RG;       // row groups of 128 rows
  int CH;       // keys per chunk (multiple of 256)
  int P;        // chunks per sequence (grid x), ceil(max_len / CH)
  int pool_rg;  // partial score planes summed by the pool kernel
  size_t off_part_ml, off_part_e, off_part_x, off_part_o, off_vnorm, off_lse2, off_no2, off_no2d, off_ohi, off_olo, off_sraw, off_jstar,
      off_cstar;
  size_t bytes;
};

// Keys per workgroup of the multi-workgroup selection, histogram width
// (2048 bins = 11-bit digits), digit levels for fp32 scores and fp64 Gumbel
// keys, per-head state slots, the points of the coarse expected-samples
// grid that brackets the search, and the step budget of the search that
// follows (a safeguarded Newton iteration in log m; started from the grid
// it needed at most 3 updates on the proposals tried; a head still outside
// the band afterwards finishes with the pages' integer binary search).
constexpr int kSelChunk = 1024;
constexpr int kSmpChunk = 1024;       // keys per workgroup of the sampling passes
constexpr int kSelBins = 2048;
constexpr int kSelLevels32 = 3;
constexpr int kSelLevels64 = 6;
constexpr int kSelGrid = 32;
constexpr int kSelSearchSteps = 3;
constexpr int kSelRStateBytes = 16;   // per-head radix threshold and count of equal keys kept
constexpr int kSelSearchBytes = 32;   // per-head search state
constexpr int kSelRCacheBytes = 16;   // per-head, per-level resolved threshold digits
// Keys of one selection chunk that share the threshold's leading digits are
// listed (their last digits) when at most this many; a chunk with more
// stores the suffix sums of their last-digit histogram instead.
constexpr int kSelListMax = 64;

struct SelectGeom {
  int S, Hkv, T, max_len, mode;
  int nchunk;                      // chunks of kSelChunk keys per (sequence, head)
  int nsmp;                        // chunks of kSmpChunk keys (sampling passes)
  int64_t total_B;
  size_t off_a, off_b;             // sampling: fp64 planes [Hkv][T]
  size_t off_hist;                 // int [levels][S*Hkv][kSelBins]
  size_t zero_end;                 // [off_hist, zero_end) is cleared on entry
  size_t off_cand;                 // int [S*Hkv][nchunk][kSelChunk] per chunk: listed last digits or suffix sums
  size_t off_cnt;                  // int [S*Hkv][nchunk][2]
  size_t off_rstate;               // [S*Hkv] radix threshold state (kSelRStateBytes each)
  size_t off_rcache;               // [S*Hkv][kSelLevels64] resolved digits (kSelRCacheBytes each)
  size_t off_part;                 // sampling: double [2][S*Hkv][nchunk][3]
  size_t off_grid;                 // sampling: float [S*Hkv][nchunk][kSelGrid]
  size_t off_state;                // sampling: [2][S*Hkv] search state (kSelSearchBytes each)
  size_t off_mvals;                // sampling: double [S*Hkv] final m
  size_t off_bsh;                  // sampling: int [S*Hkv] kept count per head (soft budget)
  size_t bytes;
};

// Literal estimator: draws per head (the per-entry counts are int32), and
// the longest sequence (its chunk offsets are held in LDS).
constexpr int64_t kLitMaxDraws = (int64_t(1) << 31) - 1;
constexpr int kLitMaxLen = 4096 * kSmpChunk;

struct LiteralGeom {
  int S, Hkv, T, nch;
  size_t off_part, off_pi, off_cdf, off_cnt, off_nz;
  size_t bytes;
};

struct MergeGeom {
  int S, Hkv, T, max_len, maxB;
  int64_t totalB;
  size_t off_invn, off_flag, off_best, off_cnt;
  size_t bytes;
};

// Cache entries per decode workgroup for bf16 caches: 4 waves, each two
// blocks of 32 entries.
constexpr int kDecodeChunkBf16 = 256;

// Device scratch the allocation-free decode entry point holds per GPU (its
// split partials: S * Hq * splits * (d + 2) floats, 256-byte aligned parts).
constexpr size_t kDecodeScratchBytes = static_cast<size_t>(8) << 20;

struct DecodeGeom {
  int S, Hq, Hkv, d, dtype, splits, split_len;
  size_t off_ml, off_o;
  size_t off_app;                  // int [S][2]: entries attended and the appended slot (or -1), per sequence
  size_t bytes;
};

// Validation of the shared layout.  Returns KVE_OK or an error code and sets
// *msg.  On success fills the geometry.
kve_status plan_score(const kve_layout* L, ScoreGeom* G, std::string* msg);
kve_status plan_select(const kve_layout* L, const int32_t* bud_off_host, int mode, SelectGeom* G,
                       std::string* msg);
kve_status check_compact(const kve_layout* L, const int32_t* bud_off_host, const int32_t* cap_off_host,
                         std::string* msg);
kve_status plan_merge(const kve_layout* L, const int32_t* bud_off_host, MergeGeom* G, std::string* msg);
kve_status plan_literal(const kve_layout* L, LiteralGeom* G, std::string* msg);
kve_status plan_decode(const kve_layout* L, const int32_t* cap_off_host, int max_cache_len,
                       DecodeGeom* G, std::string* msg);

}  // namespace kve
