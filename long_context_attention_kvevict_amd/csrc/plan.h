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
  size_t off_part_ml, off_part_o, off_vnorm, off_lse2, off_no2, off_no2d, off_ohi, off_olo, off_sraw;
  size_t bytes;
};

// Keys per workgroup of the multi-workgroup radix select and its histogram
// width (2048 bins = 11-bit digits).
constexpr int kSelChunk = 4096;
constexpr int kSelBins = 2048;
constexpr int kSelLevels32 = 3;

struct SelectGeom {
  int S, Hkv, T, max_len, mode;
  int nchunk;                      // chunks of kSelChunk keys per (sequence, head)
  int64_t total_B;
  size_t off_a, off_b;             // sample mode: fp64 planes [Hkv][T]
  size_t off_hist;                 // top-k: int [levels][S*Hkv][kSelBins]
  size_t off_cnt;                  // top-k: int [S*Hkv][nchunk][2]
  size_t off_state;                // top-k: uint32 [S*Hkv][2]
  size_t bytes;
};

struct DecodeGeom {
  int S, Hq, Hkv, d, dtype, splits, split_len;
  size_t off_ml, off_o;
  size_t bytes;
};

// Validation of the shared layout.  Returns KVE_OK or an error code and sets
// *msg.  On success fills the geometry.
kve_status plan_score(const kve_layout* L, ScoreGeom* G, std::string* msg);
kve_status plan_select(const kve_layout* L, const int32_t* bud_off_host, int mode, SelectGeom* G,
                       std::string* msg);
kve_status check_compact(const kve_layout* L, const int32_t* bud_off_host, const int32_t* cap_off_host,
                         std::string* msg);
kve_status plan_decode(const kve_layout* L, const int32_t* cap_off_host, int max_cache_len,
                       DecodeGeom* G, std::string* msg);

}  // namespace kve
