// Opt-in per-kernel timing with HIP events, recorded on the launch stream
// around each kernel of the library (instrumentation only; off by default,
// a single branch per launch when off).
#pragma once

#include <hip/hip_runtime.h>

namespace kve {

enum Stage {
  ST_SCORE_P1 = 0,
  ST_SCORE_MERGE = 1,
  ST_SCORE_P2 = 2,
  ST_SCORE_POOL = 3,
  ST_SELECT = 4,
  ST_COMPACT = 5,
  ST_DECODE_SPLIT = 6,
  ST_DECODE_MERGE = 7,
  ST_COUNT = 8
};

void stage_begin(int stage, hipStream_t st);
void stage_end(int stage, hipStream_t st);

}  // namespace kve
