// Host-only driver for the planner/validator (plan.cpp), built with g++ and
// no HIP toolchain: forces every argument error path and prints "ok".
#include <cstdio>
#include <string>

#include "../long_context_attention_kvevict_amd/csrc/plan.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      std::printf("FAILED %s:%d %s\n", __FILE__, __LINE__, #cond);   \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main() {
  using namespace kve;
  int32_t off[3] = {0, 4096, 4096 + 131072};
  kve_layout L{2, 32, 8, 128, 32, KVE_BF16, off, off};
  std::string msg;
  ScoreGeom G;
  CHECK(plan_score(&L, &G, &msg) == KVE_OK);
  CHECK(G.R == 128 && G.RG == 1 && G.CH % 256 == 0 && G.P * G.CH >= 131072);
  CHECK(G.off_sraw + static_cast<size_t>(G.Hkv) * G.T * 4 <= G.bytes);
  kve_layout Q{1, 28, 4, 128, 64, KVE_BF16, off, off};
  CHECK(plan_score(&Q, &G, &msg) == KVE_OK && G.RG == 4 && G.pool_rg == 4);

  kve_layout bad = L;
  bad.Hq = 30;
  CHECK(plan_score(&bad, &G, &msg) == KVE_EINVAL);
  bad = L; bad.d = 64;
  CHECK(plan_score(&bad, &G, &msg) == KVE_ENOTSUP);
  bad = L; bad.dtype = KVE_F32; bad.d = 64;
  CHECK(plan_score(&bad, &G, &msg) == KVE_OK);
  bad = L; bad.w = 0;
  CHECK(plan_score(&bad, &G, &msg) == KVE_EINVAL);
  bad = L; bad.seq_off_host = nullptr;
  CHECK(plan_score(&bad, &G, &msg) == KVE_EINVAL);
  int32_t desc[3] = {0, 10, 5};
  bad = L; bad.seq_off_host = desc;
  CHECK(plan_score(&bad, &G, &msg) == KVE_EINVAL);
  CHECK(plan_score(nullptr, &G, &msg) == KVE_EINVAL);

  SelectGeom SG;
  int32_t bud[3] = {0, 409, 409 + 6553};
  CHECK(plan_select(&L, bud, KVE_TOPK, &SG, &msg) == KVE_OK && SG.total_B == 409 + 6553);
  int32_t bud_big[3] = {0, 4097, 5000};
  CHECK(plan_select(&L, bud_big, KVE_TOPK, &SG, &msg) == KVE_EINVAL);
  CHECK(plan_select(&L, bud, 3, &SG, &msg) == KVE_EINVAL);
  CHECK(plan_select(&L, nullptr, KVE_TOPK, &SG, &msg) == KVE_EINVAL);

  int32_t cap[3] = {0, 409 + 128, 409 + 128 + 6553 + 128};
  CHECK(check_compact(&L, bud, cap, &msg) == KVE_OK);
  int32_t cap_small[3] = {0, 100, 200};
  CHECK(check_compact(&L, bud, cap_small, &msg) == KVE_EINVAL);

  DecodeGeom DG;
  CHECK(plan_decode(&L, cap, 6553 + 128, &DG, &msg) == KVE_OK);
  CHECK(DG.splits * DG.split_len >= 6553 + 128 && DG.split_len % 64 == 0);
  CHECK(plan_decode(&L, cap, 1 << 20, &DG, &msg) == KVE_EINVAL);
  CHECK(plan_decode(&L, cap, 0, &DG, &msg) == KVE_EINVAL);
  CHECK(plan_decode(&L, nullptr, 1000, &DG, &msg) == KVE_OK);   // sizing only
  kve_layout wide = L; wide.Hq = 8 * 17;
  CHECK(plan_decode(&wide, cap, 100, &DG, &msg) == KVE_ENOTSUP);
  std::printf("ok\n");
  return 0;
}
