// Host-side argument validation and launch geometry (pure C++).
#include "plan.h"

#include <algorithm>
#include <cstdio>

namespace kve {

namespace {

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

kve_status fail(std::string* msg, kve_status st, const char* what) {
  if (msg) *msg = what;
  return st;
}

kve_status check_layout(const kve_layout* L, std::string* msg, int* max_len, int64_t* T) {
  char buf[256];
  if (!L) return fail(msg, KVE_EINVAL, "layout is NULL");
  if (L->S < 1) return fail(msg, KVE_EINVAL, "S must be >= 1");
  if (L->Hq < 1 || L->Hkv < 1) return fail(msg, KVE_EINVAL, "Hq and Hkv must be >= 1");
  if (L->Hq % L->Hkv != 0) return fail(msg, KVE_EINVAL, "Hq must be a multiple of Hkv");
  if (L->w < 1 || L->w > 64) return fail(msg, KVE_EINVAL, "w must be in [1, 64]");
  if (L->dtype != KVE_BF16 && L->dtype != KVE_F32) return fail(msg, KVE_EINVAL, "unknown dtype");
  if (L->dtype == KVE_BF16 && L->d != 128)
    return fail(msg, KVE_ENOTSUP, "bf16 path supports d = 128 only");
  if (L->dtype == KVE_F32 && L->d != 64 && L->d != 128)
    return fail(msg, KVE_ENOTSUP, "fp32 path supports d in {64, 128}");
  if (!L->seq_off || !L->seq_off_host) return fail(msg, KVE_EINVAL, "seq_off / seq_off_host is NULL");
  if (L->seq_off_host[0] != 0) return fail(msg, KVE_EINVAL, "seq_off[0] must be 0");
  int mx = 0;
  for (int s = 0; s < L->S; ++s) {
    const int64_t n = static_cast<int64_t>(L->seq_off_host[s + 1]) - L->seq_off_host[s];
    if (n < 1) {
      std::snprintf(buf, sizeof buf, "sequence %d has %lld tokens (need >= 1)", s, (long long)n);
      return fail(msg, KVE_EINVAL, buf);
    }
    mx = std::max<int>(mx, static_cast<int>(n));
  }
  const int64_t tot = L->seq_off_host[L->S];
  if (tot <= 0 || tot >= (static_cast<int64_t>(1) << 31) / 2)
    return fail(msg, KVE_EINVAL, "total tokens T out of range");
  if (static_cast<int64_t>(L->Hkv) * tot * L->d >= (static_cast<int64_t>(1) << 40))
    return fail(msg, KVE_EINVAL, "K/V too large");
  *max_len = mx;
  *T = tot;
  return KVE_OK;
}

}  // namespace

kve_status plan_score(const kve_layout* L, ScoreGeom* G, std::string* msg) {
  int max_len = 0;
  int64_t T = 0;
  kve_status st = check_layout(L, msg, &max_len, &T);
  if (st != KVE_OK) return st;
  for (int s = 0; s < L->S; ++s) {
    if (L->seq_off_host[s + 1] - L->seq_off_host[s] < L->w)
      return fail(msg, KVE_EINVAL, "every sequence needs at least w tokens");
  }
  ScoreGeom g{};
  g.S = L->S; g.Hq = L->Hq; g.Hkv = L->Hkv; g.d = L->d; g.w = L->w;
  g.T = static_cast<int>(T); g.dtype = L->dtype; g.max_len = max_len;
  g.R = (L->Hq / L->Hkv) * L->w;
  g.RG = (g.R + 127) / 128;
  const int64_t work = static_cast<int64_t>(T) * g.Hkv * g.RG;
  const int64_t len_cap = ((max_len + 255) / 256) * 256;
  int64_t ch;
  if (L->dtype == KVE_BF16) {
    // about two 4-wave workgroups per CU (512), multiple of 256 keys, at most
    // kScoreChunkMax
    ch = (work + 511) / 512;
    ch = std::max<int64_t>(256, ((ch + 255) / 256) * 256);
    ch = std::min<int64_t>(ch, kScoreChunkMax);
  } else {
    // about 512 workgroups over the batch, multiple of 256 keys
    ch = (work + 511) / 512;
    ch = std::max<int64_t>(256, ((ch + 255) / 256) * 256);
  }
  g.CH = static_cast<int>(std::min<int64_t>(ch, len_cap));
  g.P = (max_len + g.CH - 1) / g.CH;
  g.pool_rg = (L->dtype == KVE_BF16) ? g.RG : 1;
  const size_t groups = static_cast<size_t>(g.S) * g.Hkv * g.RG;
  size_t off = 0;
  g.off_part_ml = off; off = align256(off + groups * g.P * 128 * kScoreRec * sizeof(float));
  g.off_part_e = off;  off = align256(off + groups * g.P * 128 * sizeof(float));
  g.off_part_x = off;  off = align256(off + groups * g.P * 128 * sizeof(float));
  g.off_part_o = off;  off = align256(off + groups * g.P * 128 * static_cast<size_t>(g.d) * sizeof(float));
  g.off_vnorm = off;   off = align256(off + static_cast<size_t>(g.Hkv) * g.T * sizeof(float));
  g.off_lse2 = off;    off = align256(off + groups * 128 * sizeof(float));
  g.off_no2 = off;     off = align256(off + groups * 128 * sizeof(float));
  g.off_no2d = off;    off = align256(off + groups * 128 * sizeof(float));
  // bf16: hi/lo planes of -2o; fp32: o itself (stored in the "hi" region)
  const size_t oel = (L->dtype == KVE_BF16) ? 2 : 4;
  g.off_ohi = off;     off = align256(off + groups * 128 * static_cast<size_t>(g.d) * oel);
  g.off_olo = off;     off = align256(off + groups * 128 * static_cast<size_t>(g.d) * 2);
  g.off_sraw = off;    off = align256(off + static_cast<size_t>(g.pool_rg) * g.Hkv * g.T * sizeof(float));
  g.off_jstar = off;   off = align256(off + groups * 128 * sizeof(int32_t));
  g.off_cstar = off;   off = align256(off + groups * 128 * sizeof(float));
  g.bytes = off;
  *G = g;
  return KVE_OK;
}

kve_status plan_select(const kve_layout* L, const int32_t* bud_off_host, int mode, SelectGeom* G,
                       std::string* msg) {
  int max_len = 0;
  int64_t T = 0;
  kve_status st = check_layout(L, msg, &max_len, &T);
  if (st != KVE_OK) return st;
  if (mode != KVE_TOPK && mode != KVE_SAMPLE) return fail(msg, KVE_EINVAL, "unknown selection mode");
  if (!bud_off_host) return fail(msg, KVE_EINVAL, "bud_off_host is NULL");
  if (bud_off_host[0] != 0) return fail(msg, KVE_EINVAL, "bud_off[0] must be 0");
  for (int s = 0; s < L->S; ++s) {
    const int64_t B = static_cast<int64_t>(bud_off_host[s + 1]) - bud_off_host[s];
    const int64_t n = static_cast<int64_t>(L->seq_off_host[s + 1]) - L->seq_off_host[s];
    if (B < 0) return fail(msg, KVE_EINVAL, "budget offsets must be non-decreasing");
    if (B > n) return fail(msg, KVE_EINVAL, "budget B_s exceeds the sequence length n_s");
  }
  SelectGeom g{};
  g.S = L->S; g.Hkv = L->Hkv; g.T = static_cast<int>(T); g.max_len = max_len; g.mode = mode;
  g.total_B = bud_off_host[L->S];
  g.nchunk = (max_len + kSelChunk - 1) / kSelChunk;
  g.nsmp = (max_len + kSmpChunk - 1) / kSmpChunk;
  const bool smp = mode == KVE_SAMPLE;
  const size_t SH = static_cast<size_t>(g.S) * g.Hkv;
  const size_t plane = smp ? static_cast<size_t>(g.Hkv) * g.T * sizeof(double) : 0;
  const int levels = smp ? kSelLevels64 : kSelLevels32;
  size_t off = 0;
  g.off_a = off; off = align256(off + plane);
  g.off_b = off; off = align256(off + plane);
  g.off_hist = off; off = align256(off + levels * SH * kSelBins * sizeof(int32_t));
  g.zero_end = off;
  g.off_cand = off; off = align256(off + SH * g.nchunk * static_cast<size_t>(kSelChunk) * sizeof(int32_t));
  g.off_cnt = off; off = align256(off + SH * g.nchunk * 2 * sizeof(int32_t));
  g.off_rstate = off; off = align256(off + SH * kSelRStateBytes);
  g.off_rcache = off; off = align256(off + SH * kSelLevels64 * kSelRCacheBytes);
  g.off_part = off; off = align256(off + (smp ? 2 * SH * g.nsmp * 3 * sizeof(double) : 0));
  g.off_grid = off; off = align256(off + (smp ? SH * g.nsmp * kSelGrid * sizeof(float) : 0));
  g.off_state = off; off = align256(off + (smp ? 2 * SH * kSelSearchBytes : 0));
  g.off_mvals = off; off = align256(off + (smp ? SH * sizeof(double) : 0));
  g.off_bsh = off; off = align256(off + (smp ? SH * sizeof(int32_t) : 0));
  g.bytes = off;
  *G = g;
  return KVE_OK;
}

kve_status plan_merge(const kve_layout* L, const int32_t* bud_off_host, MergeGeom* G, std::string* msg) {
  int max_len = 0;
  int64_t T = 0;
  kve_status st = check_layout(L, msg, &max_len, &T);
  if (st != KVE_OK) return st;
  if (L->dtype != KVE_BF16 || L->d != 128) return fail(msg, KVE_ENOTSUP, "the merge supports bf16 keys with d = 128");
  if (!bud_off_host) return fail(msg, KVE_EINVAL, "bud_off_host is NULL");
  if (bud_off_host[0] != 0) return fail(msg, KVE_EINVAL, "bud_off[0] must be 0");
  int maxB = 0;
  for (int s = 0; s < L->S; ++s) {
    const int64_t B = static_cast<int64_t>(bud_off_host[s + 1]) - bud_off_host[s];
    const int64_t n = static_cast<int64_t>(L->seq_off_host[s + 1]) - L->seq_off_host[s];
    if (B < 0 || B > n) return fail(msg, KVE_EINVAL, "budget B_s must be in [0, n_s]");
    maxB = B > maxB ? static_cast<int>(B) : maxB;
  }
  MergeGeom g{};
  g.S = L->S; g.Hkv = L->Hkv; g.T = static_cast<int>(T); g.max_len = max_len; g.maxB = maxB;
  g.totalB = bud_off_host[L->S];
  const size_t plane = static_cast<size_t>(g.Hkv) * g.T;
  size_t off = 0;
  g.off_invn = off; off = align256(off + plane * sizeof(float));
  g.off_flag = off; off = align256(off + plane * sizeof(int32_t));
  g.off_best = off; off = align256(off + plane * sizeof(uint64_t));
  g.off_cnt = off; off = align256(off + static_cast<size_t>(g.Hkv) * g.totalB * sizeof(int32_t));
  g.bytes = off;
  *G = g;
  return KVE_OK;
}

kve_status plan_literal(const kve_layout* L, LiteralGeom* G, std::string* msg) {
  int max_len = 0;
  int64_t T = 0;
  kve_status st = check_layout(L, msg, &max_len, &T);
  if (st != KVE_OK) return st;
  if (max_len > kLitMaxLen) return fail(msg, KVE_ENOTSUP, "literal draws support n_s <= 4194304");
  LiteralGeom g{};
  g.S = L->S; g.Hkv = L->Hkv; g.T = static_cast<int>(T);
  g.nch = (max_len + kSmpChunk - 1) / kSmpChunk;
  const size_t SH = static_cast<size_t>(g.S) * g.Hkv;
  const size_t plane = static_cast<size_t>(g.Hkv) * g.T;
  size_t off = 0;
  g.off_part = off; off = align256(off + SH * g.nch * 2 * sizeof(double));
  g.off_pi = off; off = align256(off + plane * sizeof(double));
  g.off_cdf = off; off = align256(off + plane * sizeof(double));
  g.off_cnt = off; off = align256(off + plane * sizeof(int32_t));
  g.off_nz = off; off = align256(off + SH * g.nch * sizeof(int32_t));
  g.bytes = off;
  *G = g;
  return KVE_OK;
}

kve_status check_compact(const kve_layout* L, const int32_t* bud_off_host, const int32_t* cap_off_host,
                         std::string* msg) {
  int max_len = 0;
  int64_t T = 0;
  kve_status st = check_layout(L, msg, &max_len, &T);
  if (st != KVE_OK) return st;
  if (!bud_off_host || !cap_off_host) return fail(msg, KVE_EINVAL, "bud_off_host / cap_off_host is NULL");
  if (bud_off_host[0] != 0 || cap_off_host[0] != 0) return fail(msg, KVE_EINVAL, "offsets must start at 0");
  for (int s = 0; s < L->S; ++s) {
    const int64_t B = static_cast<int64_t>(bud_off_host[s + 1]) - bud_off_host[s];
    const int64_t C = static_cast<int64_t>(cap_off_host[s + 1]) - cap_off_host[s];
    const int64_t n = static_cast<int64_t>(L->seq_off_host[s + 1]) - L->seq_off_host[s];
    if (B < 0 || B > n) return fail(msg, KVE_EINVAL, "budget B_s must be in [0, n_s]");
    if (C < B) return fail(msg, KVE_EINVAL, "capacity cap_s must be >= B_s");
  }
  return KVE_OK;
}

kve_status plan_decode(const kve_layout* L, const int32_t* cap_off_host, int max_cache_len,
                       DecodeGeom* G, std::string* msg) {
  if (!L) return fail(msg, KVE_EINVAL, "layout is NULL");
  if (L->S < 1 || L->Hq < 1 || L->Hkv < 1 || L->Hq % L->Hkv)
    return fail(msg, KVE_EINVAL, "bad S / Hq / Hkv");
  if (L->dtype != KVE_BF16 && L->dtype != KVE_F32) return fail(msg, KVE_EINVAL, "unknown dtype");
  if (L->d != 64 && L->d != 128) return fail(msg, KVE_ENOTSUP, "decode supports d in {64, 128}");
  if (L->Hq / L->Hkv > 16) return fail(msg, KVE_ENOTSUP, "decode supports at most 16 q-heads per KV head");
  if (max_cache_len < 1) return fail(msg, KVE_EINVAL, "max_cache_len must be >= 1");
  if (cap_off_host) {   // NULL: sizing only
    if (cap_off_host[0] != 0) return fail(msg, KVE_EINVAL, "cap_off[0] must be 0");
    int64_t maxcap = 0;
    for (int s = 0; s < L->S; ++s) {
      const int64_t C = static_cast<int64_t>(cap_off_host[s + 1]) - cap_off_host[s];
      if (C < 0) return fail(msg, KVE_EINVAL, "capacity offsets must be non-decreasing");
      maxcap = std::max(maxcap, C);
    }
    if (max_cache_len > maxcap) return fail(msg, KVE_EINVAL, "max_cache_len exceeds every capacity");
  }
  DecodeGeom g{};
  g.S = L->S; g.Hq = L->Hq; g.Hkv = L->Hkv; g.d = L->d; g.dtype = L->dtype;
  int64_t len;
  if (g.dtype == KVE_BF16) {
    // fixed chunks: workgroups scale with the cache, short sequences take few
    len = kDecodeChunkBf16;
  } else {
    // split-K over the cache: about 256 workgroups, >= 64 entries each
    const int64_t heads = static_cast<int64_t>(g.S) * g.Hkv;
    const int64_t splits = std::max<int64_t>(1, (256 + heads - 1) / heads);
    len = (max_cache_len + splits - 1) / splits;
    len = std::max<int64_t>(64, ((len + 63) / 64) * 64);
  }
  g.split_len = static_cast<int>(len);
  g.splits = static_cast<int>((max_cache_len + len - 1) / len);
  const size_t rows = static_cast<size_t>(g.S) * g.Hq * g.splits;
  size_t off = 0;
  g.off_ml = off; off = align256(off + rows * 2 * sizeof(float));
  g.off_o = off;  off = align256(off + rows * static_cast<size_t>(g.d) * sizeof(float));
  g.off_app = off; off = align256(off + static_cast<size_t>(g.S) * 2 * sizeof(int32_t));
  g.bytes = off;
  *G = g;
  return KVE_OK;
}

}  // namespace kve
