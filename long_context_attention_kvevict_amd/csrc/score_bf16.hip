// Two-pass fused eviction scorer, bf16 inputs, gfx950 MFMA.
//
// Pass 1 (score_p1_bf16): flash-style online softmax of every window row of a
//   GQA group against one chunk of keys, producing per-chunk (max, sum, o)
//   partials, plus ||v_j||^2 for pass 2.  ("DropKV" page, §3.4: a
//   FlashAttention-2 style forward pass yields each row's log-sum-exp and
//   output; split-K partials are merged afterwards.)
// Merge (score_merge): combines the chunk partials of each row into its
//   log2-sum-exp, ||o||^2 and a bf16 hi/lo split of -2 o.
// Pass 2 (score_p2_bf16): recomputes the logits, forms the softmax weight
//   p = 2^(x - lse2), the distance ||o - v||^2 = ||o||^2 + ||v||^2 - 2 <o, v>
//   with <o, v> from an MFMA contraction, and accumulates
//   (p / (1 - p))^2 ||o - v||^2 over all rows of the group for each key
//   ("DropKV" page, §3.3 window score and §3.4 scoring kernel).
//
// Work decomposition of both passes: one workgroup of 4 waves per
// (sequence, KV head, group of 128 window rows, chunk of keys), sized so the
// launch is about two workgroups per CU; the two run independently, so one's
// MFMA phase overlaps the other's vector-ALU phase.  K and V stream through a
// 2-stage LDS ring of 64-key tiles filled by direct global->LDS loads (no
// register staging): the next tile is in flight while one is consumed.  Wave
// w owns rows 32w..32w+31 and both 32-key halves of each tile.  Rows of a tile
// are stored unpadded with a 16-byte-chunk XOR swizzle (see swz), which keeps
// the MFMA operand reads and the transposing reads free of bank conflicts.
// Pass 1 reads V^T operands with the transposing LDS read, so V keeps its
// natural [key][d] layout in LDS as well.
#include "common.h"
#include "launch.h"
#include "timing.h"

#include <type_traits>

namespace kve {

constexpr int D = 128;          // head dim of the bf16 path
constexpr int KT = 64;          // keys per tile (one ring stage)
constexpr int NSTAGE = 2;       // ring stages
constexpr int ROWS = 128;       // window rows per workgroup
constexpr int WG = 256;         // threads per workgroup (4 waves)
constexpr int ROWB = D * 2;     // bytes per K/V row
constexpr int TILE_BYTES = KT * ROWB;          // one K (or V) tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;    // K tile then V tile
static_assert(kScoreChunkMax % KT == 0, "chunk bound must be a multiple of the tile");
static_assert(kScoreChunkMax / KT <= 32, "pass 2 marks a chunk's tiles in a 32-bit mask");

// Slot s of a 32-key block holds key keymap(s): bits 2 and 3 swapped.  With
// this order the P values a lane holds after the K.Q^T MFMA are 8
// consecutive keys, matching the k-slices of the P.V contraction.
__device__ __forceinline__ int keymap(int s) {
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}

// Key (within a 32-key block) of accumulator register r of lane half hl in
// the K.Q^T output (slot 8(r/4) + 4hl + r%4 mapped through keymap).
__device__ __forceinline__ int p1_key_of(int r, int hl) {
  return (r & 3) + 4 * ((r >> 2) & 1) + 8 * hl + 16 * (r >> 3);
}

// Chunk swizzle of a tile row: chunk c of key k is stored at chunk c ^ swz(k),
// with key bits b3..b0 mapped to swz = (b1, b0, b1^b3, b2^b3).  The 16-byte
// reads of one chunk (MFMA operands, ||v||^2) hit distinct slots whether the
// LDS serves 8 or 16 lanes per cycle, for 16 consecutive keys and for pass
// 1's keymap order alike: swz is a permutation of the 16 residues of k, and
// eight consecutive keys, or keymap(0..7), keymap(8..15), differ mod 8.  The
// transposing 8-byte reads of pass 1 touch four keys 4a..4a+3 at chunks
// 4m..4m+3 per 32 lanes; the four keys have distinct swz >> 2, so those 16
// chunks are distinct too (and, per 16 lanes, chunk pairs 2m, 2m+1 of the
// four keys, distinct by swz >> 1).
__device__ __forceinline__ int swz(int key) {
  return ((key & 3) << 2) | ((((key >> 1) ^ (key >> 3)) & 1) << 1) | (((key >> 2) ^ (key >> 3)) & 1);
}
// Byte offset of 16-byte chunk c of row `key` inside a swizzled tile.
__device__ __forceinline__ int tile_off(int key, int c) { return key * ROWB + ((c ^ swz(key)) << 4); }

struct ScoreArgs {
  const uint16_t* q_win;   // [S][Hq][w][D]
  const uint16_t* k;       // [Hkv][T][D]
  const uint16_t* v;
  const int32_t* seq_off;  // [S+1]
  int S, Hq, Hkv, w, T, RG, CH, P, causal;
  float c2;                // sm_scale * log2(e)
  float* part_ml;          // [S*Hkv*RG][P][ROWS][kScoreRec]
  float* part_e;           // [S*Hkv*RG][P][ROWS] rounding error of the candidate's weight
  float* part_x;           // [S*Hkv*RG][P][ROWS] largest logit of the row in the chunk (log2 units)
  float* part_o;           // [S*Hkv*RG][P][ROWS][D]
  float* vnorm;            // [Hkv][T]
  float* lse2;             // [S*Hkv*RG][ROWS]
  float* no2;              // [S*Hkv*RG][ROWS]  ||o_h||^2 of the bf16-rounded output o_h = -ohi / 2
  float* no2d;             // [S*Hkv*RG][ROWS]  ||o||^2 - ||o_h||^2 (used with the residual plane)
  uint16_t* ohi;           // [S*Hkv*RG][ROWS][D]  bf16 of -2 o
  uint16_t* olo;           // residual
  float* sraw;             // [RG][Hkv][T]
  int32_t* jstar;          // [S*Hkv*RG][ROWS]  key holding over half of the row's weight, or -1
  float* cstar;            // [S*Hkv*RG][ROWS]  that pair's exact term (a / (1 - a))^2 ||o - v||^2
  ScoreZero zero;          // cleared by the merge launch (p = NULL: nothing)
};

// Work item of a workgroup of either pass.  The RG row groups of one
// (sequence, KV head, key chunk) read the same K/V tiles, so their
// workgroups get consecutive dispatch slots on one XCD (workgroups are dealt
// to the 8 XCDs round-robin by linear id): tiles that one of them brings into
// that XCD's L2 serve the others.  Grid: 8 * ceil(S*Hkv*P / 8) * RG.
struct ScoreWork {
  int s, h, rg, c;
};
__device__ __forceinline__ bool score_work(const ScoreArgs& a, int lin, ScoreWork* w) {
  const int xcd = lin & 7, slot = lin >> 3;
  const int item = (slot / a.RG) * 8 + xcd;   // (s, h, c), chunk fastest
  w->rg = slot % a.RG;
  w->c = item % a.P;
  w->h = (item / a.P) % a.Hkv;
  w->s = item / (a.P * a.Hkv);
  return w->s < a.S;
}

// ------------------------------------------------------------ LDS pipeline
// Workgroup barrier that orders LDS traffic only: global->LDS loads stay in
// flight across it (a full __syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits until at most N of this wave's vector-memory operations are
// outstanding.  They complete in issue order, so every earlier one is done.
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// 16 bytes per lane from `gptr` into LDS at lds_base + 16 * lane (one 1 KiB
// block per wave).  Issued from inline assembly so that the compiler's own
// wait insertion, which cannot tell the ring stages apart, does not drain
// the whole pipeline before every LDS read; the kernels wait explicitly.
// NT: non-temporal (streaming) cache policy, for tiles no other workgroup
// reads.
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" :: "v"(gptr), "s"(lds_base) : "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(gptr), "s"(lds_base) : "memory");
}

// Makes the register operand `x` ready here: the compiler places its wait for
// the load that produced it before this point (outside the tile loop), so it
// never emits a drain of the whole vector-memory counter inside the loop.
template <typename T>
__device__ __forceinline__ void settle(const T& x) { asm volatile("" :: "v"(x)); }

// v + (the value lane l ^ 32 holds), through the cross-half lane swap
// (no LDS round trip).
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// The values lanes l % 32 and l % 32 + 32 hold, in that order, on both.
__device__ __forceinline__ void halves(uint32_t v, uint32_t* h0, uint32_t* h1) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  *h0 = r[0];
  *h1 = r[1];
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Per-lane constants of the ring fill.  Wave w loads tile rows 8w .. 8w+7:
// two 1 KiB LDS blocks of K and two of V (rows 4j .. 4j+3 for j = 2w, 2w+1),
// four 16-byte loads per lane per tile.
struct RingFill {
  static constexpr int NB = TILE_BYTES / 1024 / (WG / 64);   // 1 KiB blocks per wave and tile
  int key[NB];        // tile row loaded by this lane in block i
  int goff[NB];       // byte offset of that row's chunk from the tile's first row
  uint32_t lds[NB];   // LDS byte address of block i in stage 0 (wave-uniform)

  __device__ void init(uint32_t ring0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = NB * wave + i;               // block j holds rows 4j .. 4j+3
      key[i] = 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ swz(key[i]);   // logical chunk stored at this lane's slot
      goff[i] = key[i] * ROWB + 16 * c;
      lds[i] = __builtin_amdgcn_readfirstlane(ring0 + j * 1024);
    }
  }
  // Keys kt0 .. kt0+63 into stage `stage`; rows past the chunk end c1 repeat
  // its last key (callers mask them).
  template <bool NT = false>
  __device__ __forceinline__ void issue(const char* kb, const char* vb, int kt0, int c1, int stage) const {
    const size_t tbase = static_cast<size_t>(kt0) * ROWB;
    const uint32_t sb = static_cast<uint32_t>(stage) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      int off = goff[i];
      if (kt0 + KT > c1 && kt0 + key[i] >= c1) off += (c1 - 1 - kt0 - key[i]) * ROWB;
      dma16<NT>(kb + tbase + off, lds[i] + sb);
      dma16<NT>(vb + tbase + off, lds[i] + sb + TILE_BYTES);
    }
  }
  // K rows only, into stages of TILE_BYTES (the attention-weight scores).
  template <bool NT = false>
  __device__ __forceinline__ void issue_k(const char* kb, int kt0, int c1, int stage) const {
    const size_t tbase = static_cast<size_t>(kt0) * ROWB;
    const uint32_t sb = static_cast<uint32_t>(stage) * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      int off = goff[i];
      if (kt0 + KT > c1 && kt0 + key[i] >= c1) off += (c1 - 1 - kt0 - key[i]) * ROWB;
      dma16<NT>(kb + tbase + off, lds[i] + sb);
    }
  }
};

// Sum of squares of 16 bf16 values (two 16-byte chunks).
__device__ __forceinline__ float sumsq16(u32x4 x, u32x4 y) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = __uint_as_float(x[e] << 16), a1 = __uint_as_float(x[e] & 0xffff0000u);
    const float b0 = __uint_as_float(y[e] << 16), b1 = __uint_as_float(y[e] & 0xffff0000u);
    acc = fmaf(a0, a0, acc);
    acc = fmaf(a1, a1, acc);
    acc = fmaf(b0, b0, acc);
    acc = fmaf(b1, b1, acc);
  }
  return acc;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- pass 1
__global__ __launch_bounds__(WG, 2) void score_p1_bf16(ScoreArgs a) {
  ScoreWork wk;
  if (!score_work(a, blockIdx.x, &wk)) return;
  const int c = wk.c, h = wk.h, rg = wk.rg, s = wk.s;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int c0 = c * a.CH;
  if (c0 >= n) return;
  const int c1 = min(c0 + a.CH, n);

  __shared__ __align__(1024) char ring[NSTAGE * STAGE_BYTES];
  __shared__ __align__(16) float vn[kScoreChunkMax];
  // per lane: candidate key, its weight's rounding error, and l_run before
  // the current tile (kept out of registers; only rare paths read them)
  __shared__ int cand_j[WG];
  __shared__ float cand_e[WG], cand_lb[WG];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int g = a.Hq / a.Hkv;
  const int R = g * a.w;

  // this lane's query row (N index of the K.Q^T MFMA)
  const int row = rg * ROWS + wave * 32 + col;
  const bool row_ok = row < R;
  // A wave of the last row group can hold no window row (R not a multiple
  // of 128, e.g. 7 query heads x 64 rows): it still loads its share of the
  // tiles (and in row group 0 forms its keys' ||v||^2, which the other row
  // groups of the chunk leave to that one), but skips the attention
  // arithmetic.
  const bool wave_rows = __builtin_amdgcn_readfirstlane(rg * ROWS + wave * 32 < R ? 1 : 0) != 0;
  const int qh = h * g + (row_ok ? row / a.w : 0);
  const int wi = row_ok ? row % a.w : 0;
  const int pos = n - a.w + wi;   // causal horizon of this row

  bf16x8 qreg[D / 16];
  {
    const uint16_t* qp = a.q_win + ((static_cast<size_t>(s) * a.Hq + qh) * a.w + wi) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (row_ok) t = *reinterpret_cast<const u32x4*>(qp + 16 * kk + 8 * hl);
      qreg[kk] = as_bf16x8(t);
    }
  }
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) settle(qreg[kk]);

  const char* kb8 = reinterpret_cast<const char*>(a.k + (static_cast<size_t>(h) * a.T + base) * D);
  const char* vb8 = reinterpret_cast<const char*>(a.v + (static_cast<size_t>(h) * a.T + base) * D);
  RingFill fill;
  fill.init(lds_addr(ring), wave, lane);
  const int ntile = (c1 - c0 + KT - 1) / KT;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  // Online softmax with a lazily raised reference: p = 2^(x - m_run) with
  // m_run within 8 of the running max, so p <= 256 and the accumulators are
  // rescaled only when the max climbs by more than 8 (log2 units).
  float m_run = -INFINITY;
  float l_run = 0.f;
  // A key can hold over half of its row's final weight only if, on its
  // tile, its weight exceeds half of the row's running sum; such tiles take
  // the residual branch below, which makes this lane's largest weight of the
  // tile the lane's candidate when it exceeds the recorded one.  The
  // candidate's weight pc is kept out of l_run (so the sum of the other
  // keys, 1 - a up to the row sum, carries no cancellation), together with
  // its key (cand_j) and the rounding error (cand_e) of the weight P.V used
  // for it.
  float pc = 0.f;
  float cmax = -INFINITY;   // the row's largest logit in the chunk, log2 units
  cand_j[tid] = -1;
  cand_e[tid] = 0.f;

  // loop-invariant LDS offsets (the second 32-key half adds 32 rows = 8 KiB;
  // the swizzle depends on the row mod 16 only)
  int koff[D / 16];
  {
    const int krow = keymap(col);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) koff[kk] = tile_off(krow, 2 * kk + hl);
  }
  // ||v||^2 of tile keys 16*wave .. +15 as the diagonal of the Gram block
  // V V^T (16x16x32 MFMA, one operand register serving as A and B): lane l
  // reads key 16*wave + l%16, chunk 4j + l/16 for k-step j.  The diagonal
  // element of key l%16 sits in register l%4 of the lanes with
  // (l%16)/4 == l/16.
  const int gkey = 16 * wave + (lane & 15);
  int goffv[D / 32];
#pragma unroll
  for (int j = 0; j < D / 32; ++j) goffv[j] = tile_off(gkey, 4 * j + (lane >> 4));
  const bool gdiag = ((lane & 15) >> 2) == (lane >> 4);
  // A operand of O^T += V^T P^T: lane (d = db*32 + l%32, k-slice l/32) holds 8
  // consecutive keys of feature d, from two transposing reads; in each
  // 16-lane group lane j names row key0 + j/4 at features dbase + 4(j%4)..+4
  // and receives feature dbase + j of rows key0 .. key0+3.  Feature block db
  // toggles offset bits 6-7 (XOR db << 6).
  int toff[2][2];
  {
    const int grpl = lane >> 4, j = lane & 15;
    const int dl = 16 * (grpl & 1) + 4 * (j & 3);   // feature within a 32-block
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key0 = 16 * k2 + 8 * (grpl >> 1) + 4 * hf + (j >> 2);
        toff[k2][hf] = tile_off(key0, dl >> 3) + ((dl >> 2) & 1) * 8;
      }
    }
  }
  const bool causal = a.causal != 0;

  if (ntile > 0) fill.issue(kb8, vb8, c0, c1, 0);

  // One tile; EDGE tiles reach past the chunk end or the earliest causal
  // horizon and mask keys, interior tiles carry no masking code.
  auto tile = [&](const int t, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int kt0 = c0 + t * KT;
    const char* Kt = ring + (t & 1) * STAGE_BYTES;
    const char* Vt = Kt + TILE_BYTES;
    if (rg == 0) {   // one row group forms the tile's ||v||^2
      f32x4 gram = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 32; ++j) {
        const bf16x8 x = as_bf16x8(*reinterpret_cast<const u32x4*>(Vt + goffv[j]));
        gram = mfma16(x, x, gram);
      }
      if (gdiag) vn[t * KT + gkey] = gram[lane & 3];
    }
    if (!wave_rows) return;   // no window row in this wave (last row group)
    // S^T = K . Q^T for both 32-key halves (slot order through keymap)
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4*>(Kt + kb * 32 * ROWB + koff[kk]));
        sacc[kb] = mfma32(av, qreg[kk], sacc[kb]);
      }
    }
    if constexpr (EDGE) {   // keys past the chunk or the causal horizon
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + kb * 32 + p1_key_of(r, hl);
          const bool hidden = (key >= c1) | (causal & (key > pos));
          sacc[kb][r] = hidden ? -INFINITY : sacc[kb][r];
        }
      }
    }
    float tmax = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(sacc[0][r], sacc[1][r]));
    tmax = max_xor32(tmax) * a.c2;
    cmax = fmaxf(cmax, tmax);
    const bool raise = tmax > m_run + 8.f;
    if (__any(raise)) {
      const float m_new = raise ? tmax : m_run;
      const float scale = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= scale;
      l_run *= scale;
      pc *= scale;
      cand_e[tid] *= scale;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    cand_lb[tid] = l_run;

    f32x8 pf[2][2];
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[kb][k2][e] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * k2 + e], a.c2, -m_use));
          l_run += pf[kb][k2][e];
        }
        pb[kb][k2] = __builtin_convertvector(pf[kb][k2], bf16x8);   // round to nearest even
      }
    }
    // O^T += V^T . P^T
    auto pv = [&](const bf16x8 (&pm)[2][2]) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const char* vbase = Vt + kb * 32 * ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vbase + (toff[k2][0] ^ (db << 6))));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vbase + (toff[k2][1] ^ (db << 6))));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = mfma32(__builtin_bit_cast(bf16x8, av), pm[kb][k2], oacc[db]);
          }
        }
      }
    };
    // the P.V contraction at raised wave priority: the matrix cores take the
    // MFMAs of this wave while the other wave on the SIMD does its softmax
    __builtin_amdgcn_s_setprio(1);
    pv(pb);
    __builtin_amdgcn_s_setprio(0);
    // A dominant weight is where the bf16 rounding of P matters: it moves o
    // by 2^-9 a v_j for a key of final weight a, against ||o - v_j|| of about
    // (1 - a) ||v_j||.  The running sum of the row (this lane's half plus its
    // partner's) is a lower bound on its final sum, so a tile whose weights
    // all stay within half of it has
    // a <= 1/2 for every key and the rounding moves ||o - v_j||^2 by at most
    // 2^-9 * 2 relative (0.39 %).  Tiles with a larger weight also contract
    // the rounding residual of P, which makes the weights exact to about
    // 2^-17.  (Early tiles of a chunk, where the running sum is still small,
    // are the ones that take this path.)
    const float pmax = __builtin_amdgcn_exp2f(tmax - m_use);
    if (__any(2.f * pmax > sum_xor32(l_run + pc))) {
      float pm = 0.f;   // this lane's largest weight of the tile
#pragma unroll
      for (int i = 0; i < 32; ++i) pm = fmaxf(pm, pf[i >> 4][(i >> 3) & 1][i & 7]);
      if (pm > pc) {
        // new candidate: the first of this lane's keys (in key order) with
        // that weight; the previous one joins the other keys
        int eb = 0;
#pragma unroll
        for (int i = 31; i >= 0; --i) eb = (pf[i >> 4][(i >> 3) & 1][i & 7] == pm) ? i : eb;
        float lsum = cand_lb[tid] + pc;
#pragma unroll
        for (int i = 0; i < 32; ++i) lsum += (i == eb) ? 0.f : pf[i >> 4][(i >> 3) & 1][i & 7];
        // P.V used its weight as the bf16 value plus the bf16 residual,
        // formed exactly as above
        const float wh = static_cast<float>(static_cast<__bf16>(pm));
        const float wl = static_cast<float>(static_cast<__bf16>(pm - wh));
        l_run = lsum;
        pc = pm;
        cand_e[tid] = (wh + wl) - pm;
        cand_j[tid] = kt0 + (eb >> 4) * 32 + p1_key_of(eb & 15, hl);
      }
      bf16x8 pr[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          f32x8 rem = pf[kb][k2];
          // keeps the residual arithmetic inside this rarely taken branch
          asm volatile("" : "+v"(rem));
#pragma unroll
          for (int e = 0; e < 8; ++e) rem[e] -= static_cast<float>(pb[kb][k2][e]);
          pr[kb][k2] = __builtin_convertvector(rem, bf16x8);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      pv(pr);
    }
  };

  const int edge_from = causal ? min(c1 - KT, n - a.w - KT + 1) : c1 - KT;   // first key of an edge tile
  for (int t = 0; t < ntile; ++t) {
    wait_vm<0>();    // this lane's loads of tile t
    lds_barrier();   // everyone's loads of tile t; the other stage is free
    if (t + 1 < ntile) fill.issue(kb8, vb8, c0 + (t + 1) * KT, c1, (t + 1) & 1);
    if (c0 + t * KT > edge_from) tile(t, std::true_type{});
    else tile(t, std::false_type{});
  }
  lds_barrier();   // vn complete

  // ||v||^2 of the chunk
  if (rg == 0)
    for (int i = tid; i < c1 - c0; i += WG) a.vnorm[static_cast<size_t>(h) * a.T + base + c0 + i] = vn[i];

  // The row's candidate is the larger weight of its two halves' (the lower
  // key on equal weights); the other half's candidate joins the other keys.
  uint32_t p0, p1, e0, e1, j0, j1, l0, l1;
  halves(__float_as_uint(pc), &p0, &p1);
  halves(__float_as_uint(cand_e[tid]), &e0, &e1);
  halves(static_cast<uint32_t>(cand_j[tid]), &j0, &j1);
  halves(__float_as_uint(l_run), &l0, &l1);
  if (!row_ok) return;
  const size_t part = (static_cast<size_t>((s * a.Hkv + h) * a.RG + rg)) * a.P + c;
  const int rl = wave * 32 + col;
  if (hl == 0) {
    const float pa = __uint_as_float(p0), pb = __uint_as_float(p1);
    const bool first = (pa > pb) || (pa == pb && static_cast<int>(j0) <= static_cast<int>(j1));
    const float lo = (__uint_as_float(l0) + __uint_as_float(l1)) + (first ? pb : pa);
    *reinterpret_cast<f32x4*>(a.part_ml + (part * ROWS + rl) * kScoreRec) =
        f32x4{m_run, lo, first ? pa : pb, __uint_as_float(first ? j0 : j1)};
    a.part_e[part * ROWS + rl] = __uint_as_float(first ? e0 : e1);
    a.part_x[part * ROWS + rl] = cmax;
  }
  float* op = a.part_o + (part * ROWS + rl) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = db * 32 + 8 * q4 + 4 * hl;
      *reinterpret_cast<f32x4*>(op + d) =
          f32x4{oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]};
    }
  }
}

// ---------------------------------------------------------------- merge
// One workgroup per window row: NSTR streams of 32 lanes take every
// NSTR-th chunk (lane = DD/32 consecutive features), then combine through
// LDS in a fixed order.  Chunks wholly beyond a row's causal horizon carry max = -inf and
// weight 0.
//
// A row whose best candidate key (largest weight over the chunks'
// candidates, the lower key on equal weights) holds over half of the row's weight takes
// the exact form of its term ("DropKV" page, §3.2: the perturbation of
// dropping one key is a / (1 - a) ||o - v_j||): 1 - a is the summed weight
// of every other key, o loses the rounding error of the candidate's weight,
// and ||o - v_j||^2 is summed from the explicit difference.  Any key with a
// weight above one half has the row's unique largest weight and was
// recorded as a candidate on its tile, so this covers every such row.
template <int DD, bool BF16OUT, int NSTR>
__global__ __launch_bounds__(NSTR * 32) void score_merge(ScoreArgs a, float* o32) {
  constexpr int F = DD / 32;
  constexpr int NT = NSTR * 32;   // threads: NSTR streams of 32 lanes
  static_assert(NT % 64 == 0 && NT <= 256, "whole waves, at most four");
  const int gr = blockIdx.x;   // grp * ROWS + rl
  const int grp = gr / ROWS;
  const int rl = gr % ROWS;
  const int tid = threadIdx.x;
  if (a.zero.p) {   // a later selection's counters (one-call eviction)
    const int nt = gridDim.x * NT;
    for (int i = gr * NT + tid; i < a.zero.n; i += nt) a.zero.p[i] = 0;
    for (int i = gr * NT + tid; i < a.zero.nsh; i += nt) {
      if (a.zero.m) a.zero.m[i] = 0.0;
      if (a.zero.st) a.zero.st[i] = KVE_OK;
    }
  }
  const int st = tid >> 5, ln = tid & 31;
  const int s = grp / (a.Hkv * a.RG);
  const int h = (grp / a.RG) % a.Hkv;
  const int rg = grp % a.RG;
  const int base = a.seq_off[s];
  const int n = a.seq_off[s + 1] - base;
  const int nch = (n + a.CH - 1) / a.CH;
  const int R = (a.Hq / a.Hkv) * a.w;
  const size_t ro = static_cast<size_t>(gr);
  if (rg * ROWS + rl >= R) {   // padding row of the last row group
    if (tid == 0) {
      a.lse2[ro] = INFINITY;
      a.no2[ro] = 0.f;
      if (BF16OUT) {
        a.no2d[ro] = 0.f;
        a.jstar[ro] = -1;
        a.cstar[ro] = 0.f;
      }
    }
    if (tid < 32) {
#pragma unroll
      for (int f = 0; f < F; ++f) {
        if (BF16OUT) { a.ohi[ro * DD + ln * F + f] = 0; a.olo[ro * DD + ln * F + f] = 0; }
        else o32[ro * DD + ln * F + f] = 0.f;
      }
    }
    return;
  }
  __shared__ float red_o[NSTR][DD];
  __shared__ float red_l[NSTR][4];   // others' sum, candidate weight, key, chunk
  __shared__ float red_m[NT / 64];
  const size_t cstride_ml = static_cast<size_t>(ROWS) * kScoreRec;
  const size_t cstride_o = static_cast<size_t>(ROWS) * DD;
  const float* ml = a.part_ml + (static_cast<size_t>(grp) * a.P * ROWS + rl) * kScoreRec;
  const float* po = a.part_o + (static_cast<size_t>(grp) * a.P * ROWS + rl) * DD + ln * F;
  float M = -INFINITY;
  for (int c = tid; c < nch; c += NT) M = fmaxf(M, ml[c * cstride_ml]);
  M = wave_max(M);
  if ((tid & 63) == 0) red_m[tid >> 6] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) M = fmaxf(M, red_m[w]);
  // per stream: sum of the non-candidate weights (the candidates that lose
  // to a better one included) and the best candidate (weight, key, chunk),
  // all scaled to the reference M
  float L = 0.f, cp = 0.f;
  int cj = -1, cc = 0;
  float acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = 0.f;
#pragma unroll 4
  for (int c = st; c < nch; c += NSTR) {
    const f32x4 r0 = *reinterpret_cast<const f32x4*>(ml + c * cstride_ml);
    const float m = r0[0];
    const float wgt = (m == -INFINITY) ? 0.f : exp2f(m - M);
    L = fmaf(r0[1], wgt, L);
    const int jk = static_cast<int>(__float_as_uint(r0[3]));
    const float pk = r0[2] * wgt;
    // chunks come in key order, so on equal weights the earlier key stays
    if (pk > cp) {
      L += cp;
      cp = pk; cj = jk; cc = c;
    } else {
      L += pk;
    }
    if (F == 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(po + c * cstride_o);
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = fmaf(x[f], wgt, acc[f]);
    } else {
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = fmaf(po[c * cstride_o + f], wgt, acc[f]);
    }
  }
#pragma unroll
  for (int f = 0; f < F; ++f) red_o[st][ln * F + f] = acc[f];
  if (ln == 0) {
    red_l[st][0] = L;
    red_l[st][1] = cp;
    red_l[st][2] = __uint_as_float(static_cast<uint32_t>(cj));
    red_l[st][3] = __uint_as_float(static_cast<uint32_t>(cc));
  }
  __syncthreads();
  if (tid >= 32) return;
  L = 0.f;
  cp = 0.f; cj = -1; cc = 0;
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = 0.f;
#pragma unroll
  for (int k = 0; k < NSTR; ++k) {
    L += red_l[k][0];
    const float pk = red_l[k][1];
    const int jk = static_cast<int>(__float_as_uint(red_l[k][2]));
    if (pk > cp || (pk == cp && jk >= 0 && jk < cj)) {
      L += cp;
      cp = pk; cj = jk; cc = static_cast<int>(__float_as_uint(red_l[k][3]));
    } else {
      L += pk;
    }
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] += red_o[k][ln * F + f];
  }
  const float Lt = L + cp;
  // the candidate's exact term needs its weight above half of the row's
  const bool dom = BF16OUT && cj >= 0 && 2.f * cp > Lt;
  float vs[F];
  if (dom) {
    // the candidate's rounding error, in the reference M
    const float mc = ml[cc * cstride_ml];
    const float ce = a.part_e[(static_cast<size_t>(grp) * a.P + cc) * ROWS + rl] * exp2f(mc - M);
    const uint16_t* vr = a.v + (static_cast<size_t>(h) * a.T + base + cj) * DD + ln * F;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      vs[f] = bf16_to_f32(vr[f]);
      acc[f] = fmaf(-ce, vs[f], acc[f]);
    }
  }
  const float inv = 1.f / Lt;
  float sq = 0.f, sqh = 0.f, dd = 0.f;
  uint16_t hi[F], lo[F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    acc[f] *= inv;
    sq = fmaf(acc[f], acc[f], sq);
    if (dom) {
      const float df = acc[f] - vs[f];
      dd = fmaf(df, df, dd);
    }
    if (BF16OUT) {
      const float x = -2.f * acc[f];
      hi[f] = f32_to_bf16(x);
      const float xh = bf16_to_f32(hi[f]);
      lo[f] = f32_to_bf16(x - xh);
      sqh = fmaf(0.5f * xh, 0.5f * xh, sqh);
    }
  }
  for (int o = 16; o > 0; o >>= 1) {
    sq += __shfl_xor(sq, o, 32);
    if (BF16OUT) sqh += __shfl_xor(sqh, o, 32);
    if (dom) dd += __shfl_xor(dd, o, 32);
  }
  if (ln == 0) {
    a.lse2[ro] = M + log2f(Lt);
    if (BF16OUT) {
      a.no2[ro] = sqh;
      a.no2d[ro] = sq - sqh;
      // (a / (1 - a))^2 = (cp / L)^2; a row with a single visible key
      // (L = 0) contributes nothing for it
      const float y = (L > 0.f) ? cp / L : 0.f;
      a.jstar[ro] = dom ? cj : -1;
      a.cstar[ro] = dom ? y * y * dd : 0.f;
    } else {
      a.no2[ro] = sq;
    }
  }
#pragma unroll
  for (int f = 0; f < F; ++f) {
    if (BF16OUT) {
      a.ohi[ro * DD + ln * F + f] = hi[f];
      a.olo[ro * DD + ln * F + f] = lo[f];
    } else {
      o32[ro * DD + ln * F + f] = acc[f];
    }
  }
}

// ---------------------------------------------------------------- pass 2
// A 32x32 block of (row, key) pairs whose softmax weights all stay at or
// below 2^-6 measures distances from the bf16-rounded output o_h
// alone: ||o_h - v||^2 is then exact for o_h and differs from ||o - v||^2 by
// at most about 2^-8 ||o|| / ||o - v|| relative.  With a larger weight (where
// o can approach v_j and that bound degrades) the block also contracts the
// residual plane o - o_h, restoring an fp32-accurate distance.
constexpr float kResidX = -6.f;   // log2 p above this <=> p > 2^-6

// NT: streaming loads of the tiles (one row group per chunk, so no other
// workgroup reads them).
template <bool NT>
__global__ __launch_bounds__(WG, 2) void score_p2_bf16(ScoreArgs a) {
  ScoreWork wk;
  if (!score_work(a, blockIdx.x, &wk)) return;
  // wave-uniform work indices, held in scalar registers
  const int c = __builtin_amdgcn_readfirstlane(wk.c), h = __builtin_amdgcn_readfirstlane(wk.h);
  const int rg = __builtin_amdgcn_readfirstlane(wk.rg), s = __builtin_amdgcn_readfirstlane(wk.s);
  const int base = __builtin_amdgcn_readfirstlane(a.seq_off[s]);
  const int n = __builtin_amdgcn_readfirstlane(a.seq_off[s + 1]) - base;
  const int c0 = c * a.CH;
  if (c0 >= n) return;
  const int c1 = min(c0 + a.CH, n);

  __shared__ __align__(1024) char ring[NSTAGE * STAGE_BYTES];
  __shared__ __align__(16) float sbuf[kScoreChunkMax];   // ||v||^2 in, scores out
  __shared__ __align__(16) float red[2][4][KT];
  __shared__ __align__(16) float rowc[2 * ROWS];
  __shared__ int rowhz[ROWS];   // causal horizon (last visible key) of each row
  __shared__ int rowj[ROWS];      // key with over half of the row's weight, or -1
  __shared__ float rowcs[ROWS];   // that pair's exact term
  __shared__ uint32_t dmask[WG / 64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int g = a.Hq / a.Hkv;
  const int R = g * a.w;
  const size_t grp = static_cast<size_t>((s * a.Hkv + h) * a.RG + rg);

  // A operands: rows wave*32 + col (M index)
  const int arow = rg * ROWS + wave * 32 + col;
  const bool arow_ok = arow < R;
  // a wave of the last row group with no window row loads its share of the
  // tiles but skips the arithmetic; its partials stay zero
  const bool wave_rows = __builtin_amdgcn_readfirstlane(rg * ROWS + wave * 32 < R ? 1 : 0) != 0;
  if (!wave_rows) red[0][wave][lane] = red[1][wave][lane] = 0.f;
  // Whether some row of this wave has a weight above 2^-6 in this chunk
  // (pass 1's largest logit of the row in the chunk against its log-sum-exp):
  // only then do the tiles look for such weights at all.
  const bool wave_big = __any(arow_ok && a.part_x[(grp * a.P + c) * ROWS + wave * 32 + col] -
                                             a.lse2[grp * ROWS + wave * 32 + col] > kResidX);
  bf16x8 qa[D / 16], oha[D / 16];
  {
    const int qh = h * g + (arow_ok ? arow / a.w : 0);
    const int wi = arow_ok ? arow % a.w : 0;
    const uint16_t* qp = a.q_win + ((static_cast<size_t>(s) * a.Hq + qh) * a.w + wi) * D;
    const uint16_t* hp = a.ohi + (grp * ROWS + wave * 32 + col) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (arow_ok) t = *reinterpret_cast<const u32x4*>(qp + 16 * kk + 8 * hl);
      qa[kk] = as_bf16x8(t);
      oha[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(hp + 16 * kk + 8 * hl));
    }
  }
  // per-row constants (log2-sum-exp, ||o_h||^2); register r of the output
  // layout is row 8(r/4) + 4hl + r%4 of the wave's 32
  for (int i = tid; i < ROWS; i += WG) {
    rowc[i] = a.lse2[grp * ROWS + i];
    rowc[ROWS + i] = a.no2[grp * ROWS + i];
    const int rrow = rg * ROWS + i;
    rowhz[i] = (rrow < R) ? n - a.w + rrow % a.w : -1;
    rowj[i] = a.jstar[grp * ROWS + i];
    rowcs[i] = a.cstar[grp * ROWS + i];
  }
  {
    // tiles of this chunk holding some row's dominant key (one bit each)
    uint32_t bit = 0;
    if (tid < ROWS) {
      const int j = a.jstar[grp * ROWS + tid];
      if (j >= c0 && j < c1) bit = 1u << ((j - c0) / KT);
    }
    for (int o = 32; o > 0; o >>= 1) bit |= __shfl_xor(bit, o, 64);
    if (lane == 0) dmask[wave] = bit;
  }
  const float* vnb = a.vnorm + static_cast<size_t>(h) * a.T + base;
  for (int i = tid; i < c1 - c0; i += WG) sbuf[i] = vnb[c0 + i];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    settle(qa[kk]);
    settle(oha[kk]);
  }
  __syncthreads();

  const char* kb8 = reinterpret_cast<const char*>(a.k + (static_cast<size_t>(h) * a.T + base) * D);
  const char* vb8 = reinterpret_cast<const char*>(a.v + (static_cast<size_t>(h) * a.T + base) * D);
  RingFill fill;
  fill.init(lds_addr(ring), wave, lane);
  const int ntile = (c1 - c0 + KT - 1) / KT;

  auto reduce_tile = [&](int t, int st) {   // 4 row-block partials of tile t (ring stage st) -> sbuf
    if (tid < KT) {
      const float* rr = &red[st][0][0];
      sbuf[t * KT + tid] = (rr[tid] + rr[KT + tid]) + (rr[2 * KT + tid] + rr[3 * KT + tid]);
    }
  };
  int koff[D / 16];   // loop-invariant operand offsets (K and V share them; +8 KiB per half)
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = tile_off(col, 2 * kk + hl);
  const bool causal = a.causal != 0;

  // Tiles are taken from the chunk's end back to its start: pass 1 streamed
  // each chunk front to back, so the tiles it read last are the likeliest to
  // still be in the Infinity Cache.  The ring stage follows the step count.
  if (ntile > 0) fill.template issue<NT>(kb8, vb8, c0 + (ntile - 1) * KT, c1, 0);

  // One tile; EDGE tiles mask keys past the chunk end or a row's causal
  // horizon, interior tiles carry no masking code.
  auto tile = [&](const int t, const int st, auto edge_tag, auto big_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr bool BIG = decltype(big_tag)::value;
    const int kt0 = c0 + t * KT;
    const char* Kt = ring + st * STAGE_BYTES;
    const char* Vt = Kt + TILE_BYTES;
    // S = Q K^T and G = ||o_h||^2 + ||v||^2 - 2 O_h V^T for both 32-key
    // halves; each half's operands are read in one batch so the LDS
    // latency is paid once per chain rather than once per MFMA
    f32x16 sacc[2], gacc[2];
    // the MFMA section runs at raised wave priority, so that the other wave
    // of the SIMD tends to be in its vector-ALU section meanwhile
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kop[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        kop[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(Kt + kb * 32 * ROWB + koff[kk]));
      sacc[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) sacc[kb] = mfma32(qa[kk], kop[kk], sacc[kb]);
      const float vn2 = sbuf[t * KT + kb * 32 + col];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 nv = *reinterpret_cast<const f32x4*>(&rowc[ROWS + wave * 32 + 8 * q4 + 4 * hl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) gacc[kb][4 * q4 + e] = nv[e] + vn2;
      }
      bf16x8 vop[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        vop[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(Vt + kb * 32 * ROWB + koff[kk]));
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) gacc[kb] = mfma32(oha[kk], vop[kk], gacc[kb]);
      // issue order: four operand reads ahead of the MFMA that consumes
      // them, the K chain then the V chain
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * (D / 16) - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // x = log2 p in place of the logits; hidden pairs get x = -inf (p = 0)
    float xmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&rowc[wave * 32 + 8 * q4 + 4 * hl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[kb][4 * q4 + e] = fmaf(sacc[kb][4 * q4 + e], a.c2, -lv[e]);
      }
      if constexpr (EDGE) {
        // also hides each row's dominant key: its exact term is added after
        // the tiles
        const int key = kt0 + kb * 32 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ri = wave * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool hidden = (key >= c1) | (causal & (key > rowhz[ri])) | (key == rowj[ri]);
          sacc[kb][r] = hidden ? -INFINITY : sacc[kb][r];
        }
      }
      if constexpr (BIG) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xmax = fmaxf(xmax, sacc[kb][r]);
      }
    }
    float sc[2] = {0.f, 0.f};
    if (BIG && __any(xmax > kResidX)) {
      // some weight above 2^-6 (uniform): add the residual plane of o and
      // use the exact weight factor 1 / y^2, y = (1 - p) / p = 2^-x - 1
      const uint16_t* lp = a.olo + (grp * ROWS + wave * 32 + col) * D;
      asm volatile("" : "+v"(gacc[0]), "+v"(gacc[1]));   // keeps this work inside the branch
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 ola = as_bf16x8(*reinterpret_cast<const u32x4*>(lp + 16 * kk + 8 * hl));
          const bf16x8 vv = as_bf16x8(*reinterpret_cast<const u32x4*>(Vt + kb * 32 * ROWB + koff[kk]));
          gacc[kb] = mfma32(ola, vv, gacc[kb]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          gacc[kb][r] += a.no2d[grp * ROWS + wave * 32 + 8 * (r >> 2) + 4 * hl + (r & 3)];
          const float y = __builtin_amdgcn_exp2f(-sacc[kb][r]) - 1.f;
          const float y2 = fmaf(y, y, 9.094947e-13f);                    // + 2^-40 keeps 1/y2 finite
          sc[kb] = fmaf(gacc[kb][r], __builtin_amdgcn_rcpf(y2), sc[kb]);  // gacc = ||o - v||^2
        }
      }
    } else {
      // every p <= 2^-6: p / (1 - p) = p + p^2 to a relative p^2 <= 2^-12,
      // so its square to 2^-11
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pw = __builtin_amdgcn_exp2f(sacc[kb][r]);
          const float q = fmaf(pw, pw, pw);
          sc[kb] = fmaf(gacc[kb][r] * q, q, sc[kb]);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float tot = sum_xor32(sc[kb]);
      if (hl == 0) red[st][wave][kb * 32 + col] = tot;
    }
  };

  const int edge_from = causal ? min(c1 - KT, n - a.w - KT + 1) : c1 - KT;   // first key of an edge tile
  // tiles holding some row's dominant key take the masking tile body
  const uint32_t dtiles = __builtin_amdgcn_readfirstlane(dmask[0] | dmask[1] | dmask[2] | dmask[3]);
  // step i takes tile t = ntile - 1 - i from ring stage i % 2
  if (wave_rows) {
    for (int i = 0; i < ntile; ++i) {
      const int t = ntile - 1 - i;
      wait_vm<0>();
      lds_barrier();
      if (i > 0) reduce_tile(t + 1, (i - 1) & 1);
      if (i + 1 < ntile) fill.template issue<NT>(kb8, vb8, c0 + (t - 1) * KT, c1, (i + 1) & 1);
      const bool edge = c0 + t * KT > edge_from || ((dtiles >> t) & 1u);
      if (wave_big) {
        if (edge) tile(t, i & 1, std::true_type{}, std::true_type{});
        else tile(t, i & 1, std::false_type{}, std::true_type{});
      } else {
        if (edge) tile(t, i & 1, std::true_type{}, std::false_type{});
        else tile(t, i & 1, std::false_type{}, std::false_type{});
      }
    }
  } else {   // the same loads, barriers and reductions, no arithmetic
    for (int i = 0; i < ntile; ++i) {
      const int t = ntile - 1 - i;
      wait_vm<0>();
      lds_barrier();
      if (i > 0) reduce_tile(t + 1, (i - 1) & 1);
      if (i + 1 < ntile) fill.template issue<NT>(kb8, vb8, c0 + (t - 1) * KT, c1, (i + 1) & 1);
    }
  }
  lds_barrier();
  if (ntile > 0) reduce_tile(0, (ntile - 1) & 1);
  lds_barrier();
  // the exact terms of the rows' dominant keys in this chunk, in row order
  if (dtiles) {
    if (tid == 0) {
      for (int i = 0; i < ROWS; ++i) {
        const int j = rowj[i];
        if (j >= c0 && j < c1) sbuf[j - c0] += rowcs[i];
      }
    }
    lds_barrier();
  }
  float* sout = a.sraw + (static_cast<size_t>(rg) * a.Hkv + h) * a.T + base;
  for (int i = tid; i < c1 - c0; i += WG) sout[c0 + i] = sbuf[i];
}

// ------------------------------------------------- pass 2, attention weights
// The attention-weight scores of the proposals compared on "A Probabilistic
// Interpretation of KV Cache Eviction" (App. D, Eq. 16 and 19; App. H): per
// key, the sum over the group's window rows of c_i * p_ij, p_ij = 2^(x -
// lse2) as in pass 2, times ||v_j|| for the value-weighted kinds.  The row
// weight c_i is 1 (H2O), the harmonic prior 1 / ((w - i) H_w) of window row
// i = 0 .. w-1 (H2O-h, min-h) or the last-row indicator (TOVA, min).  Only K
// streams through the ring; ||v||^2 comes from pass 1.
__device__ float score_row_weight(int kind, int wi, int w) {
  if (kind == KVE_SCORE_H2O) return 1.f;
  if (kind == KVE_SCORE_TOVA || kind == KVE_SCORE_MIN) return (wi == w - 1) ? 1.f : 0.f;
  double hw = 0.0;   // harmonic number H_w
  for (int k = 1; k <= w; ++k) hw += 1.0 / k;
  return static_cast<float>(1.0 / ((w - wi) * hw));
}

// NT: streaming loads of the tiles, as in score_p2_bf16.
template <bool VNORM, bool NT>
__global__ __launch_bounds__(WG, 2) void score_p2w_bf16(ScoreArgs a, int kind) {
  ScoreWork wk;
  if (!score_work(a, blockIdx.x, &wk)) return;
  // wave-uniform work indices, held in scalar registers
  const int c = __builtin_amdgcn_readfirstlane(wk.c), h = __builtin_amdgcn_readfirstlane(wk.h);
  const int rg = __builtin_amdgcn_readfirstlane(wk.rg), s = __builtin_amdgcn_readfirstlane(wk.s);
  const int base = __builtin_amdgcn_readfirstlane(a.seq_off[s]);
  const int n = __builtin_amdgcn_readfirstlane(a.seq_off[s + 1]) - base;
  const int c0 = c * a.CH;
  if (c0 >= n) return;
  const int c1 = min(c0 + a.CH, n);

  __shared__ __align__(1024) char ring[NSTAGE * TILE_BYTES];
  __shared__ __align__(16) float sbuf[kScoreChunkMax];   // ||v||^2 in (value-weighted kinds), scores out
  __shared__ __align__(16) float red[2][4][KT];
  __shared__ __align__(16) float rowc[2 * ROWS];        // lse2 and weight of each row
  __shared__ int rowhz[ROWS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int col = lane & 31;
  const int g = a.Hq / a.Hkv;
  const int R = g * a.w;
  const size_t grp = static_cast<size_t>((s * a.Hkv + h) * a.RG + rg);

  const int arow = rg * ROWS + wave * 32 + col;
  const bool arow_ok = arow < R;
  // a wave of the last row group with no window row loads its share of the
  // tiles but skips the arithmetic; its partials stay zero
  const bool wave_rows = __builtin_amdgcn_readfirstlane(rg * ROWS + wave * 32 < R ? 1 : 0) != 0;
  if (!wave_rows) red[0][wave][lane] = red[1][wave][lane] = 0.f;
  bf16x8 qa[D / 16];
  {
    const int qh = h * g + (arow_ok ? arow / a.w : 0);
    const int wi = arow_ok ? arow % a.w : 0;
    const uint16_t* qp = a.q_win + ((static_cast<size_t>(s) * a.Hq + qh) * a.w + wi) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (arow_ok) t = *reinterpret_cast<const u32x4*>(qp + 16 * kk + 8 * hl);
      qa[kk] = as_bf16x8(t);
    }
  }
  for (int i = tid; i < ROWS; i += WG) {
    const int rrow = rg * ROWS + i;
    rowc[i] = a.lse2[grp * ROWS + i];
    rowc[ROWS + i] = (rrow < R) ? score_row_weight(kind, rrow % a.w, a.w) : 0.f;
    rowhz[i] = (rrow < R) ? n - a.w + rrow % a.w : -1;
  }
  if (VNORM) {
    const float* vnb = a.vnorm + static_cast<size_t>(h) * a.T + base;
    for (int i = tid; i < c1 - c0; i += WG) sbuf[i] = vnb[c0 + i];
  }
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) settle(qa[kk]);
  __syncthreads();

  const char* kb8 = reinterpret_cast<const char*>(a.k + (static_cast<size_t>(h) * a.T + base) * D);
  RingFill fill;
  fill.init(lds_addr(ring), wave, lane);
  const int ntile = (c1 - c0 + KT - 1) / KT;

  auto reduce_tile = [&](int t) {   // 4 row-block partials -> sbuf
    if (tid < KT) {
      const float* rr = &red[t & 1][0][0];
      float tot = (rr[tid] + rr[KT + tid]) + (rr[2 * KT + tid] + rr[3 * KT + tid]);
      if (VNORM) tot *= sqrtf(sbuf[t * KT + tid]);
      sbuf[t * KT + tid] = tot;
    }
  };
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = tile_off(col, 2 * kk + hl);
  const bool causal = a.causal != 0;

  auto tile = [&](const int t, auto edge_tag) {
    if (!wave_rows) return;
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int kt0 = c0 + t * KT;
    const char* Kt = ring + (t & 1) * TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kop[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        kop[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(Kt + kb * 32 * ROWB + koff[kk]));
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) sacc = mfma32(qa[kk], kop[kk], sacc);
      float sc = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&rowc[wave * 32 + 8 * q4 + 4 * hl]);
        const f32x4 cw = *reinterpret_cast<const f32x4*>(&rowc[ROWS + wave * 32 + 8 * q4 + 4 * hl]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = fmaf(sacc[4 * q4 + e], a.c2, -lv[e]);
          if constexpr (EDGE) {
            const int key = kt0 + kb * 32 + col;
            const int hz = rowhz[wave * 32 + 8 * q4 + 4 * hl + e];
            const bool hidden = (key >= c1) | (causal & (key > hz));
            x = hidden ? -INFINITY : x;
          }
          sc = fmaf(cw[e], __builtin_amdgcn_exp2f(x), sc);
        }
      }
      sc = sum_xor32(sc);
      if (hl == 0) red[t & 1][wave][kb * 32 + col] = sc;
    }
  };

  if (ntile > 0) fill.template issue_k<NT>(kb8, c0, c1, 0);
  const int edge_from = causal ? min(c1 - KT, n - a.w - KT + 1) : c1 - KT;
  for (int t = 0; t < ntile; ++t) {
    wait_vm<0>();
    lds_barrier();
    if (t > 0) reduce_tile(t - 1);
    if (t + 1 < ntile) fill.template issue_k<NT>(kb8, c0 + (t + 1) * KT, c1, (t + 1) & 1);
    if (c0 + t * KT > edge_from) tile(t, std::true_type{});
    else tile(t, std::false_type{});
  }
  lds_barrier();
  if (ntile > 0) reduce_tile(ntile - 1);
  lds_barrier();
  float* sout = a.sraw + (static_cast<size_t>(rg) * a.Hkv + h) * a.T + base;
  for (int i = tid; i < c1 - c0; i += WG) sout[c0 + i] = sbuf[i];
}

// ---------------------------------------------------------------- launchers
hipError_t launch_score_bf16(const ScoreGeom& G, const void* q_win, const void* k, const void* v,
                             const int32_t* seq_off, float sm_scale, int causal, int score_kind,
                             void* ws, hipStream_t st, const ScoreZero* zero) {
  ScoreArgs a = {};
  if (zero) a.zero = *zero;
  a.q_win = static_cast<const uint16_t*>(q_win);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.seq_off = seq_off;
  a.S = G.S; a.Hq = G.Hq; a.Hkv = G.Hkv; a.w = G.w; a.T = G.T;
  a.RG = G.RG; a.CH = G.CH; a.P = G.P; a.causal = causal;
  a.c2 = sm_scale * kLog2e;
  char* base = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float*>(base + G.off_part_ml);
  a.part_e = reinterpret_cast<float*>(base + G.off_part_e);
  a.part_x = reinterpret_cast<float*>(base + G.off_part_x);
  a.part_o = reinterpret_cast<float*>(base + G.off_part_o);
  a.vnorm = reinterpret_cast<float*>(base + G.off_vnorm);
  a.lse2 = reinterpret_cast<float*>(base + G.off_lse2);
  a.no2 = reinterpret_cast<float*>(base + G.off_no2);
  a.no2d = reinterpret_cast<float*>(base + G.off_no2d);
  a.ohi = reinterpret_cast<uint16_t*>(base + G.off_ohi);
  a.olo = reinterpret_cast<uint16_t*>(base + G.off_olo);
  a.sraw = reinterpret_cast<float*>(base + G.off_sraw);
  a.jstar = reinterpret_cast<int32_t*>(base + G.off_jstar);
  a.cstar = reinterpret_cast<float*>(base + G.off_cstar);

  const int items = G.S * G.Hkv * G.P;
  dim3 grid(8 * ((items + 7) / 8) * G.RG);
  stage_begin(ST_SCORE_P1, st);
  hipLaunchKernelGGL(score_p1_bf16, grid, dim3(WG), 0, st, a);
  stage_end(ST_SCORE_P1, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(ST_SCORE_MERGE, st);
  // a row with at most 32 chunks (a batch of many rows, such as a ragged
  // batch of 64K-token sequences) takes 2 streams in a one-wave workgroup,
  // so that the rows fit the CUs in fewer rounds; otherwise 8
  if (G.P <= 32)
    hipLaunchKernelGGL((score_merge<D, true, 2>), dim3(G.S * G.Hkv * G.RG * ROWS), dim3(64), 0, st, a,
                       static_cast<float*>(nullptr));
  else
    hipLaunchKernelGGL((score_merge<D, true, 8>), dim3(G.S * G.Hkv * G.RG * ROWS), dim3(256), 0, st, a,
                       static_cast<float*>(nullptr));
  stage_end(ST_SCORE_MERGE, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(ST_SCORE_P2, st);
  if (score_kind == KVE_SCORE_PERTURB) {
    if (G.RG == 1) hipLaunchKernelGGL(score_p2_bf16<true>, grid, dim3(WG), 0, st, a);
    else hipLaunchKernelGGL(score_p2_bf16<false>, grid, dim3(WG), 0, st, a);
  } else if (score_kind == KVE_SCORE_MIN || score_kind == KVE_SCORE_MIN_H) {
    if (G.RG == 1) hipLaunchKernelGGL((score_p2w_bf16<true, true>), grid, dim3(WG), 0, st, a, score_kind);
    else hipLaunchKernelGGL((score_p2w_bf16<true, false>), grid, dim3(WG), 0, st, a, score_kind);
  } else {
    if (G.RG == 1) hipLaunchKernelGGL((score_p2w_bf16<false, true>), grid, dim3(WG), 0, st, a, score_kind);
    else hipLaunchKernelGGL((score_p2w_bf16<false, false>), grid, dim3(WG), 0, st, a, score_kind);
  }
  stage_end(ST_SCORE_P2, st);
  return hipGetLastError();
}

hipError_t launch_merge_f32(const ScoreGeom& G, const int32_t* seq_off, void* ws, hipStream_t st) {
  ScoreArgs a = {};
  a.seq_off = seq_off;
  a.S = G.S; a.Hq = G.Hq; a.Hkv = G.Hkv; a.w = G.w; a.T = G.T;
  a.RG = G.RG; a.CH = G.CH; a.P = G.P;
  char* base = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float*>(base + G.off_part_ml);
  a.part_o = reinterpret_cast<float*>(base + G.off_part_o);
  a.lse2 = reinterpret_cast<float*>(base + G.off_lse2);
  a.no2 = reinterpret_cast<float*>(base + G.off_no2);
  float* o32 = reinterpret_cast<float*>(base + G.off_ohi);
  dim3 grid(G.S * G.Hkv * G.RG * ROWS);
  if (G.d == 64) hipLaunchKernelGGL((score_merge<64, false, 8>), grid, dim3(256), 0, st, a, o32);
  else hipLaunchKernelGGL((score_merge<128, false, 8>), grid, dim3(256), 0, st, a, o32);
  return hipGetLastError();
}

}  // namespace kve
