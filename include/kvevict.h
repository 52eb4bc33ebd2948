/*
 * kvevict.h -- C ABI of the MI355X (gfx950) windowed KV-cache eviction library.
 *
 * Four calls make up the eviction-time path and the decode step:
 *
 *   kvevict_score        output-aware per-token eviction scores
 *   kvevict_score_ex     the same, or attention-weight scores, max/avg pool
 *   kvevict_select       per-head budgeted selection (top-k or sampling)
 *   kvevict_compact      gather of the kept K/V rows and their logit bias
 *   kvevict_evict        score + select + compact of one layer in one call
 *   kvevict_decode_snis  decode attention over the compacted cache with a
 *                        per-entry logit bias (self-normalised importance
 *                        sampling correction); kvevict_decode_snis_append
 *                        is the same step with the step's own token
 *                        appended to the cache on the device
 *
 * Pages cited:
 *   [PI] "A Probabilistic Interpretation of KV Cache Eviction"
 *   [DK] "DropKV: Decoupling Residual-Output Perturbation for Near-Optimal
 *        KV-Cache Eviction"
 *   [IT] "Information-Theoretic Token Eviction and KV-Cache Compression for
 *        Memory-Bounded Long-Context LLM Inference"
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Notation: S sequences, Hq query heads, Hkv KV heads (g = Hq/Hkv query
 *    heads share one KV head: q-head qh uses KV head qh / g), d head dim,
 *    w observation-window rows, n_s tokens of sequence s, T = sum n_s.
 *  - Memory: every tensor argument is a device pointer unless its name ends
 *    in _host.  All tensors are dense, row-major, with the innermost
 *    dimension contiguous.  bf16 data is raw IEEE bfloat16 bits (uint16).
 *    K and V rows must be 16-byte aligned (d * element size is a multiple
 *    of 16 for every supported d).
 *  - Ownership: the caller owns every buffer, including the workspace.  The
 *    library never allocates device memory and keeps no state between
 *    calls except a thread-local error string.  Inputs are read-only.
 *    Outputs must not alias inputs.
 *  - Execution: each call validates its arguments on the host, then
 *    enqueues kernels on `stream` (a hipStream_t; NULL = default stream)
 *    and returns without synchronising.  Faults during execution surface
 *    at the caller's next synchronisation.  The calls enqueue kernels only
 *    (scratch that must start at zero is cleared by a kernel, never by a
 *    memset or copy), so a caller may capture them in a HIP graph and
 *    replay it.  Grid sizes are fixed at capture from the host-side
 *    arrays, so a replay computes the captured sizes: the device buffers
 *    (offsets, inputs, outputs, workspace) must stay allocated, and the
 *    device offset arrays unchanged, while the graph is replayed.
 *  - Errors: argument errors return KVE_EINVAL / KVE_ENOTSUP /
 *    KVE_EWORKSPACE before anything is launched or written; a failed launch
 *    returns KVE_EHIP.  kvevict_last_error() describes the last failure of
 *    the calling thread.
 */
#ifndef KVEVICT_H
#define KVEVICT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVE_OK = 0,
  KVE_EINVAL = 1,      /* bad argument (null pointer, inconsistent sizes) */
  KVE_ENOTSUP = 2,     /* valid but unsupported shape (e.g. head dim)      */
  KVE_EWORKSPACE = 3,  /* workspace smaller than the *_workspace() query   */
  KVE_EHIP = 4,        /* a HIP runtime call failed                        */
  KVE_ENOCONV = 5      /* per-head status only: expected-samples search did
                          not reach its tolerance band (see kvevict_select) */
} kve_status;

typedef enum { KVE_BF16 = 0, KVE_F32 = 1 } kve_dtype;
typedef enum { KVE_TOPK = 0, KVE_SAMPLE = 1 } kve_mode;

/* Shape of a (possibly ragged) batch; shared by all calls. */
typedef struct {
  int32_t S, Hq, Hkv, d, w;
  int32_t dtype;                /* kve_dtype of q/k/v                        */
  const int32_t* seq_off;       /* device [S+1]: token offsets on axis T     */
  const int32_t* seq_off_host;  /* host   [S+1]: the same values             */
} kve_layout;

/* Supported shapes: bf16 needs d = 128, fp32 d in {64, 128}; Hq % Hkv == 0;
 * 1 <= w <= 64; w <= n_s for every sequence (score); T < 2^30. */

/* ------------------------------------------------------------------ score
 * Window scoring ([DK] §3.2 single-token perturbation, §3.3 windowed
 * squared score, §3.4 two-pass fused computation; [PI] §5 GQA groups;
 * SnapKV-style pooling as described in [PI] App. D).
 *
 * For every sequence s, KV head h and key j < n_s:
 *   score[h][off_s + j] = maxpool_j( sum_{qh in group(h)} sum_{i<w}
 *        (a_ij / (1 - a_ij))^2 * || o_i - v_j ||^2 )
 * where row i of q-head qh is q_win[s][qh][i], logits are
 * sm_scale * <q_i, k_j>, a_ij is the row softmax (keys j > n_s - w + i
 * hidden when causal != 0; hidden pairs contribute 0), o_i = sum_j a_ij v_j,
 * and maxpool takes the maximum over |j' - j| <= (pool_kernel-1)/2 within
 * the sequence.  1 - a_ij is clamped below by about 2^-20 (only a key
 * holding nearly all of a row's weight is affected).
 *
 *   q_win   [S][Hq][w][d]  dtype
 *   k, v    [Hkv][T][d]    dtype
 *   scores  [Hkv][T]       float32, written for every token
 *   pool_kernel  odd, 1..31 (1 = no pooling)
 *   ws      device workspace of at least kvevict_score_workspace() bytes,
 *           no alignment beyond 256 bytes required, contents undefined
 *           on entry and on return.
 * Deterministic: no floating-point atomics; identical inputs give
 * bit-identical scores. */
size_t kvevict_score_workspace(const kve_layout* L);
kve_status kvevict_score(const kve_layout* L, const void* q_win, const void* k,
                         const void* v, float sm_scale, int32_t causal,
                         int32_t pool_kernel, float* scores, void* ws,
                         size_t ws_bytes, void* stream);

/* Other scores on the same two passes ([PI] App. D, Eq. 16-20, and App. H):
 * sum over the group's q-heads and window rows i of c_i * a_ij, times
 * ||v_j|| for the value-weighted kinds, then pooled:
 *   KVE_SCORE_H2O     c_i = 1                (H2O column sums, Eq. 16)
 *   KVE_SCORE_H2O_H   c_i = h_i              (pi_H2O-h)
 *   KVE_SCORE_TOVA    c_i = [i == w - 1]     (TOVA, Eq. 19)
 *   KVE_SCORE_MIN     c_i = [i == w - 1], times ||v_j||   (pi_min)
 *   KVE_SCORE_MIN_H   c_i = h_i, times ||v_j||            (pi_min-h)
 * with the harmonic prior h_i = 1 / ((w - i) H_w), H_w = sum_{k<=w} 1/k.
 * KVE_SCORE_PERTURB is the output-aware score of kvevict_score.  The group
 * sum stands for the layer or group mean of the pages (same ranking and
 * same normalised proposal).  pool_mode KVE_POOL_AVG takes the mean over
 * the in-sequence keys of the window instead of the maximum (SnapKV-style
 * smoothing, App. D).
 *   KVE_SCORE_KNORM   exp(80 - ||k_j||) (K-norm, App. D Eq. 18, with the
 *                     key norms of [DK]'s related work and the negative
 *                     sign of [PI]'s prose): the largest scores are the
 *                     smallest key norms, and the tempered proposal of
 *                     kvevict_select is the softmax of -||k|| / tau.  Reads K
 *                     only (q_win and v are checked but not read); the
 *                     constant 80 keeps norms up to about 167 in range.
 * The attention-weight kinds need the bf16 path (KVE_ENOTSUP for fp32);
 * PERTURB and KNORM take both dtypes; both pool modes work for all.  Same
 * workspace, layouts and determinism as kvevict_score. */
typedef enum {
  KVE_SCORE_PERTURB = 0,
  KVE_SCORE_H2O = 1,
  KVE_SCORE_H2O_H = 2,
  KVE_SCORE_TOVA = 3,
  KVE_SCORE_MIN = 4,
  KVE_SCORE_MIN_H = 5,
  KVE_SCORE_KNORM = 6
} kve_score_kind;
typedef enum { KVE_POOL_MAX = 0, KVE_POOL_AVG = 1 } kve_pool_mode;
kve_status kvevict_score_ex(const kve_layout* L, const void* q_win, const void* k,
                            const void* v, float sm_scale, int32_t causal,
                            int32_t pool_kernel, int32_t score_kind,
                            int32_t pool_mode, float* scores, void* ws,
                            size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------- select
 * Per (sequence, KV head) budgeted selection of B_s = bud_off[s+1] -
 * bud_off[s] tokens (0 <= B_s <= n_s), written to
 * idx[h][bud_off[s] .. bud_off[s+1]) as sequence-relative token indices in
 * ascending order, with the logit bias of each kept token in bias[h][..].
 *
 * KVE_TOPK ([DK] §3.3: evict the smallest scores; [PI] §4 top-k
 *   estimator): the B_s largest scores, ties -> lower index, NaN ranked
 *   below every number.  bias = 0.
 * KVE_SAMPLE ([PI] §4 probabilistic eviction with a proposal; App. D.1
 *   tempering; App. F Problem 5 / Algorithm 2 expected-samples search;
 *   §6 Eq. 10 weight temperature):
 *   proposal log pi~_j = log(max(score_j, 2^-126)) / tau, pi = pi~/sum pi~;
 *   m >= 0 integer with |sum_j 1 - (1-pi_j)^m - B_s| <= 0.5 (searched in
 *   [0, 10^12]); the kept set is the B_s largest Gumbel keys
 *   log pi~_j - log(-log u_j), u_j = ((x >> 11) + 0.5) 2^-53 with x word
 *   j mod 4 of Philox-4x64-10(counter = (floor(j / 4), h, s, 0),
 *   key = (seed, 0));
 *   bias_j = -log(q_j) / tau_w with q_j = 1 - (1 - pi_j)^m.  B_s = n_s keeps
 *   all tokens with bias 0.  If no m <= 10^12 reaches the band, m = 10^12 and
 *   status_out[s][h] = KVE_ENOCONV (outputs remain valid).
 *
 *   scores     [Hkv][T] float32 (e.g. from kvevict_score)
 *   bud_off    device [S+1], bud_off_host host [S+1] (same values)
 *   idx        [Hkv][bud_off[S]] int32 out
 *   bias       [Hkv][bud_off[S]] float32 out
 *   m_out      [S][Hkv] float64 out, or NULL (0 in top-k mode)
 *   status_out [S][Hkv] int32 out, or NULL (KVE_OK or KVE_ENOCONV)
 *   ws         at least kvevict_select_workspace() bytes. */
size_t kvevict_select_workspace(const kve_layout* L, const int32_t* bud_off_host,
                                int32_t mode);
kve_status kvevict_select(const kve_layout* L, const float* scores,
                          const int32_t* bud_off, const int32_t* bud_off_host,
                          int32_t mode, float tau, float tau_w, uint64_t seed,
                          int32_t* idx, float* bias, double* m_out,
                          int32_t* status_out, void* ws, size_t ws_bytes,
                          void* stream);

/* kvevict_select with the proposal mixed with the uniform ([PI] App. D.1):
 * in KVE_SAMPLE mode pi'_j = mix * pi_j + (1 - mix) / n_s replaces pi_j
 * everywhere above (the search, q_j, and the Gumbel keys, which become
 * log pi'_j - log(-log u_j)).  mix in [0, 1], else KVE_EINVAL; mix = 1 is
 * kvevict_select bit for bit; ignored in KVE_TOPK mode. */
kve_status kvevict_select_ex(const kve_layout* L, const float* scores,
                             const int32_t* bud_off, const int32_t* bud_off_host,
                             int32_t mode, float tau, float tau_w, float mix,
                             uint64_t seed, int32_t* idx, float* bias,
                             double* m_out, int32_t* status_out, void* ws,
                             size_t ws_bytes, void* stream);

/* Sampling selection under a soft per-sequence budget ([PI] §7 and App. F.1,
 * Eq. 33): one m for all KV heads of sequence s, found by the same search on
 * the heads' mean expected distinct count (1/Hkv) sum_h E_h(m), with target
 * B_s = bud_off[s+1] - bud_off[s]; head h then keeps
 * kept[s][h] = floor(E_h(m) + 0.5) entries, clamped to [0, min(n_s, cap_s)],
 * chosen as in KVE_SAMPLE (the kept[s][h] largest Gumbel keys, ascending)
 * with bias -log(q_j) / tau_w, q_j = 1 - (1 - pi_j)^m (bias 0 for a head
 * that keeps all n_s).  Peaked heads keep fewer entries than flat ones.
 *   cap_off    device [S+1], cap_off_host host [S+1]: output slots per head
 *              of each sequence, cap_s = cap_off[s+1] - cap_off[s] in
 *              [0, n_s], and cap_s = n_s where B_s = n_s (KVE_EINVAL
 *              otherwise)
 *   idx, bias  [Hkv][cap_off[S]] out; slots r >= kept[s][h] hold idx -1 and
 *              bias -inf (kvevict_compact turns them into zero rows with
 *              bias -inf, which the decode weighs 0)
 *   kept       [S][Hkv] int32 out, or NULL
 *   m_out      [S][Hkv] float64 out, the same m in every head of a sequence
 *   status_out [S][Hkv] as kvevict_select
 *   ws         at least kvevict_select_workspace(L, bud_off_host, KVE_SAMPLE)
 * Compact with the capacities in place of the budgets (bud_off := cap_off)
 * to carry the padded slots into the cache. */
kve_status kvevict_select_soft(const kve_layout* L, const float* scores,
                               const int32_t* bud_off, const int32_t* bud_off_host,
                               const int32_t* cap_off, const int32_t* cap_off_host,
                               float tau, float tau_w, float mix, uint64_t seed,
                               int32_t* idx, float* bias, int32_t* kept,
                               double* m_out, int32_t* status_out, void* ws,
                               size_t ws_bytes, void* stream);

/* The literal estimator of [PI] §4 (keep the entries drawn at least once in
 * m draws with replacement from the proposal) with the weights of Algorithm 1
 * step 4 tempered as Eq. 10: per (sequence, head) with m = m_in[s][h] draws
 * (a whole number in [0, 2^31 - 1]; otherwise status KVE_ENOTSUP and nothing
 * kept; the draws cost time in proportion to m), draw k takes u_k = ((x >> 11) + 0.5) 2^-53, x the first word of
 * Philox-4x64-10(counter = (k, h, s, 1), key = (seed, 0)), and lands on the
 * first entry whose cumulative proposal exceeds u_k times the total (the
 * proposal as in KVE_SAMPLE: tempered by tau, mixed with the uniform when
 * mix < 1).  Every entry drawn (count c_j > 0) is kept, ascending, with bias
 * log(c_j / (m pi_j)) / tau_w.  The kept count is random (its mean is
 * E(m) of Eq. 24; m can come from kvevict_select's m_out).
 *   m_in       device [S][Hkv] float64
 *   cap_off    device [S+1], cap_off_host host [S+1]: output slots per head
 *              of each sequence, cap_s in [0, n_s]
 *   idx, bias  [Hkv][cap_off[S]] out; the first min(kept, cap_s) slots hold
 *              the lowest-index drawn entries, the rest -1 / -inf
 *   kept       [S][Hkv] int32 out (may exceed cap_s), or NULL
 *   status_out [S][Hkv] int32 out (KVE_OK or KVE_ENOTSUP), or NULL
 *   ws         at least kvevict_select_literal_workspace() bytes
 * n_s above 4194304 is KVE_ENOTSUP. */
size_t kvevict_select_literal_workspace(const kve_layout* L);
kve_status kvevict_select_literal(const kve_layout* L, const float* scores,
                                  const double* m_in, const int32_t* cap_off,
                                  const int32_t* cap_off_host, float tau,
                                  float tau_w, float mix, uint64_t seed,
                                  int32_t* idx, float* bias, int32_t* kept,
                                  int32_t* status_out, void* ws,
                                  size_t ws_bytes, void* stream);

/* Partition-conserving merge ([IT] §4.1): for every (sequence, KV head),
 * each evicted entry e (a position of the sequence not in the kept list)
 * is assigned to the kept entry r* with the largest key cosine similarity
 * cos(k_e, k_r) (the lowest list position on ties; a zero key has
 * similarity 0), and merged into it when cos > tau_merge.  The kept entry's
 * bias then grows by log(1 + number merged into it) (its multiplicity m_r,
 * starting at 1); keys and values stay as they are, so an exact duplicate
 * leaves the softmax normaliser unchanged.  Similarities are bf16 products
 * accumulated in fp32 (MFMA), kept to about 2^-16 (the argmax packs the
 * candidate's position into the low bits of the value): candidates or a
 * threshold closer than that are resolved by position / may go either way.
 *   k          [Hkv][T][128] bf16 (the full cache the selection read)
 *   bud_off    device [S+1], bud_off_host host [S+1]: the kept counts
 *   idx        [Hkv][bud_off[S]] kept positions as written by select
 *   bias       [Hkv][bud_off[S]] float32, updated in place
 *   merged     [Hkv][bud_off[S]] int32 out (entries merged into each), or NULL
 *   target     [Hkv][T] int32 out: list position each entry merged into,
 *              -1 if none (kept entries: -1), or NULL
 *   ws         at least kvevict_merge_workspace() bytes
 * bf16 with d = 128 only (KVE_ENOTSUP otherwise).  The result does not
 * depend on workgroup order (integer counts, 64-bit atomic maximum). */
size_t kvevict_merge_workspace(const kve_layout* L, const int32_t* bud_off_host);
kve_status kvevict_merge(const kve_layout* L, const void* k, const int32_t* bud_off,
                         const int32_t* bud_off_host, const int32_t* idx,
                         float tau_merge, float* bias, int32_t* merged,
                         int32_t* target, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- compact
 * Gather of the kept entries ([PI] §2 Eq. 3: evicted attention uses the
 * rows of K and V indexed by the kept set; [PI] §5: evicted entries are
 * ignored).  For r < B_s:
 *   k_c[h][cap_off[s] + r] = k[h][seq_off[s] + idx[h][bud_off[s] + r]]
 *   v_c likewise, bias_c[h][cap_off[s] + r] = bias[h][bud_off[s] + r].
 * Slots r >= B_s of each sequence are left untouched (decode headroom).
 *   k, v      [Hkv][T][d] dtype;      idx, bias as produced by select
 *   cap_off   device [S+1] with cap_s = cap_off[s+1]-cap_off[s] >= B_s
 *   k_c, v_c  [Hkv][cap_off[S]][d] dtype out;  bias_c [Hkv][cap_off[S]] out
 * An idx entry of -1 (an empty slot of kvevict_select_soft; any negative
 * value) gives a zero row with bias -inf; one at or past n_s is skipped on
 * the device (its slot is left untouched). */
kve_status kvevict_compact(const kve_layout* L, const void* k, const void* v,
                           const int32_t* bud_off, const int32_t* bud_off_host,
                           const int32_t* idx, const float* bias,
                           const int32_t* cap_off, const int32_t* cap_off_host,
                           void* k_c, void* v_c, float* bias_c, void* stream);

/* ------------------------------------------------------------------ evict
 * One layer's eviction in one call ([DK] §3.2-3.4 scoring, [PI] §4
 * selection, [PI] §2 Eq. 3 gather): kvevict_score (output-aware scores,
 * max pooling over pool_kernel keys), then kvevict_select in `mode`, then
 * kvevict_compact -- the same outputs bit for bit (scores, idx, bias,
 * m_out, status_out, k_c, v_c, bias_c), with fewer launches: for bf16
 * inputs the pooling rides on the selection's first pass, the selection's
 * counters are cleared by the scorer's merge launch, and the selection's
 * ordered write gathers the kept rows into k_c / v_c / bias_c.  Arguments
 * as for the three calls; ws at least kvevict_evict_workspace() bytes
 * (256-byte aligned), of which the calls use disjoint parts. */
size_t kvevict_evict_workspace(const kve_layout* L, const int32_t* bud_off_host,
                               int32_t mode);
kve_status kvevict_evict(const kve_layout* L, const void* q_win, const void* k,
                         const void* v, float sm_scale, int32_t causal,
                         int32_t pool_kernel, const int32_t* bud_off,
                         const int32_t* bud_off_host, int32_t mode, float tau,
                         float tau_w, uint64_t seed, float* scores, int32_t* idx,
                         float* bias, double* m_out, int32_t* status_out,
                         const int32_t* cap_off, const int32_t* cap_off_host,
                         void* k_c, void* v_c, float* bias_c, void* ws,
                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ decode_snis
 * Corrected decode attention ([PI] §5 Definition 3-4 and Algorithm 1; GQA
 * paragraph of §5): for every sequence s and q-head qh (KV head h),
 *   out[s][qh] = sum_{r < cache_len[s]} softmax_r(sm_scale <q[s][qh], k_c[h][c+r]>
 *                                                 + bias_c[h][c+r]) v_c[h][c+r]
 * with c = cap_off[s].  With bias = log(weight) this is Algorithm 1's
 * (mu_hat + mu) / (z_hat + z): kept history entries carry bias -log q_j,
 * entries appended after eviction carry bias 0 (weight 1).  The caller
 * appends a new token by writing k_c, v_c and bias_c = 0 at slot
 * cap_off[s] + cache_len[s] and incrementing cache_len[s].
 *   q         [S][Hq][d] dtype
 *   cache_len device [S], 1 <= cache_len[s] <= cap_s
 *   max_cache_len  host upper bound of cache_len[s] (grid sizing)
 *   out       [S][Hq][d] float32
 *   ws        at least kvevict_decode_workspace() bytes. */
size_t kvevict_decode_workspace(const kve_layout* L, int32_t max_cache_len);
kve_status kvevict_decode_snis(const kve_layout* L, const void* q, const void* k_c,
                               const void* v_c, const float* bias_c,
                               const int32_t* cap_off, const int32_t* cap_off_host,
                               const int32_t* cache_len, int32_t max_cache_len,
                               float sm_scale, float* out, void* ws,
                               size_t ws_bytes, void* stream);

/* ----------------------------------------------------- decode_snis_append
 * One decode step that also appends the step's token ([PI] §5 Algorithm 1:
 * each new token enters the cache uncorrected, weight 1): for every sequence
 * s with cache_len[s] < cap_s, the token (k_new[h][s], v_new[h][s], bias 0)
 * is attended at slot cache_len[s] of every KV head h together with the
 * cache's first cache_len[s] entries -- the output of kvevict_decode_snis
 * after the caller's own append, bit for bit -- and is then stored there
 * (k_c, v_c, bias_c = 0) and cache_len[s] advanced by one, all on the
 * device, so that a decode loop takes two launches per step and can be
 * captured in a graph.  A sequence whose cache is full (cache_len[s] >=
 * cap_s) attends to its cap_s entries only; its token is neither attended
 * nor stored and its cache_len is left as it is.
 *   q              [S][Hq][d] dtype
 *   k_new, v_new   [Hkv][S][d] dtype, the step's token per (KV head, sequence)
 *   k_c, v_c, bias_c, cap_off  the compacted cache, as for decode_snis (written
 *                  at the appended slots only)
 *   cache_len      device [S], 0 <= cache_len[s]; read, then advanced
 *   max_cache_len  host upper bound of the entries attended, cache_len[s] + 1
 *                  for a sequence with room (grid sizing)
 *   ws             at least kvevict_decode_workspace() bytes
 * Errors as for kvevict_decode_snis.  Outputs must not alias inputs. */
kve_status kvevict_decode_snis_append(const kve_layout* L, const void* q, const void* k_new,
                                      const void* v_new, void* k_c, void* v_c, float* bias_c,
                                      const int32_t* cap_off, const int32_t* cap_off_host,
                                      int32_t* cache_len, int32_t max_cache_len, float sm_scale,
                                      float* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------- decode_snis_noalloc
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as kvevict_decode_snis, with the same arguments except the
 * workspace, and the same results bit for bit.  Its split partials live in
 * a device array the library holds per GPU, kvevict_decode_scratch_max()
 * bytes (8 MiB: S * Hq * ceil(max_cache_len / 256) * (d + 2) * 4 bytes plus
 * alignment must fit, e.g. 8 sequences x 32 q-heads at d = 128 up to caches
 * of about 15000 entries).  A larger batch returns KVE_EWORKSPACE with a
 * message and launches nothing.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); the first call on a device looks
 * up the array's address there once.  Calls on one GPU share the array:
 * calls that overlap on one GPU (other streams, other threads) race. */
size_t kvevict_decode_scratch_max(void);
kve_status kvevict_decode_snis_noalloc(const kve_layout* L, const void* q, const void* k_c,
                                       const void* v_c, const float* bias_c,
                                       const int32_t* cap_off, const int32_t* cap_off_host,
                                       const int32_t* cache_len, int32_t max_cache_len,
                                       float sm_scale, float* out, void* stream);

/* ------------------------------------------------------- instrumentation
 * Not part of the eviction path.  Opt-in per-kernel timing with HIP events
 * recorded on the launch stream around every kernel the four calls enqueue.
 * Stage ids: 0 score pass 1, 1 score merge, 2 score pass 2, 3 score pool,
 * 4 select, 5 compact, 6 decode split, 7 decode merge.
 * kvevict_timing_enable(mask) times the stages whose bit is set in mask
 * (bit i = stage i; 0xff = all), creates an event pool on first use (no
 * device memory) and clears previous records; 0 stops recording.
 * kvevict_timing_summary() waits for the recorded events, writes the mean
 * duration in ms and the number of launches per stage (n_stages entries),
 * and clears the records.  Process-wide, not thread-safe. */
int32_t kvevict_timing_enable(int32_t stage_mask);
int32_t kvevict_timing_summary(double* avg_ms, int32_t* counts, int32_t n_stages);

/* Message describing the last failed call on this thread ("" if none). */
const char* kvevict_last_error(void);

/* Library ABI version (major * 100 + minor). */
int32_t kvevict_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVEVICT_H */
