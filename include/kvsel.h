/*
 * kvsel.h -- attention-mass KV selection and compacted decode attention on
 * AMD Instinct MI355X (gfx950).  C ABI; every entry point is asynchronous on
 * the HIP stream it is given.
 *
 * Pipeline (one transformer layer, per batch element b and KV head kvh;
 * "segment" s = b * hkv + kvh):
 *
 *   kvsel_score        window-mass score of every cached key
 *   kvsel_lmba         per-row 90 %-mass minimum budget (layer uncertainty)
 *                      and the attention a selection keeps
 *   kvsel_select       keep tokens per segment (top-B, chunk top-k or head policy)
 *   kvsel_chunk_vote   ChunkLLM layer-wise vote: one chunk key from the layers' scores
 *   kvsel_compact      gather kept K/V rows into a packed variable-length cache
 *   kvsel_decode_attn  single-token GQA decode attention over that cache
 *   kvsel_append       add each decoded token under the head's eviction rule
 *   kvsel_zigzag_budgets  (host) bounded per-layer budgets
 *
 * Sources, cited by page title and the equation / section on it:
 *   ZigZagkv: Dynamic KV Cache Compression for Long-context Modeling based on
 *     Layer Uncertainty (arXiv 2412.09036): Eq. 7 token score, Eq. 3 minimum
 *     budget for 90 % of the attention (LMBA), §5.5 / Table 3 attention loss,
 *     Eq. 4 and Eq. 6 bounded layer budgets.
 *   Model Tells You What to Discard: Adaptive KV Cache Compression for LLMs
 *     (arXiv 2310.01801): local / special-token / global head policies.
 *   ChunkLLM: A Lightweight Pluggable Framework for Accelerating LLMs
 *     Inference (arXiv 2510.02361): §2.2 Eq. 3 chunk attention over
 *     compressed chunk keys; only top-k chunks stay in the KV cache.
 *   RAP: KV-Cache Compression via RoPE-Aligned Pruning (arXiv 2602.02599):
 *     Fig. 2 / Eq. 2 decode-step attention; pair-pruned head dims (88).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *     memory; the library never allocates, frees or synchronises.
 *   - Dense tensors are row-major and contiguous with the shapes given.
 *     Element type of q / K / V follows kvsel_shape.dtype (bf16 = 16-bit
 *     brain float words, fp32 = IEEE single); scores and outputs are fp32.
 *   - Argument checks run on the host before anything is enqueued.  A failed
 *     check returns KVSEL_EINVAL / KVSEL_EUNSUPPORTED / KVSEL_ENOSPC and
 *     enqueues nothing.  A failed launch returns KVSEL_EHIP.  The message of
 *     the last non-OK status of the calling thread is kvsel_last_error().
 *   - Preconditions on device data (indices in range, segments not
 *     overlapping, chunk ends increasing) are documented, not checked; the
 *     kernels still never read or write outside the buffers described by the
 *     host-side sizes.
 *   - Workspaces (`ws`) may hold anything on entry: each call writes what it
 *     later reads.  A workspace serves one call at a time; calls that may
 *     run concurrently (other streams) need workspaces of their own.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVSEL_OK = 0,
  KVSEL_EINVAL = 1,       /* bad argument (null pointer, bad size or shape) */
  KVSEL_EUNSUPPORTED = 2, /* head_dim / dtype / group size not built */
  KVSEL_ENOSPC = 3,       /* workspace smaller than the matching *_workspace() */
  KVSEL_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} kvsel_status;

typedef enum { KVSEL_FP32 = 0, KVSEL_BF16 = 1 } kvsel_dtype;

/* Pair-pruned rotary position embedding applied by the library (RAP page,
 * §3, Eq. 5-10 and §6.2.3: RoPE turns 2-D pairs, so a key / query that keeps
 * whole pairs is rotated pair by pair with each kept pair's own frequency,
 * and pruning commutes with the rotation).  With kvsel_shape.rope set, the
 * queries of kvsel_score, kvsel_lmba and kvsel_decode_attn and the new key of
 * kvsel_append arrive unrotated and are rotated on their way in; cached keys
 * are expected rotated (as kvsel_append writes them).
 *   cos_sin  [max_pos][half][2] fp32 (device): cos and sin of the angle of
 *            rotary pair p at position t (the unpruned model's RoPE table)
 *   max_pos  rows of cos_sin; every position rotated must be below it
 *   half     rotary pairs of the unpruned head (e.g. 64 for 128 dims),
 *            half >= head_dim / 2
 *   pairs    [hkv][head_dim / 2] int32 (device): kept pair index per KV
 *            head, each in [0, half) (a query head uses its KV head's list)
 *   q_pos    kvsel_decode_attn: position of the decode query
 * Row layout: kept pair e is elements e and e + head_dim/2 of the row.  The
 * pair (x, y) at position t becomes (x c - y s, x s + y c) with (c, s) =
 * cos_sin[t][pairs[kvh][e]]; each product and the sum are rounded to fp32 on
 * their own (no fused multiply-add), then to the storage type (bf16:
 * nearest-even).  Window query i of kvsel_score / kvsel_lmba sits at
 * q_pos0 + i; kvsel_append's key at pos.  Pair indices and positions outside
 * the table are a documented precondition: the kernels clamp them rather
 * than read outside it. */
typedef struct kvsel_rope {
  const float* cos_sin;
  int64_t max_pos;
  int32_t half;
  const int32_t* pairs;
  int64_t q_pos;
} kvsel_rope;

/* Shape of one layer's attention.
 *   batch, hq, hkv : batch size, query heads, KV heads; hq % hkv == 0;
 *                    query head h reads KV head h / G with group size
 *                    G = hq / hkv.  kvsel_score needs G * w <= 256 and
 *                    kvsel_decode_attn G <= 8 (EUNSUPPORTED otherwise);
 *                    batch * hkv <= 2048 segments.
 *   head_dim       : 64, 88 or 128 (88 = RAP pair-pruned layout).
 *   n              : cached keys per (batch, KV head); for chunk scoring the
 *                    number of chunk keys.  1 <= n < 2^31.
 *   dtype          : kvsel_dtype of q / K / V.
 *   scale          : softmax scale applied to q . k, positive and finite
 *                    (usually 1/sqrt(head dim of the unpruned model)).
 *   rope           : (host pointer) NULL when queries and new keys arrive
 *                    rotated; else the kvsel_rope that rotates them. */
typedef struct {
  int32_t batch, hq, hkv, head_dim;
  int64_t n;
  int32_t dtype;
  float scale;
  const kvsel_rope* rope;
} kvsel_shape;

/* ---------------------------------------------------------------- score --
 * ZigZagkv page, Eq. 7: the score of key j is the attention weight that the
 * last w queries put on it, summed over those queries and (GQA) over the G
 * query heads that share the KV head:
 *   scores[b][kvh][j] = sum_{g<G} sum_{i<w} softmax_j'(scale q_{b,kvh*G+g,i} . k_{b,kvh,j'})[j]
 * where window query i sees keys j' <= q_pos0 + i (causal); pass
 * q_pos0 >= n - 1 for no mask.  The same call scores ChunkLLM chunk keys
 * (w = 1, keys = compressed chunk keys, head_dim 64).
 *   q_win   [batch][hq][w][head_dim]
 *   k       [batch][hkv][n][head_dim]
 *   scores  [batch][hkv][n] fp32 (out)
 *   ws      workspace of at least kvsel_score_workspace(s, w) bytes
 * Constraints: 1 <= w, G*w <= 256, q_pos0 >= 0.  Each row of scores sums to
 * G*w up to rounding. */
size_t kvsel_score_workspace(const kvsel_shape* s /*host*/, int32_t w);
kvsel_status kvsel_score(const kvsel_shape* s /*host*/, int32_t w, int64_t q_pos0,
                         const void* q_win, const void* k, float* scores,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------- lmba --
 * Layer uncertainty (ZigZagkv page, Eq. 3) and attention kept by a selection
 * (the page's §5.5 / Table 3 attention loss is max(0, 0.9 - kept)).  For
 * every attention row of the window queries -- row g*w + i of segment s is
 * window query i of query head kvh*G + g, causal as in kvsel_score --
 *   lmba[s][row]  = smallest k such that the k largest attention weights of
 *                   the row reach 90 % of its mass (weights taken in fixed
 *                   point, floor(p * 2^40), so the count is exact for them);
 *   kept_mass[s][row] = sum of the row's weights at the positions listed in
 *                   idx[seg_off[s] .. seg_off[s] + seg_len[s]) (optional:
 *                   NULL skips it).  The positions are taken as a set: one
 *                   listed twice counts once, one outside [0, n) counts 0;
 *                   the sum is taken in the same fixed point.
 * A layer's LMBA, the ZigZagkv uncertainty, is the mean of lmba over rows.
 *   lmba       [batch][hkv][G*w] int32 (out)
 *   kept_mass  [batch][hkv][G*w] fp32 (out) or NULL; then seg_off, seg_len
 *              and idx may be NULL
 *   ws         at least kvsel_lmba_workspace(s, w) bytes (it holds the
 *              attention rows: batch*hkv*G*w*n floats)
 * Constraints as for kvsel_score; with kept_mass, n/8 bytes of position
 * mask plus the row kernel's own LDS (about 41 KB, or 45 KB for rows longer
 * than 32768 keys or not a multiple of 4) must fit in one workgroup's LDS:
 * n up to about 930 K keys on gfx950 (160 KB), else KVSEL_EUNSUPPORTED with
 * nothing enqueued. */
size_t kvsel_lmba_workspace(const kvsel_shape* s /*host*/, int32_t w);
kvsel_status kvsel_lmba(const kvsel_shape* s /*host*/, int32_t w, int64_t q_pos0,
                        const void* q_win, const void* k, int32_t* lmba, const int64_t* seg_off,
                        const int32_t* seg_len, const int32_t* idx, int64_t r_cap,
                        float* kept_mass, void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------- select --
 * Writes, per segment s, the kept token positions in ascending order to
 * idx[seg_off[s] .. seg_off[s] + seg_len[s]) and their count to seg_len[s].
 * Score order is (score descending, index ascending); NaN orders below every
 * number and -0 equals +0.
 *   TOPB   (ZigZagkv page, Eq. 7 + Eq. 6): keep the min(budget[s], n)
 *          highest-score tokens.  scores [batch][hkv][n].
 *   CHUNK  (ChunkLLM page, §2.2-§2.3 and the §3.2 operating points): the
 *          last local_chunks chunks are always kept; then either the
 *          top_chunks best other chunks (top_chunks > 0), or other chunks in
 *          score order until the kept token count (local chunks included)
 *          reaches keep_tokens (top_chunks == 0).  Kept chunks are whole and
 *          expanded to their token positions.  scores [batch][hkv][n_chunks];
 *          chunk c of batch b covers [chunk_end[b][c-1], chunk_end[b][c]).
 *          local_chunks / top_chunks > 0 need n_chunks <= 32768.
 *   POLICY (FastGen page, core claim): per KV head kind: GLOBAL keeps all n,
 *          LOCAL keeps the last min(local_window, n), SPECIAL keeps
 *          special_pos[b][0 .. n_special).  scores unused (may be NULL).
 * seg_off [batch*hkv] int64: first row of each segment in idx (and in the
 *          compacted cache).  Precondition: seg_off[s] + kept_s does not reach
 *          into another segment.  Rows at or beyond r_cap are never written
 *          (seg_len still reports the full count).  */
typedef enum { KVSEL_SEL_TOPB = 0, KVSEL_SEL_CHUNK = 1, KVSEL_SEL_POLICY = 2 } kvsel_sel_mode;
typedef enum { KVSEL_HEAD_GLOBAL = 0, KVSEL_HEAD_LOCAL = 1, KVSEL_HEAD_SPECIAL = 2 } kvsel_head_kind;

typedef struct {
  int32_t mode;                 /* kvsel_sel_mode */
  const int32_t* budget;        /* TOPB:   [batch*hkv] tokens per segment (clamped to [0, n]) */
  int64_t n_chunks;             /* CHUNK:  chunks per sequence, >= 1 */
  const int64_t* chunk_end;     /* CHUNK:  [batch][n_chunks], strictly increasing, last == n */
  int64_t keep_tokens;          /* CHUNK:  token target per segment */
  const int8_t* head_kind;      /* POLICY: [hkv] kvsel_head_kind */
  int64_t local_window;         /* POLICY: tokens LOCAL heads keep, >= 0 */
  const int32_t* special_pos;   /* POLICY: [batch][n_special], ascending, unique, in [0, n) */
  int64_t n_special;            /* POLICY: entries per batch element, >= 0 */
  int64_t local_chunks;         /* CHUNK:  trailing chunks always kept, >= 0 */
  int64_t top_chunks;           /* CHUNK:  > 0: keep this many other chunks; 0: keep_tokens */
} kvsel_select_params;

kvsel_status kvsel_select(const kvsel_shape* s /*host*/, const kvsel_select_params* p /*host*/,
                          const float* scores, const int64_t* seg_off, int32_t* seg_len,
                          int32_t* idx, int64_t r_cap, hipStream_t stream);

/* ----------------------------------------------------------- chunk vote --
 * ChunkLLM page, §2.3: the chunks stored in the cache are chosen by a vote
 * across layers (the page gives the rule only in words; reading taken):
 * each of `layers` layers votes for its own top_k chunks (its chunk scores in
 * TOPB order: score descending, lower index first); the kept set of each
 * (b, kvh) is its last local_chunks chunks plus the top_k other chunks with
 * the most votes, ties to the larger attention summed over the layers, then
 * to the lower index.  The call writes one key per chunk such that
 * kvsel_select CHUNK with local_chunks and top_chunks = top_k over `key`
 * keeps exactly that set.  With V the vote count of the top_k-th best
 * non-local chunk (0 when there are at most top_k of them):
 *   key[b][kvh][c] = +inf  for a non-local chunk with more than V votes,
 *                    -inf  for a non-local chunk with fewer than V votes,
 *                    sum_l scores[l][b][kvh][c] otherwise (fp32, layers added
 *                          in order 0 .. layers-1; local chunks get it too).
 * The summed attention is never rounded into the vote count, so chunks whose
 * sums differ in any fp32 bit are ordered by them.
 *   s            shape of the chunk scores: n = chunks per sequence
 *   local_chunks trailing chunks that the later select forces in, >= 0
 *   scores       [layers][batch][hkv][n] fp32 (kvsel_score of each layer)
 *   key          [batch][hkv][n] fp32 (out)
 *   ws           at least kvsel_chunk_vote_workspace(s, layers, top_k) bytes
 * Constraints: 1 <= layers <= 255, top_k >= 1 (top_k > n votes for every
 * chunk), n bytes of vote counters plus 2 KB must fit in one workgroup's LDS
 * (else KVSEL_EUNSUPPORTED). */
size_t kvsel_chunk_vote_workspace(const kvsel_shape* s /*host*/, int32_t layers, int32_t top_k);
kvsel_status kvsel_chunk_vote(const kvsel_shape* s /*host*/, int32_t layers, int32_t top_k,
                              int64_t local_chunks, const float* scores, float* key, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------- compact --
 * Packed variable-length cache: for every segment s and r < seg_len[s],
 *   k_c[seg_off[s] + r] = k[b][kvh][idx[seg_off[s] + r]]   (bit-exact copy)
 * and likewise v_c from v.  Rows of segments are clipped at r_cap; an index
 * outside [0, n) yields a zero row.
 *   k, v      [batch][hkv][n][head_dim]
 *   k_c, v_c  [r_cap][head_dim] (out) */
kvsel_status kvsel_compact(const kvsel_shape* s /*host*/, const void* k, const void* v,
                           const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                           void* k_c, void* v_c, int64_t r_cap, hipStream_t stream);

/* --------------------------------------------------------------- decode --
 * RAP page Fig. 2 / Eq. 2 decode step over the compacted cache:
 *   out[b][h] = sum_{r < len} softmax_r(scale q[b][h] . k_c[off + r]) v_c[off + r]
 * with off = seg_off[b*hkv + h/G], len = seg_len[...] (clipped at r_cap).
 * Split-K: every segment is cut into row chunks processed in parallel; each
 * chunk keeps (an exponent reference at or within 8 log2 units below its
 * largest logit, sum of exponentials, weighted value sum) and a second pass
 * merges them.  An empty segment gives a zero output row.
 *   q    [batch][hq][head_dim]
 *   k_c, v_c [r_cap][head_dim]
 *   out  [batch][hq][head_dim] fp32 (out)
 *   ws   at least kvsel_decode_workspace(s, r_cap) bytes */
size_t kvsel_decode_workspace(const kvsel_shape* s /*host*/, int64_t r_cap);
kvsel_status kvsel_decode_attn(const kvsel_shape* s /*host*/, const void* q, const void* k_c,
                               const void* v_c, const int64_t* seg_off, const int32_t* seg_len,
                               int64_t r_cap, float* out, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* kvsel_decode_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture that may not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * kernels and result as kvsel_decode_attn; the per-item partials go to a
 * static device array of KVSEL_DECODE_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends.  Nothing is allocated or
 * freed by the call.  Calls on one GPU share that array: calls that overlap
 * on one GPU (other streams, other threads) race and give undefined output;
 * serialise them.  No scratch content carries over between calls (each call
 * writes every partial it reads).  The first call on a device looks up the
 * array's address there.
 * Errors: as kvsel_decode_attn, and KVSEL_ENOSPC when the call's partials
 * exceed the scratch (about r_cap / 2048 + batch * hkv items of
 * 2080 bytes at head_dim 128 with 4 query heads per KV head; 8 MiB holds
 * r_cap up to about 7.8 million rows). */
#define KVSEL_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
kvsel_status kvsel_decode_attn_noalloc(const kvsel_shape* s /*host*/, const void* q,
                                       const void* k_c, const void* v_c, const int64_t* seg_off,
                                       const int32_t* seg_len, int64_t r_cap, float* out,
                                       hipStream_t stream);

/* --------------------------------------------------------------- append --
 * Decode-time maintenance of the packed cache (FastGen page, core claim and
 * method: the per-head eviction rule keeps holding during generation --
 * local heads a sliding window, special-token heads only special tokens,
 * global heads everything).  The token just produced, at position `pos`,
 * joins segment s according to limit[s]:
 *   limit[s] <  0  not added (e.g. a special-token head, ordinary token);
 *   limit[s] == 0  the segment grows up to seg_cap[s] rows;
 *   limit[s] >  0  the segment keeps at most min(limit[s], seg_cap[s]) rows.
 * Below its bound the row goes to slot seg_len[s] and seg_len[s] grows by
 * one; at (or above) the bound the row holding the smallest position in
 * idx -- the oldest token, lowest slot on ties -- is overwritten in place.
 * Rows of a segment are then no longer in position order; decode does not
 * depend on their order.
 *   k_new, v_new [batch][hkv][head_dim]  the token's key and value rows
 *   seg_cap      [batch*hkv] int64: rows reserved from seg_off[s] on
 *   limit        [batch*hkv] int32, or NULL (every segment grows)
 *   seg_len, idx, k_c, v_c  updated in place; rows at or beyond r_cap are
 *                never written.
 * Errors: EINVAL for NULL pointers, pos or r_cap outside [0, 2^31). */
kvsel_status kvsel_append(const kvsel_shape* s /*host*/, const void* k_new, const void* v_new,
                          int64_t pos, const int64_t* seg_off, const int64_t* seg_cap,
                          const int32_t* limit, int32_t* seg_len, int32_t* idx, void* k_c,
                          void* v_c, int64_t r_cap, hipStream_t stream);

/* --------------------------------------------------------------- budgets --
 * ZigZagkv page, Eq. 4 and Eq. 6 (host only, no GPU work):
 *   u_l = x_l / sum x;  beta_l = floor_budget + (avg_budget - floor_budget) * L * u_l
 * Layers with beta_l > n are fixed at n and Eq. 6 is applied again to the
 * rest with the remaining total.  Integer budgets: floor of beta, then the
 * leftover units one each to the largest fractional parts (ties to the lower
 * layer).  Result sums to L * avg_budget, each in [floor_budget, n].
 *   profile (host) [L] finite, > 0;  out (host) [L]
 * Errors: EINVAL unless 0 <= floor_budget <= avg_budget <= n and L >= 1. */
kvsel_status kvsel_zigzag_budgets(const double* profile, int32_t L, int64_t n,
                                  int64_t avg_budget, int64_t floor_budget, int32_t* out);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* kvsel_last_error(void);

/* Library version string. */
const char* kvsel_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVSEL_H */
