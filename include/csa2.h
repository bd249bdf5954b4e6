/*
 * csa2.h — C ABI of the CSA2 FP4 global-KV decode path for AMD MI355X (gfx950).
 *
 * The method (three public write-ups of DeepSeek-V4.1-Flash's KV compression):
 *   [P1] long-form post on the limits of KV-cache compression (yomxxx.com,
 *        2026-09-19), sections numbered 一..六;
 *   [P2] "DeepSeek-V4.1-Flash KV compression" (rebasdaily.com, 2026-09-21),
 *        section "same notes, many layers" (the CSA2 section);
 *   [P3] "890 bytes per token" analysis (ailily.cc), sections 二 and 三.
 *
 * A decode step of CSA2 global attention: each layer selects a few blocks
 * of history positions (top-k) and attends only to them [P2 CSA2 section];
 * layers run in one of three modes, Full / Reindex / Reuse [P2 CSA2 section;
 * P3 section 二, mode table]; the first Full layer scans everything into a
 * candidate pool that later layers search [P2 CSA2 section, hierarchical
 * sparse indexer]; the cache holds a 512-channel latent [P3 section 三] as
 * FP4 E2M1 codes with one E4M3 scale per 16 channels [P3 section 二], at a
 * fixed stride so kernels address a position from its index and dequantise
 * in parallel [P1 section 五].
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device memory owned by the caller;
 *     "host" pointers are read during the call only.  The library never
 *     allocates, frees or synchronises (except csa2_device_error) and keeps
 *     no state besides its loaded kernels, one device flag word and a host
 *     table of the workspace layout each of the last 256 workspaces was
 *     used with (see csa2_workspace_init).
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it in order; a call returns once its kernels are queued.
 *   - Host-checkable errors return a non-zero status before anything is
 *     queued.  Data-dependent problems found on the device (non-finite
 *     input, a full cache, a bad block id) set bits of a device flag word
 *     read by csa2_device_error; the kernel skips the offending item.
 *   - Nothing is thrown across the ABI and no call aborts the process.
 *   - Calls sharing a workspace must be ordered on one stream; distinct
 *     workspaces may be used from different threads and streams.
 *
 * Cache layout (per Full layer, fixed stride):
 *   codes  [batch][capacity][256] uint8: byte j of a position holds channel
 *          2j in its low nibble and channel 2j+1 in its high nibble; a
 *          nibble is sign(bit 3) | E2M1 magnitude code (bits 0..2).
 *   scales [batch][capacity][32]  uint8: byte g is the E4M3FN scale of
 *          channels 16g..16g+15.
 *   Block b of a sequence covers positions 8b..8b+7; a partial last block
 *   is used with the positions it has.
 *   Both arrays must be 256-byte aligned.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t csa2_status;
enum {
  CSA2_OK = 0,
  CSA2_E_ARG = 1,         /* null/misaligned pointer, bad mode, inconsistent sizes */
  CSA2_E_SHAPE = 2,       /* a size the kernels do not support (see each call)     */
  CSA2_E_WORKSPACE = 3,   /* workspace smaller than csa2_workspace_bytes()          */
  CSA2_E_CAPACITY = 4,    /* a host-visible bound exceeds the cache capacity        */
  CSA2_E_HIP = 5,         /* a HIP call or launch failed: csa2_last_error() says why */
  CSA2_E_UNSUPPORTED = 6  /* device is not gfx950                                   */
};

/* Layer modes [P2 CSA2 section; P3 section 二, mode table]. */
enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 };

/*
 * Indexer score rules.  The pages say the indexer keeps the top-k most
 * relevant blocks [P2 CSA2 section] but not how many query heads become one
 * block score; two plain readings are built, both in a pinned float32 order
 * so the selected indices are reproducible bit for bit:
 *   CSA2_SCORE_SUM      heads added in order into one query Qbar, score =
 *                       Qbar . key (memory-bound scan; the default);
 *   CSA2_SCORE_HEADMAX  score = the largest over the heads of q_h . key, each
 *                       head in the same order as Qbar . key (64 dot products
 *                       per block at 64 heads: bound by the vector ALU).
 * csa2_index_topk takes the rule as a flag OR-ed into its mode
 * (CSA2_FULL | CSA2_MODE_HEADMAX); csa2_step and csa2_block_scores take it
 * as a field / argument.
 */
enum { CSA2_SCORE_SUM = 0, CSA2_SCORE_HEADMAX = 1 };
#define CSA2_MODE_HEADMAX 0x100

/* Bits of the device flag word (csa2_device_error). */
enum {
  CSA2_FLAG_NONFINITE_KV = 1,   /* a quantised group held NaN/Inf: written as zeros     */
  CSA2_FLAG_CAPACITY = 2,       /* append into a full sequence, or dst_row out of range */
  CSA2_FLAG_NONFINITE_Q = 4,    /* an indexer query sum held NaN/Inf (scores unspecified) */
  CSA2_FLAG_BAD_INDEX = 8,      /* a candidate/selected block id was >= the block count */
  CSA2_FLAG_SWA_RANGE = 16,     /* an SWA row's largest magnitude exceeded 65504, the
                                   attention's fp16 operand range (stored as given)      */
  CSA2_FLAG_Q_RANGE = 32,       /* an attention query value had magnitude >= 65520 or was
                                   NaN/Inf: it has no fp16 value (the matrix-core operand),
                                   so the outputs of its sequence are unspecified         */
  CSA2_FLAG_CHECK = 64          /* checked build only (libcsa2_checked.so, compiled with
                                   -DCSA2_CHECKED): an index bound that a kernel relies on
                                   failed.  That build also scrambles the order in which
                                   workgroups take their work (environment variable
                                   CSA2_WG_ORDER, an unsigned salt; 0 = identity), and its
                                   results must equal the product library's bit for bit  */
};

#define CSA2_D 512              /* latent channels                 */
#define CSA2_BLOCK 8            /* positions per block             */
#define CSA2_CODE_BYTES 256     /* code bytes per position         */
#define CSA2_SCALE_BYTES 32     /* scale bytes per position        */
#define CSA2_MAX_POOL 8192      /* largest pool / candidate list   */
#define CSA2_MAX_TOPK 2048      /* largest top-k (blocks)          */
#define CSA2_MAX_HEADS 64       /* indexer heads 1..64; attention 16, 32 or 64 */
#define CSA2_MAX_CACHES 16      /* Full caches in one decode step  */
#define CSA2_MAX_WINDOW 1024    /* largest sliding window (positions) */
#define CSA2_MAX_SWA_SLOTS (1 << 22)  /* largest SWA ring (positions)  */
#define CSA2_MAX_SWA_LAYERS 64  /* layers with a local branch in one decode step */

/* Non-owning view of one Full layer's cache for a batch of sequences. */
typedef struct {
  uint8_t *codes;       /* device [batch][capacity][256]                            */
  uint8_t *scales;      /* device [batch][capacity][32]                             */
  int64_t *seq_len;     /* device [batch]: valid positions; appends increment it    */
  int64_t capacity;     /* positions per sequence; a multiple of 8                  */
  int64_t max_len;      /* host bound >= every seq_len[b] during the call (after any
                           append it makes); sizes grids; <= capacity               */
  int32_t batch;        /* sequences, >= 1                                          */
} csa2_kv;

/*
 * fp4_quantize_kv — quantise float32 rows into the FP4 cache format.
 *   Per 16-channel group: s = E4M3FN nearest to amax/6 (ties to even code,
 *   saturating at 448, no second-level scale since the representable maximum
 *   is 448 x 6 = 2688 [P3 section 三]); each value becomes the E2M1 code
 *   nearest to |x|/s (ties to even, saturating at 6) with its sign bit kept.
 *   Both decisions are exact.  [P3 section 二; P1 section 五]
 * x        device float32 [rows][512], 16-byte aligned.
 * rows     >= 0 (0 is a no-op).
 * dst_row  device int64 [rows]: destination row of each input row in
 *          codes/scales, or NULL for row i -> row i.  Rows outside
 *          [0, dst_rows) are skipped and flag CSA2_FLAG_CAPACITY.
 * dst_rows rows available in codes/scales (>= rows when dst_row is NULL).
 * codes    device uint8 [dst_rows][256], 8-byte aligned; scales device uint8
 *          [dst_rows][32].  Both are written, never read.
 * A group with NaN/Inf is written as zero codes and scale 0 and flags
 * CSA2_FLAG_NONFINITE_KV.
 */
csa2_status fp4_quantize_kv(const float *x, int64_t rows, const int64_t *dst_row,
                            int64_t dst_rows, uint8_t *codes, uint8_t *scales,
                            void *stream);

/*
 * csa2_append_kv — append one position per sequence (the row a Full layer
 * writes for the new token [P2 CSA2 section, mode Full]).
 *   For each b: quantise x[b] into position seq_len[b], then seq_len[b] += 1.
 *   A sequence already at capacity is left unchanged and flags
 *   CSA2_FLAG_CAPACITY.
 * kv  host pointer to the cache view.   x  device float32 [batch][512].
 */
csa2_status csa2_append_kv(const csa2_kv *kv, const float *x, void *stream);

/*
 * Non-owning view of one layer's sliding-window (SWA) cache for a batch of
 * sequences.  Local context goes through sliding-window attention [P2
 * "halve the long input"]; entries older than the window are never read by
 * the current decode step [P1 section 三]; the SWA KV stays FP8 while the
 * global KV moves to FP4 [P2 "same notes, many layers"].  Reading: E4M3FN
 * codes with one float32 scale per position, kept in a ring of `slots`
 * positions: position p of sequence b lives in slot p % slots.  A decode
 * step attends to the last `window` positions; a ring with more slots than
 * the window also holds what a prefill chunk's queries need (each query's
 * own window, see csa2_prefill_attend).
 */
typedef struct {
  uint8_t *codes;       /* device [batch][slots][512] E4M3FN, 16-byte aligned    */
  float *scales;        /* device [batch][slots]                                   */
  int64_t *seq_len;     /* device [batch]: positions written; appends increment it */
  int32_t window;       /* attention window, 1..CSA2_MAX_WINDOW                    */
  int32_t batch;        /* sequences, >= 1                                         */
  int32_t slots;        /* ring positions, window..CSA2_MAX_SWA_SLOTS; 0 = window  */
} csa2_swa;

/*
 * fp8_quantize_kv — quantise float32 rows into the SWA row format.
 *   s = fl32(amax / 448) of the row's largest magnitude; each value becomes
 *   the E4M3FN code nearest to fl32(x / s) (both divisions IEEE; ties to
 *   the even code), sign bit kept; s == 0 keeps only the signs.
 * x        device float32 [rows][512], 16-byte aligned; rows >= 0.
 * dst_row  device int64 [rows]: destination row of each input row, or NULL
 *          for row i -> row i.  Rows outside [0, dst_rows) are skipped and
 *          flag CSA2_FLAG_CAPACITY.  (A ring slot is row b*slots + p%slots.)
 * codes    device uint8 [dst_rows][512], 8-byte aligned; scales device
 *          float32 [dst_rows].
 * A row with NaN/Inf is written as zeros with scale 0 and flags
 * CSA2_FLAG_NONFINITE_KV; a row with amax > 65504 flags CSA2_FLAG_SWA_RANGE.
 */
csa2_status fp8_quantize_kv(const float *x, int64_t rows, const int64_t *dst_row,
                            int64_t dst_rows, uint8_t *codes, float *scales, void *stream);

/*
 * csa2_swa_append — for each b: quantise x[b] (device float32 [batch][512],
 * 16-byte aligned) as position seq_len[b] into slot seq_len[b] % slots,
 * then seq_len[b] += 1.  A negative seq_len[b] is left alone and flags
 * CSA2_FLAG_CAPACITY.
 */
csa2_status csa2_swa_append(const csa2_swa *swa, const float *x, void *stream);

/*
 * csa2_workspace_bytes — workspace needed by csa2_index_topk,
 * csa2_sparse_attend, and csa2_decode_step for these
 * bounds (max_len = longest sequence in positions), with or without a
 * local branch of any window up to CSA2_MAX_WINDOW.  Returns 0 for
 * unsupported bounds.
 */
size_t csa2_workspace_bytes(int32_t batch, int32_t heads, int64_t max_len,
                            int32_t pool, int32_t topk);

/*
 * csa2_workspace_init — zero-fill a workspace (with a kernel, so it can be
 * recorded in a HIP graph).  A workspace must be zero before its first use;
 * every call leaves its control words zero again when its kernels finish.
 * Where those words sit depends on the call's bounds (batch, max_len, pool,
 * topk): when a call's layout differs from the previous call's on the same
 * workspace, the library first zero-fills the part that holds them (a
 * kernel on the call's stream, up to the candidate area: about 4 bytes per
 * block per sequence plus 36 KB per sequence).
 */
csa2_status csa2_workspace_init(void *ws, size_t ws_bytes, void *stream);

/*
 * csa2_index_topk — the hierarchical sparse indexer of one layer
 * [P2 CSA2 section].
 *   mode CSA2_REUSE: idx_out[b][:] = prior_idx[b][:] (nothing when the
 *     pointers are equal); kv, q, cand and pool_out are not used.
 *   mode CSA2_FULL / CSA2_REINDEX: identical computation; the caller passes
 *     the layer's own cache (Full) or the latest Full cache (Reindex).
 *     OR-ing CSA2_MODE_HEADMAX into the mode selects the per-head score
 *     rule (CSA2_SCORE_HEADMAX, described above); the rest of this
 *     paragraph describes the default rule.
 *     Block key = mean of the block's dequantised rows (rows added in
 *     ascending order in float32, then divided by the row count); indexer
 *     query Qbar = heads added in order in float32; score = Qbar . key in a
 *     fixed float32 order (16 products of one scale group added left to
 *     right, then the 32 group sums added as a tree of adjacent pairs;
 *     products are not fused).  Selection keeps the highest scores, ties to
 *     the lowest block id.
 *     cand == NULL: all blocks 0..ceil(seq_len[b]/8)-1 are candidates
 *       (full scan).  If pool > 0, pool_out[b] receives the top-`pool`
 *       blocks and idx_out the top-`topk` of those.
 *     cand != NULL: the candidates of sequence b are cand[b][0..n_cand),
 *       distinct, -1 entries ignored (as written to pool_out by an earlier
 *       call); pool must be 0.
 *   Output: idx_out[b] lists the selected block ids, ascending (for a
 *   cand list: in the order they appear in cand), then -1 up to topk.
 *   pool_out[b] likewise, ascending.
 * q        device float32 [batch][heads][512], 16-byte aligned.
 * heads    1..64 for the indexer (the attention needs 16, 32 or 64).
 * n_cand   1..CSA2_MAX_POOL when cand != NULL.
 * topk     1..CSA2_MAX_TOPK, <= pool when pool > 0.
 * pool     0 or topk..CSA2_MAX_POOL.
 * idx_out  device int32 [batch][topk]; pool_out device int32 [batch][pool].
 * prior_idx device int32 [batch][topk] (Reuse only).
 * ws       device workspace of ws_bytes >= csa2_workspace_bytes(...).
 */
csa2_status csa2_index_topk(int32_t mode, const csa2_kv *kv, const float *q, int32_t heads,
                            const int32_t *cand, int32_t n_cand, int32_t topk,
                            int32_t *idx_out, int32_t pool, int32_t *pool_out,
                            const int32_t *prior_idx, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * csa2_sparse_attend — softmax attention of every head over the positions
 * of the selected blocks [P2 CSA2 section], dequantising them inside the
 * kernel [P1 section 五].  Keys and values are both the dequantised latent,
 * shared by all heads.  Positions 8*idx+t at or beyond seq_len[b] are
 * skipped; -1 entries are ignored; no position gives a zero output.
 *   out[b][h] = sum_p softmax_p(scale * q[b][h] . k_p) k_p
 * swa   NULL, or the layer's SWA cache (same batch): the local branch.  Its
 *       last min(window, swa->seq_len[b]) positions join the same softmax
 *       as further keys = values (reading: one softmax over both branches).
 * q     device float32 [batch][heads][512]; heads in {16, 32, 64}.
 * idx   device int32 [batch][topk], topk 1..CSA2_MAX_TOPK.
 * out   device float32 [batch][heads][512].
 * Accumulates in float32 with fp16 matrix-core operands (the FP4 values
 * are exact in fp16; q and the SWA values e4m3 * scale are rounded to fp16).
 * Rounding q moves a logit by at most 2^-11 * scale * sum_c |q_c k_c|: far
 * inside the 2e-3 output bound for rows of the latent's range (|x| <=
 * sqrt(512) after RMSNorm), not for rows near the format's maximum (2688 in
 * every channel).  A q value with |q| >= 65520, NaN or Inf flags
 * CSA2_FLAG_Q_RANGE.
 */
csa2_status csa2_sparse_attend(const csa2_kv *kv, const float *q, int32_t heads,
                               const int32_t *idx, int32_t topk, float scale,
                               const csa2_swa *swa, float *out, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * csa2_prefill_workspace_bytes — workspace needed by csa2_prefill_attend,
 * with or without a local branch of any window up to CSA2_MAX_WINDOW (0
 * when every query is handled without partials).  Returns 0 as well for
 * unsupported sizes; csa2_prefill_attend reports why.
 */
size_t csa2_prefill_workspace_bytes(int32_t n_q, int32_t heads, int32_t topk);

/*
 * csa2_prefill_attend — batched prefill-side sparse attention: n_q queries
 * of sequence `seq`, query t at cache position qpos[t] with its own block
 * selection idx[t], each attending causally to the selected positions
 * p <= qpos[t] (its own position included).  The pages put the cost of long
 * inputs in the prefill [P2 introduction]; the per-query arithmetic is the
 * decode attention's (csa2_sparse_attend).
 * kv    cache view; seq in [0, batch): the sequence whose rows are read.
 *       Positions are also clamped below kv->max_len.
 * q     device float32 [n_q][heads][512], 16-byte aligned; heads 16/32/64.
 * qpos  device int64 [n_q]: cache position of each query.
 * idx   device int32 [n_q][topk], topk 1..CSA2_MAX_TOPK; -1 = none.  A block
 *       wholly after its query's position flags CSA2_FLAG_BAD_INDEX.
 * swa   NULL, or the layer's SWA cache (same batch; its ring of sequence
 *       `seq` is read): query t also attends, in the same softmax, to the
 *       positions max(0, qpos[t] - window + 1) .. qpos[t] of that ring.  They
 *       must have been written and not yet overwritten: below seq_len[seq]
 *       and at or above seq_len[seq] - slots (so a chunk of queries spanning
 *       S positions needs slots >= S + window - 1); positions outside are
 *       skipped and flag CSA2_FLAG_BAD_INDEX.
 * out   device float32 [n_q][heads][512].
 * ws    csa2_prefill_workspace_bytes(n_q, heads, topk) bytes, 256-byte
 *       aligned (may be NULL when that is 0).
 * n_q   1..65535.
 */
csa2_status csa2_prefill_attend(const csa2_kv *kv, int32_t seq, const float *q, int32_t n_q,
                                int32_t heads, const int64_t *qpos, const int32_t *idx,
                                int32_t topk, float scale, const csa2_swa *swa, float *out,
                                void *ws, size_t ws_bytes, void *stream);

/* One layer of a decode step. */
typedef struct {
  int32_t mode;        /* CSA2_FULL / CSA2_REINDEX / CSA2_REUSE                     */
  int32_t cache;       /* Full: its own cache; others: the latest Full layer's cache */
  const float *q;      /* device float32 [batch][heads][512]                        */
  float *out;          /* device float32 [batch][heads][512]                        */
  int32_t *idx;        /* device int32 [batch][topk]: this layer's selection        */
  const csa2_swa *swa; /* host pointer: this layer's SWA cache, or NULL (no local branch) */
  const float *swa_row;/* device float32 [batch][512]: the SWA row of the new token,
                          appended before the layers run; NULL = append nothing        */
} csa2_layer;

typedef struct {
  const csa2_kv *caches;     /* host array [n_caches]; all share batch          */
  int32_t n_caches;          /* 1..CSA2_MAX_CACHES                              */
  const csa2_layer *layers;  /* host array [n_layers]; layer 0 must be Full     */
  int32_t n_layers;
  const float *new_rows;     /* device float32 [n_caches][batch][512] appended
                                first (one position per sequence), or NULL      */
  int32_t heads, topk, pool; /* pool 0 = every selecting layer scans all blocks */
  float scale;               /* attention logit scale, e.g. 1/sqrt(512)         */
  int32_t *pool_out;         /* device int32 [batch][pool] (pool > 0)            */
  void *ws;
  size_t ws_bytes;
  int32_t score_rule;        /* CSA2_SCORE_SUM or CSA2_SCORE_HEADMAX, for every
                                selecting layer                                 */
} csa2_step;

/*
 * csa2_decode_step — layer-stack driver for one decode step [P2 CSA2
 * section; P3 section 二].  Appends new_rows into every Full cache, then
 * runs the layers in order: the first Full layer scans all blocks (into
 * the pool when pool > 0); later Full/Reindex layers search the pool (or
 * all blocks when pool == 0) of their cache; Reuse layers take the previous
 * layer's selection; every layer then attends over its selection, joined
 * by its sliding window when it has an SWA cache (at most
 * CSA2_MAX_SWA_LAYERS such layers; their swa_rows are appended in the same
 * launch as new_rows).
 * Capacity: each cache's max_len must already count the appended position.
 */
csa2_status csa2_decode_step(const csa2_step *step, void *stream);

/*
 * csa2_decode_step_noalloc — csa2_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same computation, but step->ws and
 * step->ws_bytes are ignored: the workspace is the library's own array of
 * CSA2_NOALLOC_WORKSPACE_BYTES (16 MiB) per device, held until the process
 * ends, zero-filled by a kernel on `stream` at the first call on each
 * device and re-zeroed like any workspace when the bounds change.  Enough
 * for batch 1 with 64 heads up to about 1.1M positions
 * (csa2_workspace_bytes gives the need); a larger step returns
 * CSA2_E_WORKSPACE before anything is queued.  The call allocates and frees
 * nothing.  Every call on a device shares that device's array: calls that
 * overlap on one device (different streams or threads) race and must be
 * ordered by the caller.
 */
#define CSA2_NOALLOC_WORKSPACE_BYTES (16u << 20)
csa2_status csa2_decode_step_noalloc(const csa2_step *step, void *stream);

/*
 * csa2_block_scores — diagnostic export of the indexer's float32 scores
 * (the same arithmetic as csa2_index_topk) under score_rule
 * (CSA2_SCORE_SUM or CSA2_SCORE_HEADMAX).
 * cand == NULL: scores[b][j] for every block j < ceil(max_len/8) (blocks at
 * or past a shorter sequence's end get -inf); else scores[b][j] for
 * cand[b][j], j < n_cand (-inf for -1 entries).
 * scores device float32 [batch][ceil(max_len/8)] or [batch][n_cand].
 */
csa2_status csa2_block_scores(const csa2_kv *kv, const float *q, int32_t heads,
                              const int32_t *cand, int32_t n_cand, float *scores,
                              int32_t score_rule, void *stream);

/*
 * csa2_device_error — synchronise `stream`, copy the device flag word of
 * the current device to *flags_host and clear it.
 */
csa2_status csa2_device_error(int32_t *flags_host, void *stream);

/*
 * csa2_set_scan_events — diagnostic timing hook.  While set (on this host
 * thread), every full-scan kernel launch records hipEvent_t `before` just
 * before it and `after` just after it on the launch's stream, so a caller
 * can time that kernel alone with hipEventElapsedTime.  NULL, NULL clears.
 */
csa2_status csa2_set_scan_events(void *before, void *after);

/*
 * csa2_read_probe — measurement aid: the achievable HBM read rate that the
 * full scan's rate is judged against.  Reads bytes (a multiple of 16, > 0)
 * of device memory at buf (16-byte aligned) once, with 16-byte loads
 * spread over 512 workgroups of 256 threads (the full scan's grid), and
 * writes 512 * 256 uint32 xor-reductions of what it read to sink (device,
 * 4-byte aligned; their values mean nothing) so no load is dropped.
 * Errors: CSA2_E_ARG for NULL or misaligned pointers or a bad size.
 */
csa2_status csa2_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

const char *csa2_status_string(csa2_status s);
/* Message of the last failing call on this thread ("" if none). */
const char *csa2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
