// Sparse softmax attention over the selected FP4 positions (gfx950).
//
// CSA2 attends only to the positions of the selected blocks (rebasdaily.com
// "DeepSeek-V4.1-Flash KV compression", section "same notes, many layers");
// the FP4 rows are dequantised inside the kernel from a fixed-stride layout
// (yomxxx.com long-form post, section 五).  Keys and values are both the
// 512-channel latent (ailily.cc "890 bytes per token", section 三), shared
// by all heads.
//
// Design (matrix cores, fp16 operands, fp32 accumulation):
//  * A workgroup (4 waves) takes one 16-head tile and a range of "stages"
//    of 64 gathered positions.  Per stage the 256 threads load the FP4 codes
//    and E4M3 scales of the 64 positions and write code*scale as fp16 rows
//    into LDS (exact: at most 6 significant bits, range 2^-10..2688).
//  * S^T = K Q^T on v_mfma_f32_16x16x32_f16 (K rows read from LDS with
//    b128 reads, Q in registers as fp16), one 16-position tile per wave;
//    online softmax in the exp2 domain with the stage's per-head max and
//    sum exchanged through LDS; P stored to LDS as fp16;
//    O^T += V^T P^T for 8 channel tiles per wave, V^T read straight from
//    the row-major LDS tile with ds_read_b64_tr_b16.
//  * Each workgroup writes its (max, sum, O) partial; a combine kernel
//    merges the partials of every head (split-K over positions).
//  * Optional local branch: the sliding window of the newest positions in
//    an FP8 (E4M3, float32 row scale) ring [rebasdaily.com, sections "halve
//    the long input" and "same notes, many layers"] is appended as further
//    stages of the same softmax; its rows are dequantised as e4m3 * scale
//    rounded to fp16 (rows need |x| <= 65504).
//  * Prefill side with 64 heads (many queries, each with its own
//    selection): attend64_kernel below covers all four head tiles of a
//    query in one workgroup, so each gathered row is dequantised once.
//  * The query is rounded to fp16 for the matrix cores: a logit moves by at
//    most 2^-11 * scale * sum_c |q_c k_c|, far inside the output bound for
//    rows of the latent's range (|x| <= sqrt(512) after RMSNorm); a query
//    value of magnitude 65520 or more (or not finite) has no fp16 value and
//    raises FLAG_Q_RANGE.
//
// MFMA 16x16x32 f16 lane layout (checked on gfx950): A row = lane%16 with
// k = 8*(lane/16)..+7; B column = lane%16, same k; C column = lane%16,
// rows 4*(lane/16)..+3.  ds_read_b64_tr_b16: within each 16-lane group,
// result lane i, element r comes from element i%4 of the 8 bytes addressed
// by lane 4r + i/4.
#include "common.hpp"

namespace csa2 {

constexpr int ATT_THREADS = 256;
constexpr int ATT_SP = 64;                        // gathered positions per stage
constexpr int ROW_HALVES = D;                     // LDS row stride: 1,024 bytes (swizzled chunks)

// P (fp16, heads x the stage's 64 positions) in LDS, laid out as the P.V
// matrix operand is read: lane (n16, g) of position chunk kk takes the 8
// values of positions 32 kk + 4 g + 0..3 and 32 kk + 16 + 4 g + 0..3 of
// head 16 * tile + n16, stored as one 16-byte vector, and the 16 heads of a
// (kk, g, tile) fill one 256-byte block: one conflict-free 128-bit read per
// operand (two 64-bit reads 32 or 144 bytes apart took twice as long).
// Returns the element offset (halves) of position pos of head 16 * tile + n16.
__device__ __forceinline__ int p_offset(int tile, int ntiles, int n16, int pos) {
  return ((((pos >> 5) * 4 + ((pos >> 2) & 3)) * ntiles + tile) * 16 + n16) * 8 + 4 * ((pos >> 4) & 1) + (pos & 3);
}

// LDS rows of a stage (and the staged query) are 64 chunks of 8 channels
// (16 bytes); chunk c of row p sits at chunk slot (c & ~15) | ((c ^ p) & 15)
// of the row.  Measured on gfx950 with the LDS bank-conflict counter: a
// 128-bit read by 16 lanes runs without conflict when the lanes hit 16
// distinct 16-byte slots of one 256-byte window (address bits 4-9; with a
// padded 1,040-byte row, the reads of 16 rows at one chunk straddle two
// windows and take twice as long), and a transposing 64-bit read by 32 lanes
// when they hit 32 distinct 8-byte slots of one window.  Rows of a
// 16-aligned group then put any one chunk in 16 distinct slots of the same
// window (the matrix operands' reads), and the two chunks c and c ^ 8 of
// eight rows fill a window (the V^T reads).  Returns the row's element
// offset in halves.
__device__ __forceinline__ int row_chunk(int p, int c) { return p * ROW_HALVES + 8 * ((c & ~15) | ((c ^ p) & 15)); }

// The matrix operands' 16-byte read: chunk 4 * kc + g of row p (channels
// 32 * kc + 8 * g .. +7), i.e. row_chunk(p, 4 * kc + g) written so that
// the four values of kc & 3 give four per-lane bases and kc >> 2 an
// immediate offset.
__device__ __forceinline__ int k_offset(int p, int kc, int g) {
  return p * ROW_HALVES + 128 * (kc >> 2) + 8 * ((4 * (kc & 3) + g) ^ (p & 15));
}

// The O^T tile ct (16 channels) covers chunks tile_chunk(ct) and
// tile_chunk(ct) ^ 8 of window ct & 3; its matrix row m holds channel
// 8 * (tile_chunk(ct) ^ (8 * (m / 8))) + m % 8, so lane (n16, g) of the
// accumulator holds the four channels from tile_channel(ct, g).  Tiles
// ct and ct + 1 sit in neighbouring windows at the same slots, so a wave's
// V^T reads of consecutive tiles differ by an immediate offset.
__device__ __forceinline__ int tile_chunk(int ct) { return 16 * (ct & 3) + (ct >> 2); }
__device__ __forceinline__ int tile_channel(int ct, int g) { return 8 * (tile_chunk(ct) ^ (8 * (g >> 1))) + 4 * (g & 1); }
// The transposing read of tile ct by the lane that points at row p and
// quarter q (channels 4 * (q & 1) .. +3 of chunk tile_chunk(ct) ^ (8 * (q >> 1))):
// row_chunk(p, tile_chunk(ct) ^ (8 * (q >> 1))) + 4 * (q & 1).
__device__ __forceinline__ int vt_offset(int p, int ct, int q) {
  return p * ROW_HALVES + 128 * (ct & 3) + 8 * ((((ct >> 2) | (8 * (q >> 1))) ^ p) & 15) + 4 * (q & 1);
}

// A thread dequantises 16 code bytes (chunks 4 * i16 .. 4 * i16 + 3 of its
// row) and stores them as four 16-byte chunks.  A 128-bit LDS write serves 8
// lanes at a time, without conflict when they hit 8 distinct 16-byte slots
// modulo 128 bytes; chunk 4 * i16 + s of row p falls in slot
// ((4 * i16 + s) ^ p) & 7, so each lane starts at chunk chunk_rot(i16) and
// wraps, which keeps the even lanes of any 8 on distinct slots, and the odd
// ones too.
__device__ __forceinline__ int chunk_rot(int i16) { return ((i16 >> 1) + (i16 >> 3)) & 3; }
// element s of the result is v[(s + rot) & 3]
__device__ __forceinline__ u32x4 rotate4(u32x4 v, int rot) {
  if (rot & 1) v = u32x4{v[1], v[2], v[3], v[0]};
  if (rot & 2) v = u32x4{v[2], v[3], v[0], v[1]};
  return v;
}

// A split's O^T accumulators (four channels of one head) divided by that
// head's sum, as fp16: the normalised values are averages of V rows, so they
// stay within fp16 range, and the combine re-weights them by the sums.
__device__ __forceinline__ u32x2 pack_partial(f32x4 v, float inv) {
  const f16x2 lo = {(_Float16)(v[0] * inv), (_Float16)(v[1] * inv)};
  const f16x2 hi = {(_Float16)(v[2] * inv), (_Float16)(v[3] * inv)};
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
// (the words are copied to scalars before the bit casts: this compiler
// turned a bit cast of a vector element u[1] into a read of u[0])
__device__ __forceinline__ float4 unpack_partial(u32x2 u) {
  const uint32_t w0 = u.x, w1 = u.y;
  const f16x2 lo = __builtin_bit_cast(f16x2, w0);
  const f16x2 hi = __builtin_bit_cast(f16x2, w1);
  return float4{(float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y};
}

struct AttendArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const int64_t *seq_len;
  int64_t capacity;
  int64_t limit;            // min(capacity, max_len)
  const float *q;           // [batch][heads][512]
  const int32_t *idx;       // [batch][topk]
  int32_t topk;
  int32_t heads;            // 16, 32 or 64
  float scale_log2;         // scale * log2(e)
  int32_t n_stages;         // n_sparse + ceil(window / ATT_SP)
  int32_t splits;           // workgroups per (sequence, head tile)
  _Float16 *part_o;         // [batch][splits][heads/16][32 tiles][64 lanes][4]: O^T of the split
                            // divided by its sum (so |O| <= max |V|), fp16, in lane order
                            // (contiguous stores)
  float *part_ml;           // [batch][splits][heads/16][16 heads][2]: running max (log2) and sum
  // selecting variant only: the top-k is taken inside the kernel from a
  // scored candidate list (every workgroup takes the same, deterministic
  // choice; the first workgroup of each sequence also writes it to idx_out)
  const int32_t *cand;      // [batch][n_cand] block ids (-1 = empty)
  const float *cand_scores; // [batch][n_cand] their indexer scores
  int32_t n_cand;           // 1..SEL_CAND_MAX
  int32_t *idx_out;         // [batch][topk]
  // batch row b of the cache is at codes + b * seq_stride rows (capacity for
  // decode; 0 when every row b is a query of one sequence, prefill side)
  int64_t seq_stride;
  int32_t len_add;          // valid positions of row b: seq_len[b] + len_add
  float *out;               // splits == 1: final output [batch][heads][512] written here
  // local branch: stages n_sparse .. n_stages-1 hold up to `window`
  // positions of an FP8 ring (position p in slot p % swa_slots), attended in
  // the same softmax as the gathered ones.  The window ends at the ring's
  // length (decode) or, with win_at_query, at row b's own length
  // seq_len[b] + len_add (prefill); only positions still in the ring
  // (below its length, at or above length - swa_slots) are read.
  int32_t n_sparse;         // stages of gathered positions: ceil(topk*8 / ATT_SP)
  int32_t window;           // 0 = no local branch
  int32_t swa_slots;        // ring positions (>= window)
  int32_t swa_stride;       // rings per row b: 1 (decode), 0 (prefill: one sequence's ring)
  int32_t win_at_query;
  const uint8_t *swa_codes; // [rows][swa_slots][512] E4M3
  const float *swa_scales;  // [rows][swa_slots]
  const int64_t *swa_len;   // [rows]; any valid int64 array when window == 0
};

constexpr int SEL_CAND_MAX = 2048;  // candidates of the in-kernel top-k (8 per thread)

// A lane's value combined with that of lane ^ 16 (or lane ^ 32) by the
// permlane swap instructions: VALU lane moves, no LDS round trip as with a
// bpermute.  With the value in both operands the two results hold the lane's
// own value and its partner's (in an order that differs between lanes; max
// and sum are symmetric, so every lane gets the same result as own (op) partner).
template <int X>
__device__ __forceinline__ f32x2 xor_lanes_pair(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto s = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return f32x2{__uint_as_float(s[0]), __uint_as_float(s[1])};
}
template <int X>
__device__ __forceinline__ float xor_lanes_max(float v) {
  const f32x2 p = xor_lanes_pair<X>(v);
  return fmaxf(p.x, p.y);
}
template <int X>
__device__ __forceinline__ float xor_lanes_sum(float v) {
  const f32x2 p = xor_lanes_pair<X>(v);
  return p.x + p.y;
}

// One workgroup = one 16-head tile x a range of stages of 64 gathered
// positions.  Per stage: the 256 threads dequantise the 64 rows into LDS as
// fp16; wave w computes S^T for positions 16w..16w+15 (16 MFMA k-steps);
// the per-head max and sum of the stage are exchanged through LDS; P is
// written to LDS as fp16; wave w then accumulates O^T for channel tiles
// 8w..8w+7 over all 64 positions.
template <bool SELECT, bool WIN>
__global__ void __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(2))) attend_partial_kernel(AttendArgs a) {
  // 16-byte aligned: rows are read and written as 128-bit vectors
  extern __shared__ __attribute__((aligned(16))) _Float16 s_v[];   // [ATT_SP][ROW_HALVES]; first holds q
  __shared__ __attribute__((aligned(16))) _Float16 s_p[16 * ATT_SP];   // P of 16 heads (p_offset)
  __shared__ float s_max[4][16], s_sum[4][16];
  __shared__ uint8_t s_ok[ATT_SP];
  __shared__ int32_t s_sel[SELECT ? CSA2_TOPK_MAX + SEL_PAD : 1];   // in-kernel selection
  __shared__ uint64_t s_state[2];
  __shared__ uint32_t s_wave[16];

  const int b = blockIdx.y;
  const int HT = a.heads >> 4;
  const uint32_t wx = wg_x();
  const int ht = wx % HT, split = wx / HT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  // The sequence length is only needed to mask positions: loads are bounded
  // by the cache capacity, so they are issued without waiting for it.
  const int64_t cap_blocks = a.capacity / BLOCK;  // blocks a load may touch
  const int32_t *idx = a.idx + (int64_t)b * a.topk;
  const uint8_t *codes = a.codes + (int64_t)b * a.seq_stride * CODE_BYTES;
  const uint8_t *scales = a.scales + (int64_t)b * a.seq_stride * SCALE_BYTES;
  const int total_pos = a.topk * BLOCK;
  const int st0 = (int)((int64_t)a.n_stages * split / a.splits);
  const int st1 = (int)((int64_t)a.n_stages * (split + 1) / a.splits);
  CSA2_CHECK(split < a.splits && st0 < st1 && st1 <= a.n_stages && a.topk <= CSA2_TOPK_MAX);
  // local branch: read now, with the first ids, so that the window rows'
  // addresses are known when the first window stage is fetched
  const int64_t wlen_raw = WIN ? a.swa_len[(int64_t)b * a.swa_stride] : 0;
  const int64_t wq_raw = WIN && a.win_at_query ? a.seq_len[b] + a.len_add : 0;

  // ---- gathered rows of a stage: block ids, then rows (two round trips) --
  constexpr int PASSES = ATT_SP / 16;     // rows per thread per stage
  const int i16 = tid & 15;               // this thread's 16-byte column of a row
  // (the window variants keep the plain order: the rotation's registers
  // would halve their occupancy)
  const int rot = WIN ? 0 : chunk_rot(i16);
  const bool rhi0 = (rot & 2) != 0, rhi1 = ((rot + 1) & 2) != 0;   // chunk rot, rot + 1 (mod 4) >= 2
  int32_t blkv[PASSES];
  bool okv[PASSES];
  u32x4 wr[PASSES];
  uint32_t scr[PASSES];
  auto fetch_ids_into = [&](int st, int32_t (&dst)[PASSES]) {
    if (WIN && st >= a.n_sparse) {               // window stage: the position's index in the window
#pragma unroll
      for (int k = 0; k < PASSES; ++k) dst[k] = (st - a.n_sparse) * ATT_SP + (tid >> 4) + 16 * k;
      return;
    }
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int j = st * ATT_SP + (tid >> 4) + 16 * k;
      if (SELECT)
        dst[k] = s_sel[min(j, total_pos - 1) >> 3];
      else
        dst[k] = idx[min(j, total_pos - 1) >> 3];    // unconditional: one batch
    }
  };
  auto fetch_ids = [&](int st) { fetch_ids_into(st, blkv); };
  int32_t nxt[PASSES];                    // block ids of the stage after the one in flight
  u32x4 wr2[PASSES];                      // window rows: second 16 bytes of the thread's 32
  // window: nw positions from wfirst; those in [wlo, wrl) are in the ring;
  // wbase = slot of wfirst
  int64_t nw = 0, wbase = 0, wfirst = 0, wlo = 0, wrl = 0;
  const uint8_t *wcodes = a.swa_codes + (int64_t)b * a.swa_stride * a.swa_slots * D;
  const float *wscales = a.swa_scales + (int64_t)b * a.swa_stride * a.swa_slots;
  auto fetch_rows = [&](int st) {
    if (WIN && st >= a.n_sparse) {
      // window rows: 512 code bytes (32 per thread) and the row scale
#pragma unroll
      for (int k = 0; k < PASSES; ++k) {
        const int64_t p = wfirst + blkv[k];
        okv[k] = blkv[k] < nw && p >= wlo && p < wrl;
        int64_t slot = wbase + blkv[k];
        slot = okv[k] ? (slot >= a.swa_slots ? slot - a.swa_slots : slot) : 0;
        CSA2_CHECK(slot >= 0 && slot < a.swa_slots);
        const uint8_t *row = wcodes + slot * D + 32 * i16;
        wr[k] = *reinterpret_cast<const u32x4 *>(row);
        wr2[k] = *reinterpret_cast<const u32x4 *>(row + 16);
        scr[k] = __float_as_uint(wscales[slot]);
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      // in bounds (masked by the sequence length later); an id outside the
      // cache reads row 0 and is dropped, so every load is unconditional and
      // the stage's loads go out as one batch
      if (st * ATT_SP + (tid >> 4) + 16 * k >= total_pos) blkv[k] = -1;   // past the selection
      okv[k] = blkv[k] >= 0 && blkv[k] < cap_blocks;
      const int64_t pos = okv[k] ? (int64_t)blkv[k] * BLOCK + (((tid >> 4) + 16 * k) & 7) : 0;
      wr[k] = *reinterpret_cast<const u32x4 *>(codes + pos * CODE_BYTES + 16 * i16);
      scr[k] = *reinterpret_cast<const uint16_t *>(scales + pos * SCALE_BYTES + 2 * i16);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  CSA2_TS(0);
  // the tile's 16 query rows (32 KB), 8 float4 per thread
  constexpr int NV = 16 * D / 4 / ATT_THREADS;
  const float4 *qsrc = reinterpret_cast<const float4 *>(a.q + ((int64_t)b * a.heads + 16 * ht) * D);
  float4 v[NV];
  // Selecting variant: candidates, their scores and the sequence length in
  // one batch, then the block top-k in LDS (the key/id/bin arrays borrow the
  // row buffer, which is free until the query is staged).  The query rows
  // are requested right behind the candidates: the in-order memory counter
  // lets the top-k start once the candidates are in, and the query's latency
  // hides behind the selection.
  if constexpr (SELECT) {
    constexpr int KPT = SEL_CAND_MAX / ATT_THREADS;
    const int m = a.n_cand;
    CSA2_CHECK(m >= 1 && m <= SEL_CAND_MAX);
    const int32_t *cb = a.cand + (int64_t)b * m;
    const float *sb = a.cand_scores + (int64_t)b * m;
    int32_t cid[KPT];
    float csc[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int j = min(64 * KPT * wv + 64 * k + lane, m - 1);     // wave wv: a quarter of the list
      cid[k] = cb[j];
      csc[k] = sb[j];
    }
    const int64_t nsel = clamp_len(a.seq_len[b] + a.len_add, a.limit);
#pragma unroll
    for (int u = 0; u < NV; ++u) v[u] = qsrc[tid + u * ATT_THREADS];
    __builtin_amdgcn_sched_barrier(0);
    const int64_t nbs = (nsel + BLOCK - 1) / BLOCK;
    uint64_t *s_keys = reinterpret_cast<uint64_t *>(s_v);     // for the radix fallback only
    uint32_t *s_hist = reinterpret_cast<uint32_t *>(s_keys + SEL_CAND_MAX);
    static_assert(SEL_CAND_MAX * sizeof(uint64_t) + TOPK_HIST_BINS * sizeof(uint32_t) <=
                      (size_t)ATT_SP * ROW_HALVES * sizeof(_Float16),
                  "the selection's keys and bins fit in the row buffer");
    uint64_t kr[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int j = 64 * KPT * wv + 64 * k + lane;
      const bool ok = j < m && cid[k] >= 0 && cid[k] < nbs;
      kr[k] = ok ? make_key(csc[k], (uint32_t)cid[k]) : 0ull;
      if (j < m) s_keys[j] = kr[k];
    }
    int32_t *io = wx == 0 ? a.idx_out + (int64_t)b * a.topk : nullptr;
    select_top_regs<KPT>(kr, csc, cid, s_keys, m, a.topk, io, s_sel, a.topk, s_hist, s_state, s_wave);
  }
  // request order: the first stage's block ids, the query tile, then (once
  // the ids are in) the rows, so the query and id latencies overlap
  // every split owns at least one stage (splits <= stages)
  fetch_ids(st0);
  __builtin_amdgcn_sched_barrier(0);
  CSA2_TS(24);

  // ---- Q^T operand: head 16*ht + n16, channels 32*kc + 8*g + 0..7.  The
  // tile's 16 query rows (32 KB) are staged through LDS as fp16 with one
  // batch of coalesced float4 loads per thread, then read into registers.
  f16x8 qop[16];
  {
    if constexpr (!SELECT) {
#pragma unroll
      for (int u = 0; u < NV; ++u) v[u] = qsrc[tid + u * ATT_THREADS];
    }
    __builtin_amdgcn_sched_barrier(0);    // query loads go out before the ids are awaited
    if (WIN) {
      wrl = wlen_raw < 0 ? 0 : wlen_raw;                      // positions in the ring
      wlo = wrl - a.swa_slots;                                // older ones are overwritten
      const int64_t wend = a.win_at_query ? (wq_raw < 0 ? 0 : wq_raw) : wrl;
      nw = wend < a.window ? wend : a.window;
      wfirst = wend - nw;
      wbase = wfirst % a.swa_slots;
      if (tid == 0 && nw > 0 && (wfirst < wlo || wend > wrl)) raise_flag(FLAG_BAD_INDEX);
    }
    fetch_rows(st0);
    if (st0 + 1 < st1) fetch_ids_into(st0 + 1, nxt);
    CSA2_TS(25);
    uint32_t mb = 0;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = tid + u * ATT_THREADS;                    // head e/128, channels 4*(e%128)
      mb = max(mb, max(max(__float_as_uint(v[u].x) & 0x7fffffffu, __float_as_uint(v[u].y) & 0x7fffffffu),
                       max(__float_as_uint(v[u].z) & 0x7fffffffu, __float_as_uint(v[u].w) & 0x7fffffffu)));
      f16x2 lo = {(_Float16)v[u].x, (_Float16)v[u].y}, hi = {(_Float16)v[u].z, (_Float16)v[u].w};
      *reinterpret_cast<u32x2 *>(s_v + row_chunk(e >> 7, (e & 127) >> 1) + 4 * (e & 1)) =
          u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
    // no fp16 value for |q| >= 65520 (or NaN/Inf): flag it
    if (__builtin_amdgcn_ballot_w64(mb >= 0x477ff000u) && lane == 0) raise_flag(FLAG_Q_RANGE);
    CSA2_TS(26);
    __syncthreads();
    CSA2_TS(27);
#pragma unroll
    for (int kc = 0; kc < 16; ++kc) qop[kc] = *reinterpret_cast<const f16x8 *>(s_v + k_offset(n16, kc, g));
  }

  const int64_t n = clamp_len(a.seq_len[b] + a.len_add, a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;
  CSA2_TS(1);
  f32x4 acc[8];                           // O^T tiles 8*wv .. 8*wv+7
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf();   // running max of head n16 (log2 domain)
  float l_run = 0.f;                      // running sum of head n16

  // V^T operand: rows (k) of chunk kk are positions 32*kk + 4g + 0..3 then
  // 32*kk + 16 + 4g + 0..3; source lane s = 4r + q points at row k0 + r,
  // channels 4 * (q & 1) .. +3 of chunk tile_chunk(ct) ^ (8 * (q >> 1)), so
  // row m of O^T tile ct holds channel 8 * (tile_chunk(ct) ^ (8 * (m / 8))) + m % 8.
  const int r_src = n16 >> 2, q_src = n16 & 3;

#pragma unroll 1
  for (int st = st0; st < st1; ++st) {
    __syncthreads();                      // q / previous stage fully consumed
    // ---- dequantise the stage's rows into LDS as fp16 (16 threads per row) ----
    if (WIN && st >= a.n_sparse) {
      // window rows: e4m3 * row scale, rounded to fp16 (16 threads per row,
      // 32 channels each)
#pragma unroll
      for (int k = 0; k < PASSES; ++k) {
        const int pp = (tid >> 4) + 16 * k;
        if (!okv[k]) { wr[k] = u32x4{0u, 0u, 0u, 0u}; wr2[k] = wr[k]; }   // masked: finite zeros
        const float sc = okv[k] ? __uint_as_float(scr[k]) : 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = h ? wr2[k] : wr[k];
          uint32_t o[8];
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[dw], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[dw], true);
            const f16x2 a0 = {(_Float16)(lo.x * sc), (_Float16)(lo.y * sc)};
            const f16x2 a1 = {(_Float16)(hi.x * sc), (_Float16)(hi.y * sc)};
            o[2 * dw] = __builtin_bit_cast(uint32_t, a0);
            o[2 * dw + 1] = __builtin_bit_cast(uint32_t, a1);
          }
          *reinterpret_cast<u32x4 *>(s_v + row_chunk(pp, 4 * i16 + 2 * h)) = u32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<u32x4 *>(s_v + row_chunk(pp, 4 * i16 + 2 * h + 1)) = u32x4{o[4], o[5], o[6], o[7]};
        }
        if (i16 == 0) s_ok[pp] = okv[k] ? 1 : 0;
      }
    } else {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int pp = (tid >> 4) + 16 * k;
      const int j = st * ATT_SP + pp;
      const int32_t blk = blkv[k];
      if ((j & 7) == 0 && i16 == 0 && blk >= nblk) raise_flag(FLAG_BAD_INDEX);
      okv[k] = blk >= 0 && blk < nblk && (int64_t)blk * BLOCK + (j & 7) < n;
      if (!okv[k]) { wr[k] = u32x4{0u, 0u, 0u, 0u}; scr[k] = 0u; }
      const _Float16 s0 = (_Float16)e4m3_to_f32(scr[k] & 0xffu);
      const _Float16 s1 = (_Float16)e4m3_to_f32(scr[k] >> 8);
      const f16x2 sv0 = {s0, s0}, sv1 = {s1, s1};
      const u32x4 wrot = rotate4(wr[k], rot);
      // chunk (s + rot) & 3 takes scale 1 when it is 2 or 3
      const f16x2 svr[4] = {rhi0 ? sv1 : sv0, rhi1 ? sv1 : sv0, rhi0 ? sv0 : sv1, rhi1 ? sv0 : sv1};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int dw = (s + rot) & 3;
        const uint32_t w = wrot[s];
        const f16x2 sv = svr[s];
        f16x2 h0 = e2m1x2_to_f16<0>(w) * sv;
        f16x2 h1 = e2m1x2_to_f16<1>(w) * sv;
        f16x2 h2 = e2m1x2_to_f16<2>(w) * sv;
        f16x2 h3 = e2m1x2_to_f16<3>(w) * sv;
        *reinterpret_cast<u32x4 *>(s_v + row_chunk(pp, 4 * i16 + dw)) =
            u32x4{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                  __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
      }
      if (i16 == 0) s_ok[pp] = okv[k] ? 1 : 0;
    }
    }
    // the next stage's rows (and the ids of the one after) are requested now,
    // so they arrive while this stage is computed
    if (st + 1 < st1) {
#pragma unroll
      for (int k = 0; k < PASSES; ++k) blkv[k] = nxt[k];
      fetch_rows(st + 1);
      if (st + 2 < st1) fetch_ids_into(st + 2, nxt);
    }
    __syncthreads();

    CSA2_TS(2);
    // ---- S^T for positions 16*wv .. 16*wv+15 ----
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    {
#pragma unroll
      for (int kc = 0; kc < 16; ++kc) {
        f16x8 kop = *reinterpret_cast<const f16x8 *>(s_v + k_offset(16 * wv + n16, kc, g));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[kc], sacc, 0, 0, 0);
      }
    }
    // lane (head n16, group g) holds positions 16*wv + 4g + r
    float z[4];
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = s_ok[16 * wv + 4 * g + r] ? sacc[r] * a.scale_log2 : -__builtin_huge_valf();
      mx = fmaxf(mx, z[r]);
    }
    mx = xor_lanes_max<16>(mx);
    mx = xor_lanes_max<32>(mx);
    if (g == 0) s_max[wv][n16] = mx;
    __syncthreads();
    const float m_new = fmaxf(m_run, fmaxf(fmaxf(s_max[0][n16], s_max[1][n16]),
                                           fmaxf(s_max[2][n16], s_max[3][n16])));
    _Float16 ph[4];
    float psum = 0.f, corr = 1.f;
    if (m_new == -__builtin_huge_valf()) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ph[r] = (_Float16)0.f;
    } else {
      corr = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ph[r] = (_Float16)__builtin_amdgcn_exp2f(z[r] - m_new);
        psum += (float)ph[r];
      }
    }
    *reinterpret_cast<u32x2 *>(s_p + p_offset(0, 1, n16, 16 * wv + 4 * g)) =
        u32x2{__builtin_bit_cast(uint32_t, f16x2{ph[0], ph[1]}),
              __builtin_bit_cast(uint32_t, f16x2{ph[2], ph[3]})};
    psum = xor_lanes_sum<16>(psum);
    psum = xor_lanes_sum<32>(psum);
    if (g == 0) s_sum[wv][n16] = psum;
    __syncthreads();
    CSA2_TS(3);
    l_run = l_run * corr + ((s_sum[0][n16] + s_sum[1][n16]) + (s_sum[2][n16] + s_sum[3][n16]));
    m_run = m_new;
    if (corr != 1.f) {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= corr;
    }

    // ---- O^T tiles 8*wv .. 8*wv+7 over the stage's 64 positions ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int base = 32 * kk;
      const f16x8 pop = *reinterpret_cast<const f16x8 *>(s_p + p_offset(0, 1, n16, base + 4 * g));
      const int vrow = base + 4 * g + r_src;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ct = 8 * wv + t;
        const _Float16 *v0 = s_v + vt_offset(vrow, ct, q_src);
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(v0));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(v0 + 16 * ROW_HALVES));
        f16x8 vop = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop, acc[t], 0, 0, 0);
      }
    }
  }

  CSA2_TS(4);
  if (a.splits == 1) {
    // one workgroup holds the whole softmax of its heads: normalise here.
    // lane (n16, g) of tile ct holds channels tile_channel(ct, g) + 0..3
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float *orow = a.out + ((int64_t)b * a.heads + 16 * ht + n16) * D;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int ct = 8 * wv + t;
      *reinterpret_cast<float4 *>(orow + tile_channel(ct, g)) =
          float4{acc[t][0] * inv, acc[t][1] * inv, acc[t][2] * inv, acc[t][3] * inv};
    }
    CSA2_TS(5);
    return;
  }
  // ---- partial of this (sequence, split, head tile) ----
  // fp16, normalised by the split's sum: half the bytes of float32
  // accumulators to write here and to read in the combine (a 20-layer step
  // at 1M: 0.420 -> 0.402 ms).  Ordinary stores for them (0.399 ms; streaming
  // stores helped while they were float32); the (max, sum) pairs stream.
  const int64_t slot = ((int64_t)b * a.splits + split) * HT + ht;
  u32x2 *po = reinterpret_cast<u32x2 *>(a.part_o) + slot * (16 * D / 4) + lane;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) po[(8 * wv + t) * 64] = pack_partial(acc[t], inv);
  if (wv == 0 && g == 0) {
    float *pm = a.part_ml + (slot * 16 + n16) * 2;
    __builtin_nontemporal_store(m_run, &pm[0]);
    __builtin_nontemporal_store(l_run, &pm[1]);
  }
  CSA2_TS(5);
}

template __global__ void attend_partial_kernel<false, false>(AttendArgs);
template __global__ void attend_partial_kernel<true, false>(AttendArgs);
template __global__ void attend_partial_kernel<false, true>(AttendArgs);
template __global__ void attend_partial_kernel<true, true>(AttendArgs);

// ---- 64 heads per workgroup (prefill side) ------------------------------
//
// Many queries, each with its own selection: one workgroup takes one query
// and a range of stages for all four 16-head tiles, so a gathered row is
// dequantised once for 64 heads.  Eight waves in two roles, one of each per
// SIMD, so that one role's matrix instructions run beside the other's vector
// work:
//  * producer wave w < 4 (head tile w): S^T = K Q^T of its 16 heads over
//    all 64 positions of the stage (its query rows in registers as fp16,
//    K fragments from LDS), masked and scaled, to LDS; then it dequantises
//    a quarter of the next stage's rows into the other stage buffer and
//    requests the rows of the stage after;
//  * consumer wave 4 + w (head tile w): the online softmax of its 16 heads
//    over the stage (the S values a lane reads are exactly the P.V operand
//    it needs, so P stays in registers) and O^T for all 32 channel tiles,
//    V^T read with the transposing read.
// Two workgroup barriers per stage: stage ready (and the S buffer free),
// then S ready.  The consumers' P.V and the producers' dequantisation of the
// next stage overlap.
constexpr int ATT64_THREADS = 512;
constexpr size_t ATT64_LDS = (size_t)2 * ATT_SP * ROW_HALVES * sizeof(_Float16);
__global__ void __launch_bounds__(ATT64_THREADS) attend64_kernel(AttendArgs a) {
  // 16-byte aligned: rows are read and written as 128-bit vectors
  extern __shared__ __attribute__((aligned(16))) _Float16 s_v[];   // [2][ATT_SP][ROW_HALVES]; first holds q (64 heads)
  // S of the stage: [head tile][position tile u][lane][4], in the matrix
  // accumulator's lane order (lane (n16, g): head n16, positions 16 u + 4 g + 0..3)
  __shared__ __attribute__((aligned(16))) float s_s[4 * 4 * 64 * 4];
  __shared__ uint8_t s_ok[2][ATT_SP];

  const int b = blockIdx.y, split = wg_x();
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const bool producer = wv < 4;                   // wave-uniform role
  const int ht = wv & 3;                          // the wave's head tile
  const int64_t cap_blocks = a.capacity / BLOCK;
  const int32_t *idx = a.idx + (int64_t)b * a.topk;
  const uint8_t *codes = a.codes + (int64_t)b * a.seq_stride * CODE_BYTES;
  const uint8_t *scales = a.scales + (int64_t)b * a.seq_stride * SCALE_BYTES;
  const int total_pos = a.topk * BLOCK;
  const int st0 = (int)((int64_t)a.n_stages * split / a.splits);
  const int st1 = (int)((int64_t)a.n_stages * (split + 1) / a.splits);
  CSA2_CHECK(split < a.splits && st0 < st1 && st1 <= a.n_stages && a.topk <= CSA2_TOPK_MAX);

  // producers: rows (tid >> 4) + 16 k of a stage, 16 code bytes each
  constexpr int PASSES = ATT_SP / 16;
  const int i16 = tid & 15;
  const int rot = chunk_rot(i16);
  const bool rhi0 = (rot & 2) != 0, rhi1 = ((rot + 1) & 2) != 0;   // chunk rot, rot + 1 (mod 4) >= 2
  int32_t blkv[PASSES], nxt[PASSES];
  u32x4 wr[PASSES];
  uint32_t scr[PASSES];
  auto fetch_ids_into = [&](int st, int32_t (&dst)[PASSES]) {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int j = st * ATT_SP + (tid >> 4) + 16 * k;
      dst[k] = idx[min(j, total_pos - 1) >> 3];
    }
  };
  auto fetch_rows = [&](int st) {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      if (st * ATT_SP + (tid >> 4) + 16 * k >= total_pos) blkv[k] = -1;
      const bool ok = blkv[k] >= 0 && blkv[k] < cap_blocks;
      const int64_t pos = ok ? (int64_t)blkv[k] * BLOCK + (((tid >> 4) + 16 * k) & 7) : 0;
      wr[k] = *reinterpret_cast<const u32x4 *>(codes + pos * CODE_BYTES + 16 * i16);
      scr[k] = *reinterpret_cast<const uint16_t *>(scales + pos * SCALE_BYTES + 2 * i16);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  CSA2_TS(0);
  if (producer) fetch_ids_into(st0, blkv);
  __builtin_amdgcn_sched_barrier(0);

  // One register array serves both roles (a wave uses one branch only, but
  // the compiler allocates for both): a consumer's O^T accumulators, tiles
  // 0..31; a producer's query operand, 16 steps of 8 channels as fp16
  // (reg[kc], bit-cast).
  f32x4 reg[32];
  // ---- the query's 64 x 512 tile -> fp16 in LDS (one batch of 16 float4
  // per thread), then each producer's 16 rows of its head tile into registers
  {
    constexpr int NV = 16;
    const float4 *src = reinterpret_cast<const float4 *>(a.q + (int64_t)b * 64 * D);
    float4 v[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) v[u] = src[tid + u * ATT64_THREADS];
    __builtin_amdgcn_sched_barrier(0);
    if (producer) {
      fetch_rows(st0);
      if (st0 + 1 < st1) fetch_ids_into(st0 + 1, nxt);
    }
    uint32_t mb = 0;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = tid + u * ATT64_THREADS;                  // head e/128, channels 4*(e%128)
      mb = max(mb, max(max(__float_as_uint(v[u].x) & 0x7fffffffu, __float_as_uint(v[u].y) & 0x7fffffffu),
                       max(__float_as_uint(v[u].z) & 0x7fffffffu, __float_as_uint(v[u].w) & 0x7fffffffu)));
      f16x2 lo = {(_Float16)v[u].x, (_Float16)v[u].y}, hi = {(_Float16)v[u].z, (_Float16)v[u].w};
      *reinterpret_cast<u32x2 *>(s_v + row_chunk(e >> 7, (e & 127) >> 1) + 4 * (e & 1)) =
          u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
    // no fp16 value for |q| >= 65520 (or NaN/Inf): flag it
    if (__builtin_amdgcn_ballot_w64(mb >= 0x477ff000u) && lane == 0) raise_flag(FLAG_Q_RANGE);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 32; ++t) reg[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (producer) {
#pragma unroll
      for (int kc = 0; kc < 16; ++kc)
        reg[kc] = *reinterpret_cast<const f32x4 *>(s_v + k_offset(16 * ht + n16, kc, g));
    }
  }

  const int64_t n = clamp_len(a.seq_len[b] + a.len_add, a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;

  // producers: dequantise stage st (its rows are in wr/scr) into buffer
  // `buf`, then request the rows of stage st + 1 (ids in nxt) and the ids of
  // st + 2
  auto dequant_and_fetch = [&](int st, int buf) {
    _Float16 *sv = s_v + buf * (ATT_SP * ROW_HALVES);
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int pp = (tid >> 4) + 16 * k;
      const int j = st * ATT_SP + pp;
      const int32_t blk = blkv[k];
      if ((j & 7) == 0 && i16 == 0 && blk >= nblk) raise_flag(FLAG_BAD_INDEX);
      const bool ok = blk >= 0 && blk < nblk && (int64_t)blk * BLOCK + (j & 7) < n;
      if (!ok) { wr[k] = u32x4{0u, 0u, 0u, 0u}; scr[k] = 0u; }
      const _Float16 s0 = (_Float16)e4m3_to_f32(scr[k] & 0xffu);
      const _Float16 s1 = (_Float16)e4m3_to_f32(scr[k] >> 8);
      const f16x2 sv0 = {s0, s0}, sv1 = {s1, s1};
      const u32x4 wrot = rotate4(wr[k], rot);
      const f16x2 svr[4] = {rhi0 ? sv1 : sv0, rhi1 ? sv1 : sv0, rhi0 ? sv0 : sv1, rhi1 ? sv0 : sv1};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int dw = (s + rot) & 3;
        const uint32_t w = wrot[s];
        const f16x2 svs = svr[s];
        f16x2 h0 = e2m1x2_to_f16<0>(w) * svs;
        f16x2 h1 = e2m1x2_to_f16<1>(w) * svs;
        f16x2 h2 = e2m1x2_to_f16<2>(w) * svs;
        f16x2 h3 = e2m1x2_to_f16<3>(w) * svs;
        *reinterpret_cast<u32x4 *>(sv + row_chunk(pp, 4 * i16 + dw)) =
            u32x4{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                  __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
      }
      if (i16 == 0) s_ok[buf][pp] = ok ? 1 : 0;
    }
    if (st + 1 < st1) {
#pragma unroll
      for (int k = 0; k < PASSES; ++k) blkv[k] = nxt[k];
      fetch_rows(st + 1);
      if (st + 2 < st1) fetch_ids_into(st + 2, nxt);
    }
  };
  __syncthreads();                        // the producers hold their query rows: buffer 0 is free
  if (producer) dequant_and_fetch(st0, 0);

  CSA2_TS(1);
  f32x4 (&acc)[32] = reg;                 // consumers: O^T tiles 0..31 of head tile ht
  float m_run = -__builtin_huge_valf();   // consumers: head 16*ht + n16 (log2 domain)
  float l_run = 0.f;
  const int r_src = n16 >> 2, q_src = n16 & 3;
  f32x4 *s_mine = reinterpret_cast<f32x4 *>(s_s) + (ht * 4) * 64 + lane;   // [u * 64]

#pragma unroll 1
  for (int st = st0; st < st1; ++st) {
    const int cur = (st - st0) & 1;
    const _Float16 *sv = s_v + cur * (ATT_SP * ROW_HALVES);
    __syncthreads();                      // stage st is in buffer cur; buffer cur^1 and s_s are free
    CSA2_TS(2);
    if (producer) {
      // ---- S^T of head tile ht over the stage's 4 position tiles ----
      // (the K fragments of step kc + 2 are requested before step kc's four
      // matrix instructions; the scheduling barriers keep the register
      // footprint to three steps)
      f32x4 sacc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      f16x8 k0[4], k1[4], k2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        k0[u] = *reinterpret_cast<const f16x8 *>(sv + k_offset(16 * u + n16, 0, g));
        k1[u] = *reinterpret_cast<const f16x8 *>(sv + k_offset(16 * u + n16, 1, g));
      }
#pragma unroll
      for (int kc = 0; kc < 16; ++kc) {
        if (kc + 2 < 16) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            k2[u] = *reinterpret_cast<const f16x8 *>(sv + k_offset(16 * u + n16, kc + 2, g));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0[u], __builtin_bit_cast(f16x8, reg[kc]), sacc[u], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) { k0[u] = k1[u]; k1[u] = k2[u]; }
      }
      // lane (head n16, group g) holds positions 16 u + 4 g + r
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sacc[u][r] = s_ok[cur][16 * u + 4 * g + r] ? sacc[u][r] * a.scale_log2 : -__builtin_huge_valf();
        s_mine[u * 64] = sacc[u];
      }
    }
    __syncthreads();                      // S of the stage is in s_s
    CSA2_TS(3);
    if (producer) {
      // the next stage's rows, while the consumers run P.V
      if (st + 1 < st1) dequant_and_fetch(st + 1, cur ^ 1);
    } else {
      // ---- online softmax of head 16*ht + n16 over the stage ----
      f32x4 sl[4];
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sl[u] = s_mine[u * 64];
        mx = fmaxf(mx, fmaxf(fmaxf(sl[u][0], sl[u][1]), fmaxf(sl[u][2], sl[u][3])));
      }
      mx = xor_lanes_max<16>(mx);
      mx = xor_lanes_max<32>(mx);
      // The reference moves only when the stage's max exceeds it by more
      // than 8 (log2 domain), so P <= 256 (fp16-safe) and the 128
      // accumulators are rescaled only on such jumps (with the exact running
      // max they were rescaled almost every stage); the output and the
      // partials are relative to the same reference, so the result is the
      // same up to rounding.
      const float m_new = mx > m_run + 8.f ? mx : m_run;
      float psum = 0.f, corr = 1.f;
      u32x4 pw[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
      if (m_new != -__builtin_huge_valf()) {
        corr = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          _Float16 pv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pv[r] = (_Float16)__builtin_amdgcn_exp2f(sl[u][r] - m_new);
            psum += (float)pv[r];
          }
          // P.V operand of position chunk u / 2: positions 32 kk + 4 g + 0..3
          // (tile 2 kk) then 32 kk + 16 + 4 g + 0..3 (tile 2 kk + 1)
          pw[u >> 1][2 * (u & 1)] = __builtin_bit_cast(uint32_t, f16x2{pv[0], pv[1]});
          pw[u >> 1][2 * (u & 1) + 1] = __builtin_bit_cast(uint32_t, f16x2{pv[2], pv[3]});
        }
      }
      psum = xor_lanes_sum<16>(psum);
      psum = xor_lanes_sum<32>(psum);
      l_run = l_run * corr + psum;
      m_run = m_new;
      if (corr != 1.f) {
#pragma unroll
        for (int t = 0; t < 32; ++t) acc[t] *= corr;
      }
      // ---- O^T tiles 0..31 of head tile ht over the stage's 64 positions ----
      // (the V^T fragments of the next 4 tiles are requested before this
      // group's 4 matrix instructions; scheduling barriers bound the
      // registers held in flight)
      auto read_vt = [&](int kk, int ct) -> f16x8 {
        const _Float16 *v0 = sv + vt_offset(32 * kk + 4 * g + r_src, ct, q_src);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(v0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(v0 + 16 * ROW_HALVES));
        return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      f16x8 vcur[4], vnext[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vcur[i] = read_vt(0, i);
#pragma unroll
      for (int grp = 0; grp < 16; ++grp) {          // 8 groups of 4 tiles per position chunk kk
        const int kk = grp >> 3, ct0 = 4 * (grp & 7);
        if (grp + 1 < 16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) vnext[i] = read_vt((grp + 1) >> 3, 4 * ((grp + 1) & 7) + i);
        }
        const f16x8 pop = __builtin_bit_cast(f16x8, pw[kk]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[ct0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vcur[i], pop, acc[ct0 + i], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) vcur[i] = vnext[i];
      }
    }
  }

  CSA2_TS(4);
  if (producer) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (a.splits == 1) {
    float *orow = a.out + ((int64_t)b * 64 + 16 * ht + n16) * D;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
      *reinterpret_cast<float4 *>(orow + tile_channel(ct, g)) =
          float4{acc[ct][0] * inv, acc[ct][1] * inv, acc[ct][2] * inv, acc[ct][3] * inv};
    CSA2_TS(5);
    return;
  }
  // partials in the 16-head kernel's layout: slot (b, split, tile ht)
  const int64_t slot = ((int64_t)b * a.splits + split) * 4 + ht;
  u32x2 *po = reinterpret_cast<u32x2 *>(a.part_o) + slot * (16 * D / 4) + lane;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) po[ct * 64] = pack_partial(acc[ct], inv);
  if (g == 0) {
    float *pm = a.part_ml + (slot * 16 + n16) * 2;
    pm[0] = m_run;
    pm[1] = l_run;
  }
  CSA2_TS(5);
}

struct CombineArgs {
  const _Float16 *part_o;   // as AttendArgs::part_o
  const float *part_ml;
  int32_t splits;
  int32_t heads;
  float *out;               // [batch][heads][512]
};

// LDS-staged combine for more than 64 splits (up to MAX_SPLITS; the
// register-only combine below takes 64 or fewer).
// grid (heads/16 * 32, batch), NW waves per workgroup: workgroup (ht, ct)
// merges O^T tile ct (1 KB) of head tile ht over every split, so the
// partials spread over heads/16 * 32 workgroups per sequence.  Wave w takes
// splits 32w.. of each batch of 32*NW; the (max, sum) pairs of the first
// 32*NW splits and each wave's first 32 tiles are requested in one batch,
// before any of them is used (one memory round trip for <= 32*NW splits);
// further splits follow in batches.  With two waves, wave 1 hands its
// partial sum to wave 0 through LDS.
constexpr int MAX_SPLITS = 256;
constexpr int CMB_U = 32;                 // splits per wave per batch
template <int NW>
__global__ void __launch_bounds__(64 * NW) attend_combine_kernel(CombineArgs a) {
  __shared__ float2 s_ml[MAX_SPLITS * 16];
  __shared__ float4 s_o[NW > 1 ? 64 : 1];
  __shared__ float s_l[NW > 1 ? 64 : 1];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int HT = a.heads / 16, ht = wg_x() >> 5, ct = wg_x() & 31;
  CSA2_CHECK(ht < HT);
  const int nslots = a.splits, nml = nslots * 16;
  const int n16 = lane & 15, g = lane >> 4;
  constexpr int BATCH = CMB_U * NW;       // splits per batch
  constexpr int MLV = BATCH * 16 / (64 * NW);
  CSA2_TS(8);
  const float2 *pml = reinterpret_cast<const float2 *>(a.part_ml);
  const u32x2 *po = reinterpret_cast<const u32x2 *>(a.part_o) + ct * 64 + lane;
  auto slot_of = [&](int s) { return ((int64_t)b * a.splits + s) * HT + ht; };
  // (max, sum) of the first BATCH splits: entry tid + 64*NW*u is split
  // (tid + 64*NW*u) / 16, head (tid + 64*NW*u) % 16 (slots are contiguous in
  // the partial layout only per head tile, so the index goes through slot_of)
  float2 mlv[MLV];
#pragma unroll
  for (int u = 0; u < MLV; ++u) {
    const int e = min(tid + 64 * NW * u, nml - 1);
    mlv[u] = pml[slot_of(e >> 4) * 16 + (e & 15)];
  }
  u32x2 ov[CMB_U];
#pragma unroll
  for (int u = 0; u < CMB_U; ++u) ov[u] = po[slot_of(min(CMB_U * wv + u, nslots - 1)) * (16 * D / 4)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < MLV; ++u) {
    const int e = tid + 64 * NW * u;
    if (e < nml) s_ml[e] = mlv[u];
  }
  // splits beyond the first batch (long selections): their (max, sum) pairs
  for (int e0 = BATCH * 16; e0 < nml; e0 += 64 * NW) {
    const int e = e0 + tid;
    if (e < nml) s_ml[e] = pml[slot_of(e >> 4) * 16 + (e & 15)];
  }
  __syncthreads();
  CSA2_TS(9);
  float M = -__builtin_huge_valf();
  for (int s0 = 0; s0 < nslots; s0 += 16) {
    float mv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) mv[u] = s_ml[min(s0 + u, nslots - 1) * 16 + n16].x;
#pragma unroll
    for (int u = 0; u < 16; ++u) M = fmaxf(M, mv[u]);     // a repeated split changes nothing
  }
  float L = 0.f;
  float4 o = {0.f, 0.f, 0.f, 0.f};
  if (M != -__builtin_huge_valf()) {
    // every partial is written (an empty one as m = -inf, O = 0), so a
    // batch past the last split re-reads that split with weight 0
#pragma unroll 1
    for (int s0 = 0; s0 < nslots; s0 += BATCH) {
      const int sw = s0 + CMB_U * wv;    // this wave's first split of the batch
      if (s0 > 0) {
#pragma unroll
        for (int u = 0; u < CMB_U; ++u) ov[u] = po[slot_of(min(sw + u, nslots - 1)) * (16 * D / 4)];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < CMB_U; ++u) {
        const int su = min(sw + u, nslots - 1);
        const float2 ml = s_ml[su * 16 + n16];
        const float e = (sw + u < nslots && ml.x != -__builtin_huge_valf()) ? __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
        const float we = e * ml.y;          // the partial is O / sum
        const float4 v = unpack_partial(ov[u]);
        L += we;
        o.x += we * v.x; o.y += we * v.y; o.z += we * v.z; o.w += we * v.w;
      }
    }
  }
  if constexpr (NW > 1) {
    if (wv == 1) { s_o[lane] = o; s_l[lane] = L; }
    __syncthreads();
    if (wv != 0) return;
    const float4 o1 = s_o[lane];
    o.x += o1.x; o.y += o1.y; o.z += o1.z; o.w += o1.w;
    L += s_l[lane];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
  // lane (n16, g) of tile ct holds channels tile_channel(ct, g) + 0..3
  const int c0 = tile_channel(ct, g);
  *reinterpret_cast<float4 *>(a.out + ((int64_t)b * a.heads + 16 * ht + n16) * D + c0) = o;
  CSA2_TS(10);
}

// Register-only combine for up to U * NW splits: grid (heads/16 * 32,
// batch), NW waves.  Lane (n16, g) of wave w merges head 16*ht + n16,
// channels of O^T tile ct, over splits Uw..Uw+U-1: its U (max, sum) pairs
// and U partial float4s are requested in one batch (split s of a head tile
// sits at a fixed stride, so the addresses are a base plus s times it), and
// the maximum, weights, sum and output are formed in registers; with more
// waves, waves 1.. hand (max, sum, output) to wave 0 through LDS.
template <int NW, int U>
__global__ void __launch_bounds__(64 * NW) attend_combine_regs_kernel(CombineArgs a) {
  __shared__ float4 s_o[NW > 1 ? NW - 1 : 1][64];
  __shared__ float s_m[NW > 1 ? NW - 1 : 1][64], s_l[NW > 1 ? NW - 1 : 1][64];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int HT = a.heads >> 4, ht = wg_x() >> 5, ct = wg_x() & 31;
  CSA2_CHECK(ht < HT);
  const int n16 = lane & 15, g = lane >> 4;
  const int ns = a.splits, s0 = U * wv;
  CSA2_TS(8);
  const int64_t slot0 = (int64_t)b * ns * HT + ht;                 // slot of split 0
  const u32x2 *po = reinterpret_cast<const u32x2 *>(a.part_o) + slot0 * (16 * D / 4) + ct * 64 + lane;
  const float2 *pm = reinterpret_cast<const float2 *>(a.part_ml) + slot0 * 16 + n16;
  const int64_t so = (int64_t)HT * (16 * D / 4), sm = (int64_t)HT * 16;   // per split
  float2 ml[U];
  u32x2 ov[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t sc = min(s0 + u, ns - 1);                        // clamped: one batch, no branch
    ml[u] = pm[sc * sm];
    ov[u] = po[sc * so];
  }
  __builtin_amdgcn_sched_barrier(0);
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (s0 + u < ns) M = fmaxf(M, ml[u].x);
  float L = 0.f;
  float4 o = {0.f, 0.f, 0.f, 0.f};
  if (M != -__builtin_huge_valf()) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = (s0 + u < ns && ml[u].x != -__builtin_huge_valf()) ? __builtin_amdgcn_exp2f(ml[u].x - M) : 0.f;
      const float we = e * ml[u].y;         // the partial is O / sum
      const float4 v = unpack_partial(ov[u]);
      L += we;
      o.x += we * v.x; o.y += we * v.y; o.z += we * v.z; o.w += we * v.w;
    }
  }
  CSA2_TS(9);
  if constexpr (NW > 1) {
    // waves 1.. hand (max, sum, output) to wave 0, which merges them in order
    if (wv > 0) { s_o[wv - 1][lane] = o; s_m[wv - 1][lane] = M; s_l[wv - 1][lane] = L; }
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float M1 = s_m[w - 1][lane], L1 = s_l[w - 1][lane];
      const float4 o1 = s_o[w - 1][lane];
      const float Mx = fmaxf(M, M1);
      if (Mx != -__builtin_huge_valf()) {
        const float e0 = M == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(M - Mx);
        const float e1 = M1 == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(M1 - Mx);
        L = e0 * L + e1 * L1;
        o.x = e0 * o.x + e1 * o1.x; o.y = e0 * o.y + e1 * o1.y;
        o.z = e0 * o.z + e1 * o1.z; o.w = e0 * o.w + e1 * o1.w;
        M = Mx;
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
  // lane (n16, g) of tile ct holds channels tile_channel(ct, g) + 0..3
  const int c0 = tile_channel(ct, g);
  *reinterpret_cast<float4 *>(a.out + ((int64_t)b * a.heads + 16 * ht + n16) * D + c0) = o;
  CSA2_TS(10);
}

template __global__ void attend_combine_regs_kernel<1, 8>(CombineArgs);
template __global__ void attend_combine_regs_kernel<4, 8>(CombineArgs);
template __global__ void attend_combine_regs_kernel<4, 16>(CombineArgs);
template __global__ void attend_combine_kernel<2>(CombineArgs);

}  // namespace csa2
