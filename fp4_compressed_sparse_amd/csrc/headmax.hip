// Per-head indexer score of CSA2 (gfx950).
//
// The pages say the indexer keeps the top-k most relevant blocks of 8
// positions (rebasdaily.com "DeepSeek-V4.1-Flash KV compression", section
// "same notes, many layers") but not how it turns many query heads into one
// score per block.  index.hip sums the heads first; this file computes the
// other plain reading: every head scores the block on its own, in the same
// pinned float32 order as the summed rule, and the block's score is the best
// head's:
//   key[c]  = mean of the block's dequantised rows (rows added in position
//             order, x 0.125 for a full block, / row count otherwise)
//   S_h     = for head h: p_c = fl(q_h[c] * key[c]) (never fused), the 16
//             products of a scale group added left to right, the 32 group
//             sums added as a tree of adjacent pairs, plus 0.0
//   score   = max over h of S_h                       (exact)
// so the selected indices stay reproducible bit for bit.  At 64 heads this
// is about 65,536 float32 operations per block, 64 times the summed rule:
// the kernel is bound by the vector ALU, not by HBM.
//
// Work layout (a workgroup takes tiles of NT blocks, or of NT candidates):
//   1. keys: 32 lanes per block, lane j owns scale group j (8 code bytes and
//      one scale byte of each row), add the rows by FMA (each code x scale is
//      exact in float32) and scale them; the keys go to LDS.
//   2. partial scores: wave w owns the channels [w*C, w*C + C), C = 512 /
//      waves, and lane = head, the heads rounded up to 16, 32 or 64 (with
//      fewer heads a wave takes 4 or 2 blocks at once, one per 16- or 32-lane
//      part).  A lane keeps its head's C query values in registers.  Each
//      16-lane row of the wave reads the key values of one block from LDS,
//      lane r of the row holding channels 4r..4r+3 of a 64-channel chunk, and
//      a DPP row broadcast (row_newbcast, folded into v_mul_f32) hands every
//      lane of the row the value it multiplies: one LDS read serves 64
//      products per lane.  The wave adds its groups' sums as the subtree of
//      the pinned tree that covers them.
//   3. combine: the waves' subtree results are the nodes of one level of
//      the tree; the levels above are added in order, plus 0.0, and a wave
//      max over the heads gives the block's score.
#include "common.hpp"

namespace csa2 {

struct HeadmaxArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const int64_t *seq_len;
  int64_t capacity;
  int64_t limit;            // min(capacity, max_len)
  const float *q;           // [batch][heads][512]
  int32_t heads;            // 1..64
  const int32_t *cand;      // [batch][n_cand]; NULL: every block of the sequence
  int32_t n_cand;
  int32_t nblk_grid;        // without a candidate list: ceil(max_len / 8)
  float *scores;            // [batch][score_stride]
  int64_t score_stride;
  uint32_t *hist;           // without a candidate list, when selecting:
                            // [batch][HIST_COPIES][HIST_BINS] digit counts
  int32_t fill_invalid;     // without a candidate list: -inf for blocks past the end
};

// Key of one block as lane j of its 32-lane slot computes it: key[16j ..
// 16j+15].  The arithmetic and its order are those of block_score32: row 0's
// value code x scale, then each later row added by FMA (exact product), in
// position order; x 0.125 for a full block, else / cnt rounded to nearest.
__device__ __forceinline__ void block_key32(const BlockRows32 &r, int cnt, float key[16]) {
  float S[16];
#pragma unroll
  for (int t = 0; t < BLOCK; ++t) {
    if (t < cnt) {
      const float s = e4m3_to_f32(r.sc[t]);
#pragma unroll
      for (int dw = 0; dw < 2; ++dw) {
        const uint32_t word = r.w[t][dw];
        const f32x2 v0 = e2m1x2_to_f32<0>(word);
        const f32x2 v1 = e2m1x2_to_f32<1>(word);
        const f32x2 v2 = e2m1x2_to_f32<2>(word);
        const f32x2 v3 = e2m1x2_to_f32<3>(word);
        float *o = S + 8 * dw;
        if (t == 0) {
          o[0] = v0.x * s; o[1] = v0.y * s; o[2] = v1.x * s; o[3] = v1.y * s;
          o[4] = v2.x * s; o[5] = v2.y * s; o[6] = v3.x * s; o[7] = v3.y * s;
        } else {
          o[0] = __builtin_fmaf(v0.x, s, o[0]); o[1] = __builtin_fmaf(v0.y, s, o[1]);
          o[2] = __builtin_fmaf(v1.x, s, o[2]); o[3] = __builtin_fmaf(v1.y, s, o[3]);
          o[4] = __builtin_fmaf(v2.x, s, o[4]); o[5] = __builtin_fmaf(v2.y, s, o[5]);
          o[6] = __builtin_fmaf(v3.x, s, o[6]); o[7] = __builtin_fmaf(v3.y, s, o[7]);
        }
      }
    }
  }
  if (cnt == BLOCK) {
#pragma unroll
    for (int c = 0; c < 16; ++c) key[c] = S[c] * 0.125f;
  } else {
    const float fc = (float)cnt;
#pragma unroll
    for (int c = 0; c < 16; ++c) key[c] = __fdiv_rn(S[c], fc);
  }
}

// DPP row broadcast (control row_newbcast:R = 0x150 + R): every lane of a
// 16-lane row receives lane R of that row.  Used as the first operand of a
// multiply, the compiler folds it into v_mul_f32_dpp.
template <int R>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + R, 0xf, 0xf, true));
}

// Sum of one scale group for this lane's head: its 16 query values qg[0..15]
// times the group's 16 key values, added left to right.  kv holds a
// 64-channel chunk (lane r of each row: channels 4r..4r+3); group G of the
// chunk sits in row lanes 4G..4G+3.
template <int G>
__device__ __forceinline__ float group_dot(const float *qg, const f32x4 &kv) {
  float g = row_bcast<4 * G>(kv[0]) * qg[0];
  g = g + row_bcast<4 * G>(kv[1]) * qg[1];
  g = g + row_bcast<4 * G>(kv[2]) * qg[2];
  g = g + row_bcast<4 * G>(kv[3]) * qg[3];
  g = g + row_bcast<4 * G + 1>(kv[0]) * qg[4];
  g = g + row_bcast<4 * G + 1>(kv[1]) * qg[5];
  g = g + row_bcast<4 * G + 1>(kv[2]) * qg[6];
  g = g + row_bcast<4 * G + 1>(kv[3]) * qg[7];
  g = g + row_bcast<4 * G + 2>(kv[0]) * qg[8];
  g = g + row_bcast<4 * G + 2>(kv[1]) * qg[9];
  g = g + row_bcast<4 * G + 2>(kv[2]) * qg[10];
  g = g + row_bcast<4 * G + 2>(kv[3]) * qg[11];
  g = g + row_bcast<4 * G + 3>(kv[0]) * qg[12];
  g = g + row_bcast<4 * G + 3>(kv[1]) * qg[13];
  g = g + row_bcast<4 * G + 3>(kv[2]) * qg[14];
  g = g + row_bcast<4 * G + 3>(kv[3]) * qg[15];
  return g;
}

// Adjacent-pair tree over x[0..N) (N a power of two): level 1 adds x[0]+x[1],
// x[2]+x[3], ...; each later level adds adjacent results of the one before.
template <int N>
__device__ __forceinline__ float pair_tree(float *x) {
#pragma unroll
  for (int step = 1; step < N; step *= 2) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * step) x[i] = x[i] + x[i + step];
  }
  return x[0];
}

// NW waves (each C = 512 / NW channels), tiles of NT blocks (or candidates).
// CAND: score the candidate list; else every block, with HIST the digit
// counts of the scores for the selection kernel.  grid (workgroups, batch).
template <int NW, int NT, bool CAND, bool HIST>
__global__ void __launch_bounds__(64 * NW) headmax_kernel(HeadmaxArgs a) {
  constexpr int C = D / NW;            // channels per wave
  constexpr int NG = C / 16;           // scale groups per wave
  constexpr int NTHR = 64 * NW;
  constexpr int KPASS = NTHR / 32;     // blocks whose keys one pass builds
  constexpr int NPASS = (NT + KPASS - 1) / KPASS;
  constexpr int QR = 32;               // query channels per staging round and wave
  constexpr int QPAD = 65;             // heads per staged row (one more: stores spread over the banks)
  static_assert(C % 64 == 0 && (NG & (NG - 1)) == 0 && NT % 4 == 0 && C % QR == 0, "tile shape");
  // The tile arrays (keys, partial scores) and the query staging area share
  // one LDS buffer: the query is staged once, before the first tile.
  constexpr int TILE_FLOATS = NT * D + NW * NT * 64;
  constexpr int STAGE_FLOATS = NW * (QR / 4) * QPAD * 4;
  __shared__ __attribute__((aligned(16))) float s_buf[TILE_FLOATS > STAGE_FLOATS ? TILE_FLOATS : STAGE_FLOATS];
  float (*s_key)[D] = reinterpret_cast<float (*)[D]>(s_buf);
  float (*s_part)[NT][64] = reinterpret_cast<float (*)[NT][64]>(s_buf + NT * D);
  __shared__ uint32_t s_hist[HIST ? HIST_BINS : 1];
  const int b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int H = a.heads;
  const int hp = H <= 16 ? 16 : (H <= 32 ? 32 : 64);   // lanes per block in phase 2
  const int bpw = 64 / hp;                             // blocks per wave step
  const int h = lane & (hp - 1), sub = lane / hp;
  if (HIST) {
    for (int j = t; j < HIST_BINS; j += NTHR) s_hist[j] = 0;
  }
  const uint8_t *codes = a.codes + (int64_t)b * a.capacity * CODE_BYTES;
  const uint8_t *scales = a.scales + (int64_t)b * a.capacity * SCALE_BYTES;
  const int64_t cap_blocks = a.capacity / BLOCK;       // loads stay inside the cache
  const int64_t n = clamp_len(a.seq_len[b], a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;
  const int64_t nitems = CAND ? a.n_cand : a.nblk_grid;
  const int64_t ntiles = (nitems + NT - 1) / NT;
  const int32_t *cand = CAND ? a.cand + (int64_t)b * a.n_cand : nullptr;
  float *scores = a.scores + (int64_t)b * a.score_stride;

  // Rows of a tile's blocks: pass p, thread t holds the rows of block
  // p * KPASS + t / 32 (an item without a block reads block 0, which always
  // exists; its score is never written).
  const int j32 = t & 31;
  auto block_of = [&](int64_t tile, int bl) -> int64_t {
    const int64_t item = tile * NT + bl;
    if (CAND) return item < a.n_cand ? (int64_t)cand[item] : -1;
    return item;
  };
  BlockRows32 rows[NPASS];
  auto load_tile = [&](int64_t tile) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int bl = p * KPASS + (t >> 5);
      if (bl < NT) {
        const int64_t blk = block_of(tile, bl);
        const int64_t lb = (blk >= 0 && blk < cap_blocks) ? blk : 0;
        load_block32(rows[p], codes + lb * BLOCK * CODE_BYTES, scales + lb * BLOCK * SCALE_BYTES, j32);
      }
    }
  };
  const uint32_t wx = wg_x();
  int64_t tile = wx;
  if (tile < ntiles) load_tile(tile);     // the first tile's rows overlap the query staging

  // This lane's query values: head h, channels w*C .. w*C + C - 1 (zeros for
  // a lane past the last head; its scores are dropped at the max).  Staged
  // through LDS in rounds of QR channels: a load instruction reads 8 heads'
  // QR-channel runs (8 lanes x 16 bytes each, so a few cache lines per
  // instruction instead of one per lane), stored as [channel quad][head], and
  // each lane then reads its head's QR channels back.
  float qv[C];
  {
    float *sq = s_buf + w * (QR / 4) * QPAD * 4;
    const int cq = lane & 7, hl0 = lane >> 3;
    bool fin = true;
    f32x4 v[C / QR][8];                   // every round's loads in one batch
#pragma unroll
    for (int r = 0; r < C / QR; ++r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int hl = hl0 + 8 * i;
        v[r][i] = *reinterpret_cast<const f32x4 *>(a.q + ((int64_t)b * H + min(hl, H - 1)) * D + w * C + r * QR +
                                                   4 * cq);
      }
    }
#pragma unroll
    for (int r = 0; r < C / QR; ++r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int hl = hl0 + 8 * i;
        if (hl >= H) v[r][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4 *>(sq + (cq * QPAD + hl) * 4) = v[r][i];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < QR / 4; ++k) {
        const f32x4 u = *reinterpret_cast<const f32x4 *>(sq + (k * QPAD + h) * 4);
        fin = fin && __builtin_isfinite(u[0]) && __builtin_isfinite(u[1]) && __builtin_isfinite(u[2]) &&
              __builtin_isfinite(u[3]);
        qv[r * QR + 4 * k] = u[0]; qv[r * QR + 4 * k + 1] = u[1];
        qv[r * QR + 4 * k + 2] = u[2]; qv[r * QR + 4 * k + 3] = u[3];
      }
      __syncthreads();                    // the area is refilled next round, then holds the tiles
    }
    if (__builtin_amdgcn_ballot_w64(!fin) && lane == 0) raise_flag(FLAG_NONFINITE_Q);
  }

  for (; tile < ntiles; tile += gridDim.x) {
    const int64_t base = tile * NT;
    // 1. keys of the tile's blocks into LDS, then the next tile's rows are
    //    requested (in flight during phases 2 and 3)
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int bl = p * KPASS + (t >> 5);
      if (bl < NT) {
        const int64_t blk = block_of(tile, bl);
        const bool ok = blk >= 0 && blk < nblk;
        const int cnt = ok ? (int)min((int64_t)BLOCK, n - blk * BLOCK) : BLOCK;
        float key[16];
        block_key32(rows[p], cnt, key);
        f32x4 *dst = reinterpret_cast<f32x4 *>(&s_key[bl][16 * j32]);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = f32x4{key[4 * k], key[4 * k + 1], key[4 * k + 2], key[4 * k + 3]};
      }
    }
    if (tile + gridDim.x < ntiles) load_tile(tile + gridDim.x);
    __syncthreads();
    // 2. per-head subtree of this wave's groups, bpw blocks per step
    for (int st = 0; st < NT / bpw; ++st) {
      const int bl = st * bpw + sub;
      const float *kp = &s_key[bl][w * C + 4 * (lane & 15)];
      float gs[NG];
#pragma unroll
      for (int k = 0; k < C / 64; ++k) {
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(kp + 64 * k);
        gs[4 * k + 0] = group_dot<0>(qv + 64 * k, kv);
        gs[4 * k + 1] = group_dot<1>(qv + 64 * k + 16, kv);
        gs[4 * k + 2] = group_dot<2>(qv + 64 * k + 32, kv);
        gs[4 * k + 3] = group_dot<3>(qv + 64 * k + 48, kv);
      }
      s_part[w][bl][h] = pair_tree<NG>(gs);
    }
    __syncthreads();
    // 3. the tree's upper levels per head, then the best head; wave w takes
    //    blocks w, w + NW, ...  (s_key is free again: the next tile's phase 1
    //    may start; s_part is rewritten only after its barrier)
    for (int bl = w; bl < NT; bl += NW) {
      float v = -__builtin_huge_valf();
      if (lane < H) {
        float p[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) p[i] = s_part[i][bl][lane];
        v = pair_tree<NW>(p) + 0.0f;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
      if (lane == 0) {
        const int64_t item = base + bl;
        if (CAND) {
          if (item < a.n_cand) {
            const int64_t blk = cand[item];
            if (blk >= 0 && blk < nblk) {
              scores[item] = v;
            } else {
              scores[item] = -__builtin_huge_valf();
              if (blk >= nblk) raise_flag(FLAG_BAD_INDEX);
            }
          }
        } else if (item < nblk) {
          scores[item] = v;
          if (HIST) atomicAdd(&s_hist[ord_key(v) >> HIST_SHIFT], 1u);
        } else if (a.fill_invalid && item < a.score_stride) {
          scores[item] = -__builtin_huge_valf();
        }
      }
    }
  }
  if (!HIST) return;
  __syncthreads();
  uint32_t *mine = a.hist + ((int64_t)b * HIST_COPIES + (wx % HIST_COPIES)) * HIST_BINS;
  for (int j = t; j < HIST_BINS; j += NTHR) {
    const uint32_t c = s_hist[j];
    if (c) atomic_add_agent(mine + j, c);
  }
}

// Top-k of a scored candidate list, one workgroup per sequence: the
// finishing step of rescore_kernel<true> for scores another kernel wrote.
__global__ void __launch_bounds__(SCAN_THREADS) select_cand_kernel(RescoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint64_t s_keys[];
  __shared__ int32_t s_ids[LDS_KEYS];
  __shared__ int32_t s_sel[CSA2_TOPK_MAX + SEL_PAD];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[TOPK_HIST_BINS];
  __shared__ uint64_t s_state[2];
  __shared__ uint32_t s_wave[16];
  const int b = blockIdx.y;
  const int64_t n = clamp_len(a.seq_len[b], a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;
  cand_keys_to_lds<false>(a.cand + (int64_t)b * a.n_cand, a.scores + (int64_t)b * a.score_stride, a.n_cand,
                          nblk, s_keys, s_ids);
  select_in_lds(s_keys, s_ids, a.n_cand, a.topk, a.idx_out + (int64_t)b * a.topk, s_sel, a.topk, s_hist,
                s_state, s_wave);
}

template __global__ void headmax_kernel<4, 16, false, true>(HeadmaxArgs);
template __global__ void headmax_kernel<4, 16, false, false>(HeadmaxArgs);
template __global__ void headmax_kernel<4, 4, true, false>(HeadmaxArgs);

}  // namespace csa2
