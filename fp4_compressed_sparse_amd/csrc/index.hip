// Hierarchical sparse indexer of CSA2 (gfx950).
//
// Method: each layer picks the top-k most relevant blocks of 8 positions;
// the first Full layer scans the whole range into a candidate pool
// (2,048 blocks x 8 = 16,384 positions in the example) and later layers
// search only the pool (rebasdaily.com "DeepSeek-V4.1-Flash KV
// compression", section "same notes, many layers").  The cache rows are FP4
// E2M1 codes with an E4M3 scale per 16 channels (ailily.cc "890 bytes per
// token", section 二), read at a fixed stride and dequantised inside the
// kernel (yomxxx.com long-form post, section 五).
//
// Score definition (the pages give none; this fixes one so that indices are
// reproducible bit for bit):
//   key[c]  = (rows of the block added in ascending position order, float32)
//             / row count   (x 0.125 for a full block: exact)
//   Qbar    = q_0 + q_1 + ... + q_{H-1}, float32, heads in order
//   p_c     = fl(Qbar[c] * key[c])                  (never fused)
//   g_j     = p_{16j} + ... + p_{16j+15}            left to right
//   score   = adjacent-pair tree over g_0..g_31, plus 0.0 (no -0)
// The row sum uses FMA: each dequantised value code*scale is exact in
// float32, so fma(code, scale, acc) == fl(acc + code*scale).
//
// Work layout: the full scan gives each block 32 lanes (lane j owns scale
// group j: 8 code bytes and 1 scale byte of each of the 8 rows; the five
// tree levels are lane butterflies xor 1..16); the pool rescoring gives
// each block 16 lanes (lane i owns channels 32i..32i+31, the two groups of a
// lane summed in-lane, levels 2..5 as butterflies xor 1..8).  Same
// arithmetic, same order.
//
// Selection: keys are (order-preserving score bits << 32) | ~block_id, so
// all keys differ and ties go to the lowest id.  The scan adds the top 10
// key bits of every block to a histogram (8 copies); every select
// workgroup finds the digit that holds the R-th largest key from it and
// writes the keys of its blocks at or above that digit to its own region;
// the last select workgroup ranks those keys in LDS and writes the chosen
// ids in ascending order (select2_kernel; select_kernel, with a global
// bitmap and tie lists, serves selections whose bitmap exceeds LDS).
// A top-k inside one workgroup (a candidate list, the finishers' ranks)
// uses linear bins over the score range with an exact pairwise finish
// (select_top_regs, threshold_linear).
#include "common.hpp"

namespace csa2 {

constexpr int SCAN_THREADS = 256;
constexpr int BLOCKS_PER_ITER = 16;      // 4 waves x 4 blocks
constexpr int LDS_KEYS = 8192;           // finisher key capacity (64 KB)
constexpr int CSA2_TOPK_MAX = 2048;      // largest top-k (staged output in LDS)

struct ScanArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const int64_t *seq_len;
  int64_t capacity;
  int64_t limit;            // min(capacity, max_len)
  const float *q;
  int32_t heads;
  int32_t nblk_grid;        // blocks covered by the grid: ceil(max_len / 8)
  float *scores;            // [batch][score_stride]
  int64_t score_stride;
  Ctrl *ctrl;               // [batch]
  uint32_t *hist;           // [batch][HIST_BINS]
  int32_t R;                // keys to select (pool or topk)
  int32_t fill_invalid;     // write -inf for blocks >= nblk (export only)
  const float *qbar;        // [batch][512] precomputed Qbar (required with the histogram),
                            // or NULL (computed in-kernel)
};

// Qbar in LDS for the 32-lane scorers: channel 16 j + 4 k + e (group j,
// quarter k) at float 256 (j >> 4) + 64 k + 4 (j & 15) + e, so that when
// lane j reads quarter k of its group (a 128-bit read), 16 lanes hit 16
// distinct 16-byte slots of one 256-byte window (in channel order, lanes 64
// bytes apart met four to a slot and the read took four times as long).
__device__ __forceinline__ int qbar32_index(int c) {
  return 256 * (c >> 8) + 64 * ((c >> 2) & 3) + 4 * ((c >> 4) & 15) + (c & 3);
}
__device__ __forceinline__ int qbar32_base(int j) { return 256 * (j >> 4) + 4 * (j & 15); }

// Qbar of sequence b into LDS; all 256 threads call.  Each thread owns two
// channels and adds the heads in order; the loads of HB heads are issued
// together so the sum costs heads/HB memory round trips, not one per head
// (HB = 16 keeps the scan's register budget; the pool rescoring uses 64).
template <int HB, bool QB32 = false>
__device__ __forceinline__ void compute_qbar(const float *__restrict__ q, int heads, int b,
                                             float *s_qbar) {
  const int t = threadIdx.x;
  const float2 *qp = reinterpret_cast<const float2 *>(q + (int64_t)b * heads * D) + t;
  float2 acc = make_float2(0.f, 0.f);
  for (int h0 = 0; h0 < heads; h0 += HB) {
    // unconditional loads (a head past the end re-reads the last one and is
    // dropped below), so the batch is issued back to back
    float2 v[HB];
#pragma unroll
    for (int j = 0; j < HB; ++j) v[j] = qp[(int64_t)min(h0 + j, heads - 1) * (D / 2)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      const int h = h0 + j;
      if (h == 0) {
        acc = v[j];
      } else if (h < heads) {
        acc.x = acc.x + v[j].x;
        acc.y = acc.y + v[j].y;
      }
    }
  }
  if (!(__builtin_isfinite(acc.x) && __builtin_isfinite(acc.y))) raise_flag(FLAG_NONFINITE_Q);
  if (QB32)
    *reinterpret_cast<float2 *>(s_qbar + qbar32_index(2 * t)) = acc;   // QB32: the 32-lane scorers' layout
  else
    reinterpret_cast<float2 *>(s_qbar)[t] = acc;
  __syncthreads();
}

// The 8 rows of one block as one lane of its 16-lane slot sees them.
struct BlockRows {
  u32x4 w[BLOCK];       // code bytes 16i..16i+15 of each row
  uint32_t sc[BLOCK];   // scale bytes 2i, 2i+1 of each row
};

__device__ __forceinline__ void load_block(BlockRows &r, const uint8_t *__restrict__ rowbase,
                                           const uint8_t *__restrict__ srow, int i) {
#pragma unroll
  for (int t = 0; t < BLOCK; ++t) {
    r.w[t] = *reinterpret_cast<const u32x4 *>(rowbase + (int64_t)t * CODE_BYTES + 16 * i);
    r.sc[t] = *reinterpret_cast<const uint16_t *>(srow + (int64_t)t * SCALE_BYTES + 2 * i);
  }
}

// One level of the score's pairwise tree: v plus the value of lane ^ M.
// M = 1 and 2 are exact quad permutes (DPP).  For M = 4, 8 and 16 the lower
// levels have already made every group of M lanes hold one value, so any
// lane of the partner group serves: the half-row and row mirrors (DPP) and
// the permlane16 row swap (whose two results are the lane's own value and
// its partner's, in either order; the sum is the same).  All are lane moves
// in the vector unit, with no LDS round trip, and each lane adds the same
// two values as with an exchange by lane ^ M.
template <int M>
__device__ __forceinline__ float tree_add(float v) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (M == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
  } else {
    constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : M == 4 ? 0x141 : 0x140;   // quad [1,0,3,2], [2,3,0,1]; half-row, row mirror
    return v + __uint_as_float(CSA2_DPP(u, ctrl, 0xf));
  }
}

// Score of one block from its loaded rows; the 16 lanes of a slot call it
// together (lane16 = i).  cnt: rows present (1..8).  qb: this lane's 32
// Qbar values (LDS).  RELOAD: as soon as row t is consumed its registers
// receive row t of the block at (nrow, nsrow), so the next block's loads
// are in flight while this one is scored (unconditional loads).
template <bool RELOAD = false>
__device__ __forceinline__ float block_score(BlockRows &r, int cnt, const float *qb,
                                             const uint8_t *__restrict__ nrow = nullptr,
                                             const uint8_t *__restrict__ nsrow = nullptr, int i = 0) {
  u32x4 *w = r.w;
  uint32_t *sc = r.sc;
  float S[32];
#pragma unroll
  for (int t = 0; t < BLOCK; ++t) {
    if (t < cnt) {
      const float s0 = e4m3_to_f32(sc[t] & 0xffu), s1 = e4m3_to_f32(sc[t] >> 8);
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        const float s = dw < 2 ? s0 : s1;
        f32x2 v0 = e2m1x2_to_f32<0>(w[t][dw]);
        f32x2 v1 = e2m1x2_to_f32<1>(w[t][dw]);
        f32x2 v2 = e2m1x2_to_f32<2>(w[t][dw]);
        f32x2 v3 = e2m1x2_to_f32<3>(w[t][dw]);
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
    if (RELOAD) {
      w[t] = *reinterpret_cast<const u32x4 *>(nrow + (int64_t)t * CODE_BYTES + 16 * i);
      sc[t] = *reinterpret_cast<const uint16_t *>(nsrow + (int64_t)t * SCALE_BYTES + 2 * i);
    }
  }
  float g0, g1;
  if (cnt == BLOCK) {
    g0 = qb[0] * (S[0] * 0.125f);
#pragma unroll
    for (int c = 1; c < 16; ++c) g0 = g0 + qb[c] * (S[c] * 0.125f);
    g1 = qb[16] * (S[16] * 0.125f);
#pragma unroll
    for (int c = 17; c < 32; ++c) g1 = g1 + qb[c] * (S[c] * 0.125f);
  } else {
    const float fc = (float)cnt;
    g0 = qb[0] * __fdiv_rn(S[0], fc);
    for (int c = 1; c < 16; ++c) g0 = g0 + qb[c] * __fdiv_rn(S[c], fc);
    g1 = qb[16] * __fdiv_rn(S[16], fc);
    for (int c = 17; c < 32; ++c) g1 = g1 + qb[c] * __fdiv_rn(S[c], fc);
  }
  float v = g0 + g1;                    // tree level 1: groups 2i, 2i+1
  v = tree_add<1>(v);                   // level 2
  v = tree_add<2>(v);                   // level 3
  v = tree_add<4>(v);                   // level 4
  v = tree_add<8>(v);                   // level 5
  return v + 0.0f;
}

// Full-scan variant: 32 lanes per block, lane j owns scale group j
// (channels 16j..16j+15: 8 code bytes and 1 scale byte of each row), so a
// wave scores two blocks per step with about half the registers of the
// 16-lane layout (twice the resident waves to cover memory latency).  Same
// arithmetic in the same order: row sums by FMA in position order, x 0.125
// (or / count), products with Qbar added left to right inside the group,
// then the adjacent-pair tree over the 32 groups as lane butterflies
// (xor 1, 2, 4, 8, 16).
struct BlockRows32 {
  u32x2 w[BLOCK];       // code bytes 8j..8j+7 of each row
  uint32_t sc[BLOCK];   // scale byte j of each row
};

__device__ __forceinline__ void load_block32(BlockRows32 &r, const uint8_t *__restrict__ rowbase,
                                             const uint8_t *__restrict__ srow, int j) {
#pragma unroll
  for (int t = 0; t < BLOCK; ++t) {
    r.w[t] = *reinterpret_cast<const u32x2 *>(rowbase + (int64_t)t * CODE_BYTES + 8 * j);
    r.sc[t] = srow[(int64_t)t * SCALE_BYTES + j];
  }
}

// cnt: rows present (1..8); qb: s_qbar + qbar32_base(j), so that channel
// 16 j + c is qb[64 * (c >> 2) + (c & 3)] (LDS).  RELOAD: as each
// row is consumed its registers receive the same row of the block at (nrow,
// nsrow), so the next block's loads are in flight while this one is scored.
template <bool RELOAD = true>
__device__ __forceinline__ float block_score32(BlockRows32 &r, int cnt, const float *qb,
                                               const uint8_t *__restrict__ nrow,
                                               const uint8_t *__restrict__ nsrow, int j) {
  float S[16];
#pragma unroll
  for (int t = 0; t < BLOCK; ++t) {
    if (t < cnt) {
      const float s = e4m3_to_f32(r.sc[t]);
#pragma unroll
      for (int dw = 0; dw < 2; ++dw) {
        const uint32_t word = r.w[t][dw];
        f32x2 v0 = e2m1x2_to_f32<0>(word);
        f32x2 v1 = e2m1x2_to_f32<1>(word);
        f32x2 v2 = e2m1x2_to_f32<2>(word);
        f32x2 v3 = e2m1x2_to_f32<3>(word);
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
    if (RELOAD) {
      r.w[t] = *reinterpret_cast<const u32x2 *>(nrow + (int64_t)t * CODE_BYTES + 8 * j);
      r.sc[t] = nsrow[(int64_t)t * SCALE_BYTES + j];
    }
  }
  float g;
  if (cnt == BLOCK) {
    g = qb[0] * (S[0] * 0.125f);
#pragma unroll
    for (int c = 1; c < 16; ++c) g = g + qb[64 * (c >> 2) + (c & 3)] * (S[c] * 0.125f);
  } else {
    const float fc = (float)cnt;
    g = qb[0] * __fdiv_rn(S[0], fc);
    for (int c = 1; c < 16; ++c) g = g + qb[64 * (c >> 2) + (c & 3)] * __fdiv_rn(S[c], fc);
  }
  g = tree_add<1>(g);                   // tree level 1: groups 2k, 2k+1
  g = tree_add<2>(g);
  g = tree_add<4>(g);
  g = tree_add<8>(g);
  g = tree_add<16>(g);                  // level 5
  return g + 0.0f;
}

// ---- block-level helpers (256 threads) ---------------------------------

// Exclusive prefix sum over the threads of a workgroup of `nthreads`
// (multiple of 64, <= 1024); returns the total in *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *total,
                                                         uint32_t *s_wave) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int j = 0; j < nw; ++j) {
    uint32_t s = s_wave[j];
    if (j < wv) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

constexpr int RADIX_BINS = 2048;   // 11-bit digits

// Among the nonzero keys of keys[0..m) (LDS; 0 marks an empty entry), find
// the key T such that exactly r of them are >= T (keys distinct,
// 1 <= r <= #nonzero).  Digits of 11 bits
// from bit `hi` down; every valid key must share the bits above `hi` (63:
// no assumption).  Stops as soon as a digit bucket is taken whole.  All
// threads call; s_hist holds RADIX_BINS counters.
__device__ __forceinline__ uint64_t radix_threshold(const uint64_t *keys, int m, int r, int hi,
                                    uint32_t *s_hist, uint64_t *s_state, uint32_t *s_wave) {
  const int t = threadIdx.x, nt = blockDim.x;
  uint64_t pmask = hi >= 63 ? 0ull : ~((2ull << hi) - 1);   // bits above hi
  if (t == 0) {
    uint64_t common = 0;
    for (int j = 0; j < m; ++j)
      if (keys[j]) { common = keys[j] & pmask; break; }
    s_state[0] = common;
  }
  __syncthreads();
  uint64_t prefix = s_state[0];
  int remaining = r;
  __syncthreads();
  for (; hi >= 0; hi -= 11) {
    const int lo = hi >= 10 ? hi - 10 : 0;
    const int nb = 1 << (hi - lo + 1);
    for (int j = t; j < nb; j += nt) s_hist[j] = 0;
    __syncthreads();
    for (int j = t; j < m; j += nt) {
      const uint64_t k = keys[j];
      if (k && (k & pmask) == prefix) atomicAdd(&s_hist[(uint32_t)(k >> lo) & (nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins nb-1-(per*t+j), top thread first
    const int per = (nb + nt - 1) / nt;
    uint32_t sum = 0;
    for (int j = 0; j < per; ++j) {
      const int bin = nb - 1 - (per * t + j);
      sum += bin >= 0 ? s_hist[bin] : 0u;
    }
    uint32_t total;
    const uint32_t above = block_exclusive_scan(sum, &total, s_wave);
    if (above < (uint32_t)remaining && (uint32_t)remaining <= above + sum) {
      uint32_t acc = above;
      for (int j = 0; j < per; ++j) {
        const int bin = nb - 1 - (per * t + j);
        const uint32_t c = bin >= 0 ? s_hist[bin] : 0u;
        if (acc + c >= (uint32_t)remaining) {
          s_state[0] = prefix | ((uint64_t)bin << lo);
          const uint32_t rem = (uint32_t)remaining - acc;
          s_state[1] = (uint64_t)rem | ((rem == c) ? (1ull << 63) : 0ull);
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
#ifdef CSA2_PROBE_TOPK
    CSA2_TS(7 + (63 - hi) / 11);
#endif
    prefix = s_state[0];
    const uint64_t st = s_state[1];
    pmask |= ((2ull << hi) - 1) & ~((1ull << lo) - 1);
    __syncthreads();
    remaining = (int)(uint32_t)st;
    if ((st >> 63) || lo == 0) return prefix;   // bucket taken whole, or every bit fixed
  }
  return prefix;
}

// Qbar of every sequence, once per call: the full scan's workgroups then
// read 2 KB each instead of every one of them summing the query heads (1,024
// workgroups reading the same 128 KB of queries contended for ~13 us).
__global__ void __launch_bounds__(SCAN_THREADS) qbar_kernel(const float *__restrict__ q, int heads,
                                                            float *__restrict__ qbar) {
  __shared__ float s_qbar[D];
  const uint32_t b = wg_x();
  compute_qbar<64>(q, heads, b, s_qbar);
  reinterpret_cast<float2 *>(qbar + (int64_t)b * D)[threadIdx.x] =
      reinterpret_cast<const float2 *>(s_qbar)[threadIdx.x];
}

// ---- full scan ----------------------------------------------------------

// 80 registers (room for six waves per SIMD).  The host launches two
// workgroups per compute unit, which streamed the rows faster than six
// waves per SIMD; a second block of prefetched rows per wave (114
// registers) did not help either (57.9 against 56.6 us at 1M, cold).
template <bool HIST>
__global__ void __launch_bounds__(SCAN_THREADS) __attribute__((amdgpu_waves_per_eu(6))) scan_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) float s_qbar[D];   // qbar32_index layout
  __shared__ uint32_t s_hist[HIST ? HIST_BINS : 1];
  __shared__ uint32_t s_wave[16];
  const int b = blockIdx.y;
  const uint32_t wx = wg_x();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  CSA2_TS(0);
  if (HIST) {
    for (int j = threadIdx.x; j < HIST_BINS; j += SCAN_THREADS) s_hist[j] = 0;
  }
  const uint8_t *codes = a.codes + (int64_t)b * a.capacity * CODE_BYTES;
  const uint8_t *scales = a.scales + (int64_t)b * a.capacity * SCALE_BYTES;
  float *scores = a.scores + (int64_t)b * a.score_stride;
  // Rows of the first chunk are requested before the query sum so the two
  // latencies overlap; afterwards each row of the next chunk is requested
  // as soon as the same row of the current chunk is consumed.
  Ctrl *ctrl = a.ctrl + b;
  int64_t n, nblk;
  if constexpr (HIST) {
    // Dynamic schedule.  Each wave scores chunks of 2 blocks (one per half
    // wave): its first chunk is fixed (wg_x() * 4 + wave); later ones
    // come from its group's counter, group g of the workgroups (wg_x() =
    // g mod G, G = min(64, grid), spanning every dispatch slot of the compute
    // units) sharing chunks first + g, first + g + G, ...  Older workgroups
    // win the issue arbiter, so a static split leaves the youngest finishing
    // last; here the waves finish within about one chunk of each other.
    // The grab of the next chunk is in flight while the current one is
    // scored, and so are the next chunk's rows.
    const int half = lane >> 5, j = lane & 31;
    const int ngrp = min(SCAN_GROUPS, (int)gridDim.x);   // every group has a workgroup
    const int grp = wx % ngrp;
    uint32_t *ctr = &ctrl->work[grp * 32];
    const int64_t nchunks = (a.nblk_grid + 1) / 2;
    const int64_t first = (int64_t)gridDim.x * 4;
    auto grab = [&]() {
      uint32_t k = 0;
      if (lane == 0) k = atomic_add_agent(ctr, 1u);
      return k;
    };
    // request order: length, query sum, first grab, first rows (the rows
    // unconditionally, clamped into the cache), so no use waits on a later
    // request
    const int64_t seq = a.seq_len[b];
    const float2 qv = reinterpret_cast<const float2 *>(a.qbar + (int64_t)b * D)[threadIdx.x];
    int64_t c = (int64_t)wx * 4 + wv;
    uint32_t pending = grab();
    BlockRows32 cur;
    {
      const int64_t blk = max((int64_t)0, min(2 * c + half, (int64_t)a.nblk_grid - 1));  // block 0 always exists
      load_block32(cur, codes + blk * BLOCK * CODE_BYTES, scales + blk * BLOCK * SCALE_BYTES, j);
    }
    __builtin_amdgcn_sched_barrier(0);
    n = clamp_len(seq, a.limit);
    nblk = (n + BLOCK - 1) / BLOCK;
    CSA2_CHECK((int64_t)a.nblk_grid * BLOCK <= a.capacity && nblk <= a.score_stride);
    *reinterpret_cast<float2 *>(s_qbar + qbar32_index(2 * threadIdx.x)) = qv;
    __syncthreads();
    CSA2_TS(1);
    const float *qb = s_qbar + qbar32_base(j);
    while (c < nchunks) {
      const int64_t blk = 2 * c + half;
      const int64_t cn = first + grp + (int64_t)ngrp * __builtin_amdgcn_readlane(pending, 0);
      pending = grab();
      // past the end (or the sequence) block 0 is re-read, an L2 hit
      int64_t nb = 2 * cn + half;
      if (cn >= nchunks || nb >= nblk) nb = 0;
      const int cnt = (int)max((int64_t)1, min((int64_t)BLOCK, n - blk * BLOCK));
      const float sc = block_score32(cur, cnt, qb, codes + nb * BLOCK * CODE_BYTES,
                                     scales + nb * BLOCK * SCALE_BYTES, j);
      if (j == 0 && blk < nblk) {
        scores[blk] = sc;
        atomicAdd(&s_hist[ord_key(sc) >> HIST_SHIFT], 1u);
      }
      c = cn;
    }
  } else {
    // static schedule (score export): wave chunks wg_x() * 4 + wave,
    // then every gridDim.x * 4 chunks
    const int half = lane >> 5, j = lane & 31;
    const int64_t nchunks = (a.nblk_grid + 1) / 2;
    const int64_t step = (int64_t)gridDim.x * 4;
    int64_t c = (int64_t)wx * 4 + wv;
    BlockRows32 cur;
    {
      const int64_t blk = max((int64_t)0, min(2 * c + half, (int64_t)a.nblk_grid - 1));
      load_block32(cur, codes + blk * BLOCK * CODE_BYTES, scales + blk * BLOCK * SCALE_BYTES, j);
    }
    n = clamp_len(a.seq_len[b], a.limit);
    nblk = (n + BLOCK - 1) / BLOCK;
    CSA2_CHECK((int64_t)a.nblk_grid * BLOCK <= a.capacity && nblk <= a.score_stride);
    if (a.qbar) {
      *reinterpret_cast<float2 *>(s_qbar + qbar32_index(2 * threadIdx.x)) =
          reinterpret_cast<const float2 *>(a.qbar + (int64_t)b * D)[threadIdx.x];
      __syncthreads();
    } else {
      compute_qbar<16, true>(a.q, a.heads, b, s_qbar);
    }
    CSA2_TS(1);
    const float *qb = s_qbar + qbar32_base(j);
    for (; c < nchunks; c += step) {
      const int64_t blk = 2 * c + half;
      int64_t nb = 2 * (c + step) + half;
      if (c + step >= nchunks || nb >= nblk) nb = 0;
      const int cnt = (int)max((int64_t)1, min((int64_t)BLOCK, n - blk * BLOCK));
      const float sc = block_score32(cur, cnt, qb, codes + nb * BLOCK * CODE_BYTES,
                                     scales + nb * BLOCK * SCALE_BYTES, j);
      if (j == 0) {
        if (blk < nblk) {
          scores[blk] = sc;
          if (HIST) atomicAdd(&s_hist[ord_key(sc) >> HIST_SHIFT], 1u);
        } else if (a.fill_invalid && blk < a.score_stride) {
          scores[blk] = -__builtin_huge_valf();
        }
      }
    }
  }
  if (!HIST) return;
  __syncthreads();
  CSA2_TS(2);
  uint32_t *gh = a.hist + (int64_t)b * HIST_COPIES * HIST_BINS;
  {
    uint32_t *mine = gh + (wx % HIST_COPIES) * HIST_BINS;
    for (int j = threadIdx.x; j < HIST_BINS; j += SCAN_THREADS) {
      uint32_t c = s_hist[j];
      if (c) atomic_add_agent(mine + j, c);
    }
  }
  // The threshold digit is found by every workgroup of the select kernel
  // from these copies (no last-workgroup hand-off here); the select
  // kernel's last workgroup clears the copies and the work counters.
}

// ---- full scan of a batch over the flattened (sequence, chunk) space --------
//
// The same scoring and the same per-sequence outputs (scores, the 8 digit
// histogram copies) as scan_kernel<true>, for batches: the chunks of 2 blocks
// of every sequence are laid end to end (sequence b's chunks after those of
// sequences 0..b-1), the whole range is cut into SCAN_GROUPS equal contiguous
// regions, and the workgroups of group g (wg_x() mod SCAN_GROUPS) take the
// chunks of region g, the first 4 per workgroup fixed, the rest from the
// group's counter.  So no workgroup idles while long sequences still have
// chunks, whatever the length mix.  Each wave keeps its current sequence's
// Qbar in LDS and reloads it when its next chunk lies in another sequence
// (a region spans one or a few sequences); its digit counts collect in a
// per-wave LDS histogram, added to the sequence's copy when the wave moves
// on and at the end.
constexpr int SCAN_FLAT_MAXB = 512;     // sequences whose chunk prefix fits in LDS
// Needs batch <= SCAN_FLAT_MAXB and batch * ceil(blocks / 2) < 2^31 (checked
// by the host), so chunk indices are 32-bit.
__global__ void __launch_bounds__(SCAN_THREADS) __attribute__((amdgpu_waves_per_eu(5)))
scan_flat_kernel(ScanArgs a, int32_t batch) {
  __shared__ __attribute__((aligned(16))) float s_qbar[4][D];   // per wave, qbar32_index layout
  __shared__ int32_t s_pre[SCAN_FLAT_MAXB + 1];    // chunks before sequence b
  __shared__ int64_t s_len[SCAN_FLAT_MAXB];        // clamped lengths
  __shared__ uint32_t s_wave[16];
  __shared__ uint32_t s_hw[4][HIST_BINS];          // per wave: digit counts of its current sequence
  const int lane = threadIdx.x & 63, t = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int half = lane >> 5, j = lane & 31;
  const uint32_t wx = wg_x();
  CSA2_TS(0);
  uint32_t *hw = s_hw[wv];
#pragma unroll
  for (int i = 0; i < HIST_BINS / 64; ++i) hw[lane + 64 * i] = 0;
  // the wave's counts into sequence sb's histogram copy, then cleared
  auto flush = [&](int sb) {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint32_t *gh = a.hist + ((int64_t)sb * HIST_COPIES + (wx % HIST_COPIES)) * HIST_BINS;
#pragma unroll
    for (int i = 0; i < HIST_BINS / 64; ++i) {
      const uint32_t v = hw[lane + 64 * i];
      if (v) {
        __hip_atomic_fetch_add(&gh[lane + 64 * i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hw[lane + 64 * i] = 0;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  CSA2_CHECK(batch <= SCAN_FLAT_MAXB);
  // lengths -> chunks per sequence -> exclusive prefix, 256 sequences a pass
  uint32_t carry = 0;
  for (int b0 = 0; b0 < batch; b0 += SCAN_THREADS) {
    const int b = b0 + t;
    int64_t n = 0;
    if (b < batch) {
      n = clamp_len(a.seq_len[b], a.limit);
      s_len[b] = n;
    }
    const uint32_t ch = (uint32_t)(((n + BLOCK - 1) / BLOCK + 1) / 2);
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(ch, &tot, s_wave);
    if (b < batch) s_pre[b] = (int32_t)(carry + ex);
    carry += tot;
  }
  if (t == 0) s_pre[batch] = (int32_t)carry;
  __syncthreads();
  const int total = s_pre[batch];
  const int ngrp = min(SCAN_GROUPS, (int)gridDim.x);
  const int grp = wx % ngrp;
  const int in_grp = wx / ngrp;                        // workgroup index inside the group
  const int per_grp = ((int)gridDim.x - grp + ngrp - 1) / ngrp;  // workgroups of this group
  const int r0 = (int)((int64_t)total * grp / ngrp), r1 = (int)((int64_t)total * (grp + 1) / ngrp);
  uint32_t *ctr = &a.ctrl[0].work[grp * 32];
  const int first = 4 * per_grp;                               // fixed chunks of the group
  auto grab = [&]() {
    uint32_t k = 0;
    if (lane == 0) k = atomic_add_agent(ctr, 1u);
    return k;
  };
  // chunk -> sequence: largest b with s_pre[b] <= c (wave-uniform)
  auto seq_of = [&](int c) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return __builtin_amdgcn_readfirstlane(lo);
  };
  // this half-wave's block of chunk c (sequence b) and its first row; row 0
  // of sequence 0 when past the region or the sequence (valid, never scored)
  auto rows_of = [&](int c, int b, int &blk) {
    blk = 2 * (c - s_pre[b]) + half;
    const bool ok = c < r1 && (int64_t)blk * BLOCK < s_len[b];
    return ok ? (int64_t)b * a.capacity + (int64_t)blk * BLOCK : (int64_t)0;
  };
  int c = r0 + 4 * in_grp + wv;
  uint32_t pending = grab();
  int cb = seq_of(c < r1 ? c : r0);
  int blk;
  BlockRows32 cur;
  {
    const int64_t row = rows_of(c, cb, blk);
    load_block32(cur, a.codes + row * CODE_BYTES, a.scales + row * SCALE_BYTES, j);
  }
  int qb_seq = -1;
  float *qbw = s_qbar[wv];
  CSA2_TS(1);
  while (c < r1) {
    if (cb != qb_seq) {
      if (qb_seq >= 0) flush(qb_seq);
      // this wave's Qbar: 8 floats per lane (wave-local LDS, qbar32_index layout)
      const float4 *src = reinterpret_cast<const float4 *>(a.qbar + (int64_t)cb * D);
      const float4 v0 = src[2 * lane], v1 = src[2 * lane + 1];
      *reinterpret_cast<float4 *>(qbw + qbar32_index(8 * lane)) = v0;
      *reinterpret_cast<float4 *>(qbw + qbar32_index(8 * lane + 4)) = v1;
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      qb_seq = cb;
    }
    const int64_t nl = s_len[cb];                               // wave-uniform
    const int64_t n = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(nl >> 32)) << 32) |
                                (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)nl));
    const int cn_raw = r0 + first + (int)__builtin_amdgcn_readlane(pending, 0);
    pending = grab();
    const int cn = cn_raw < r1 ? cn_raw : r1;
    const int nbq = seq_of(cn < r1 ? cn : r0);
    int blk_next;
    const int64_t nrow = rows_of(cn, nbq, blk_next);
    const bool valid = (int64_t)blk * BLOCK < n;
    const int cnt = (int)max((int64_t)1, min((int64_t)BLOCK, n - (int64_t)blk * BLOCK));
    const float sc = block_score32(cur, cnt, qbw + qbar32_base(j), a.codes + nrow * CODE_BYTES,
                                   a.scales + nrow * SCALE_BYTES, j);
    if (j == 0 && valid) {
      a.scores[(int64_t)cb * a.score_stride + blk] = sc;
      atomicAdd(&hw[ord_key(sc) >> HIST_SHIFT], 1u);
    }
    c = cn;
    cb = nbq;
    blk = blk_next;
  }
  if (qb_seq >= 0) flush(qb_seq);
  CSA2_TS(2);
}

// ---- select (after a full scan) ------------------------------------------

struct SelectArgs {
  const int64_t *seq_len;
  int64_t limit;
  const float *scores;      // [batch][score_stride]
  int64_t score_stride;
  Ctrl *ctrl;
  uint32_t *bitmap;         // [batch][nwords]
  int32_t nwords;           // per row, even
  uint64_t *cands;          // [batch][CAND_COPIES][cand_stride]
  int64_t cand_stride;
  int32_t R;                // first-level count (pool or topk)
  int32_t *first_out;       // [batch][R]: pool_out, or idx_out when no pool
  int32_t topk;             // second level (pool > 0) or 0
  int32_t *idx_out;         // [batch][topk] when topk > 0
  int32_t lds_keys;         // dynamic LDS keys (>= R, <= LDS_KEYS)
  float *pool_scores;       // [batch][R]: scores of first_out in its order (or NULL)
  uint32_t *hist;           // [batch][HIST_COPIES][HIST_BINS] from the full scan (cleared here)
};

__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
  return ((uint64_t)ord_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

// Ids of the set bits of bitmap[0..nwords), ascending, into s_out[0..len)
// (LDS) and then out[0..len) with coalesced stores, -1 padded.  All
// threads.  Each thread owns a contiguous run of words; with MAXW > 0 the run
// (at most MAXW words) is loaded once into registers, one memory round trip;
// MAXW = 0 streams it twice in batches of 16 (any length).
template <int MAXW>
__device__ __forceinline__ void compact_bitmap_t(const uint32_t *bm, int nwords, int32_t *out,
                                                 int32_t *s_out, int len, uint32_t *s_wave) {
  constexpr int U = MAXW > 0 ? MAXW : 16;
  const int t = threadIdx.x, nt = blockDim.x;
  const int per = (nwords + nt - 1) / nt;
  const int w0 = min(nwords, t * per), w1 = min(nwords, w0 + per);
  uint32_t v[U];
  uint32_t cnt = 0;
  if (MAXW > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_agent(bm + max(0, min(w0 + u, w1 - 1)));   // clamped: no branch
#pragma unroll
    for (int u = 0; u < U; ++u) cnt += (w0 + u < w1) ? __popc(v[u]) : 0u;
  } else {
    for (int wb = w0; wb < w1; wb += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld_agent(bm + min(wb + u, w1 - 1));
#pragma unroll
      for (int u = 0; u < U; ++u) cnt += (wb + u < w1) ? __popc(v[u]) : 0u;
    }
  }
  uint32_t total;
  uint32_t off = block_exclusive_scan(cnt, &total, s_wave);
  for (int wb = w0; wb < w1 && off < (uint32_t)len; wb += U) {
    if (MAXW == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld_agent(bm + min(wb + u, w1 - 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t bits = (wb + u < w1) ? v[u] : 0u;
      while (bits && off < (uint32_t)len) {
        const int bpos = __ffs(bits) - 1;
        bits &= bits - 1;
        s_out[off++] = (wb + u) * 32 + bpos;
      }
    }
  }
  for (int j = (int)total + t; j < len; j += nt) s_out[j] = -1;
  __syncthreads();
  for (int j = t; j < len; j += nt) out[j] = s_out[j];
}

__device__ __forceinline__ void compact_bitmap(const uint32_t *bm, int nwords, int32_t *out,
                                               int32_t *s_out, int len, uint32_t *s_wave) {
  const int per = (nwords + (int)blockDim.x - 1) / (int)blockDim.x;
  if (per <= 16)
    compact_bitmap_t<16>(bm, nwords, out, s_out, len, s_wave);
  else if (per <= 32)
    compact_bitmap_t<32>(bm, nwords, out, s_out, len, s_wave);
  else
    compact_bitmap_t<0>(bm, nwords, out, s_out, len, s_wave);
}

__device__ __forceinline__ float unord_key(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

constexpr int TIE_MAX = 256;     // threshold-bin members ranked pairwise

#ifndef CSA2_TOPK_TS
#define CSA2_TOPK_TS(k) do { } while (0)
#endif

constexpr int SEL_PAD = 64;          // s_sel slots past len: unchosen lanes' stores land there
constexpr int TOPK_HIST_BINS = RADIX_BINS + 64;   // block top-k bins; the last 64 take empty entries

// Ordered compaction of the keys >= T (nonzero; none when reff <= 0): the
// four wave totals are exchanged through LDS, then each wave's chosen
// entries follow in list order.  Ids to s_sel[0..len) (-1 padded) and,
// unless out is NULL, to out.
template <int KPT>
__device__ __forceinline__ void compact_ge(const uint64_t (&kr)[KPT], const int32_t (&ids)[KPT], uint64_t T,
                                           int reff, int32_t *out, int32_t *s_sel, int len, uint32_t *s_wtot) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  uint32_t wtot = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    wtot += (uint32_t)__popcll(__ballot(reff > 0 && kr[k] != 0 && kr[k] >= T));
  if (lane == 0) s_wtot[wv] = wtot;
  __syncthreads();
  uint32_t base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = s_wtot[w];
    base += w < wv ? v : 0u;
    total += v;
  }
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool f = reff > 0 && kr[k] != 0 && kr[k] >= T;
    const uint64_t mask = __ballot(f);
    const uint32_t pos = base + lanes_below(mask);
    s_sel[(f && pos < (uint32_t)len) ? pos : len + lane] = ids[k];
    base += (uint32_t)__popcll(mask);
  }
  for (int j = (int)total + t; j < len; j += 256) s_sel[j] = -1;
  __syncthreads();
  if (out)
    for (int j = t; j < len; j += 256) out[j] = s_sel[j];
}

// The bin of s_hist[0..RADIX_BINS) (counts, bin RADIX_BINS - 1 the highest)
// holding the r-th largest key, found by one wave on its own (every wave of
// a workgroup gets the same answer from the same counts, so no exchange is
// needed): lane l sums bins [2016 - 32 l, 2047 - 32 l] (read in a rotated
// order, so eight neighbouring lanes cover all banks), a wave scan finds the
// lane, and lanes 0..31 scan that lane's bins.  *rem: keys still needed from
// the bin, *cbin: keys in it, *total: keys in all bins.  Returns false when
// the bins hold fewer than r keys.
__device__ __forceinline__ bool find_threshold_bin(const uint32_t *s_hist, int r, uint32_t *bstar, uint32_t *rem,
                                                   uint32_t *cbin, uint32_t *total) {
  const int lane = threadIdx.x & 63;
  const uint32_t *hb = s_hist + (RADIX_BINS - 32 - 32 * lane);
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = *reinterpret_cast<const uint4 *>(hb + 4 * ((i + lane) & 7));
    sum += v.x + v.y + v.z + v.w;
  }
  const uint32_t incl = wave_incl_scan(sum);
  *total = __builtin_amdgcn_readlane(incl, 63);
  const uint64_t fm = __ballot(incl - sum < (uint32_t)r && (uint32_t)r <= incl);
  const int L = fm ? __builtin_ctzll(fm) : 0;
  const uint32_t aboveL = __builtin_amdgcn_readlane(incl - sum, L);
  const uint32_t cc = lane < 32 ? s_hist[RADIX_BINS - 1 - 32 * L - lane] : 0u;
  const uint32_t ic = wave_incl_scan(cc);
  const uint64_t bm = __ballot(lane < 32 && aboveL + ic - cc < (uint32_t)r && (uint32_t)r <= aboveL + ic);
  const int B = bm ? __builtin_ctzll(bm) : 0;
  *bstar = (uint32_t)(RADIX_BINS - 1 - 32 * L - B);
  *rem = (uint32_t)r - aboveL - __builtin_amdgcn_readlane(ic - cc, B);
  *cbin = __builtin_amdgcn_readlane(cc, B);
  return fm != 0 && bm != 0;
}

// Register form of the block top-k (256 threads): wave w holds list
// entries 64*KPT*w + 64k + lane, k < KPT (a contiguous quarter of the list:
// keys kr, 0 = empty, their float scores sc and ids); s_keys is the same
// list in LDS, read only by the radix fallback.  The chosen entries' ids,
// in list order, go to s_sel[0..len) (-1 padded; s_sel holds len + SEL_PAD
// entries) and, unless out is NULL, to out.  s_hist holds TOPK_HIST_BINS
// counters.
//
// One pass of RADIX_BINS linear bins over the scores' range [lo, hi]
// (monotone in the score, equal scores share a bin; empty entries count in
// the extra bins).  Every wave then finds the bin holding the r-th largest
// key on its own (lane sums of 32 bins, a wave scan, then the found lane's
// 32 bins), so no exchange is needed for it.  The bin's members, a handful,
// are ranked pairwise; each chosen member counts itself for its wave and
// each wave counts its keys above the bin, so every wave knows its output
// offset when the threshold is published and the ordered compaction
// follows without another exchange (five workgroup barriers in all).  A
// NaN or infinite score, a degenerate range or a crowded bin falls back to
// the radix select above.
template <int KPT>
__device__ __forceinline__ void select_top_regs(const uint64_t (&kr)[KPT], const float (&sc)[KPT],
                                                const int32_t (&ids)[KPT], const uint64_t *s_keys, int m, int r,
                                                int32_t *out, int32_t *s_sel, int len, uint32_t *s_hist,
                                                uint64_t *s_state, uint32_t *s_wave) {
  __shared__ uint32_t s_red[12];
  __shared__ uint32_t s_cnt[12];     // [w]: keys above the threshold bin; [4 + w]: chosen members; [8]: member slots
  __shared__ __attribute__((aligned(16))) uint64_t s_tie[TIE_MAX];
  __shared__ uint8_t s_tiew[TIE_MAX];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // ---- valid count and the range of the keys' score halves
  uint32_t hmax = 0u, hmin1 = 0xFFFFFFFFu, cnt = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const uint32_t h = (uint32_t)(kr[k] >> 32);
    hmax = max(hmax, h);
    hmin1 = min(hmin1, h - 1u);                    // an empty entry (0) wraps to the top
    cnt += (uint32_t)__popcll(__ballot(kr[k] != 0));
  }
#pragma unroll
  for (int k = 0; k < RADIX_BINS / 256; ++k) s_hist[t + 256 * k] = 0;
  if (t < TOPK_HIST_BINS - RADIX_BINS) s_hist[RADIX_BINS + t] = 0;
  if (t < 9) s_cnt[t] = 0;
  hmax = wave_umax(hmax);
  hmin1 = wave_umin(hmin1);
  if (lane == 0) { s_red[wv] = cnt; s_red[4 + wv] = hmin1; s_red[8 + wv] = hmax; }
  __syncthreads();
  CSA2_TOPK_TS(1);
  const uint32_t nvalid = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  const uint32_t umin = min(min(s_red[4], s_red[5]), min(s_red[6], s_red[7])) + 1u;
  const uint32_t umax = max(max(s_red[8], s_red[9]), max(s_red[10], s_red[11]));
  r = min(r, (int)nvalid);
  if (r <= 0 || r == (int)nvalid) {                // none, or every valid key
    compact_ge<KPT>(kr, ids, r <= 0 ? ~0ull : 0ull, r, out, s_sel, len, s_wave);
    return;
  }
  // finite scores only: a NaN's or an infinity's key lies at or beyond
  // key(-inf) = 0x007FFFFF and key(+inf) = 0xFF800000
  const float lo = unord_key(umin), hi = unord_key(umax);
  const float inv = (float)RADIX_BINS * __builtin_amdgcn_rcpf(hi - lo);   // any positive scale keeps bins monotone
  if (umin >= umax || umin <= 0x007FFFFFu || umax >= 0xFF800000u || !(inv < __builtin_huge_valf()) ||
      !(inv > 0.f)) {
    const uint64_t T = radix_threshold(s_keys, m, r, 63, s_hist, s_state, s_wave);
    compact_ge<KPT>(kr, ids, T, r, out, s_sel, len, s_wave);
    return;
  }
  uint32_t bin[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int bf = min(RADIX_BINS - 1, (int)((sc[k] - lo) * inv));
    bin[k] = kr[k] != 0 ? (uint32_t)bf : (uint32_t)(RADIX_BINS + lane);   // empty: a lane's own spare bin
    atomicAdd(&s_hist[bin[k]], 1u);
  }
  __syncthreads();
  CSA2_TOPK_TS(2);
  // ---- the bin holding the r-th largest key, found by every wave alone
  uint32_t bstar, rem, cbin, binned;
  const bool ok = find_threshold_bin(s_hist, r, &bstar, &rem, &cbin, &binned);
  CSA2_TOPK_TS(3);
  if (!ok || cbin > (uint32_t)TIE_MAX) {           // uniform: every wave read the same bins
    const uint64_t T = radix_threshold(s_keys, m, r, 63, s_hist, s_state, s_wave);
    compact_ge<KPT>(kr, ids, T, r, out, s_sel, len, s_wave);
    return;
  }
  // ---- the bin's members into LDS; each wave's count of keys above the bin
  uint32_t above_w = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    above_w += (uint32_t)__popcll(__ballot(bin[k] - bstar - 1u < (uint32_t)RADIX_BINS - 1u - bstar));
    if (bin[k] == bstar) {
      const uint32_t slot = atomicAdd(&s_cnt[8], 1u);
      s_tie[slot] = kr[k];
      s_tiew[slot] = (uint8_t)wv;
    }
  }
  if (lane == 0) s_cnt[wv] = above_w;
  __syncthreads();
  CSA2_TOPK_TS(4);
  // ---- rank the members pairwise: the rem-th largest is the threshold T;
  // a member is chosen when fewer than rem members beat it (that is, when
  // it is >= T), and counts itself for its wave
  if (t < (int)cbin) {
    const uint64_t k = s_tie[t];
    uint32_t gt = 0, ge = 0;
    uint32_t i2 = 0;
    for (; i2 + 2 <= cbin; i2 += 2) {             // two members per 16-byte read
      const uint64_t o0 = s_tie[i2], o1 = s_tie[i2 + 1];
      gt += (o0 > k ? 1u : 0u) + (o1 > k ? 1u : 0u);
      ge += (o0 >= k ? 1u : 0u) + (o1 >= k ? 1u : 0u);
    }
    if (i2 < cbin) {
      const uint64_t o = s_tie[i2];
      gt += o > k ? 1u : 0u;
      ge += o >= k ? 1u : 0u;
    }
    if (gt < rem) {
      atomicAdd(&s_cnt[4 + s_tiew[t]], 1u);
      if (rem <= ge) s_state[0] = k;
    }
  }
  __syncthreads();
  CSA2_TOPK_TS(5);
  const uint64_t T = s_state[0];
  // ---- ordered compaction at the offsets the counts give
  uint32_t base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = s_cnt[w] + s_cnt[4 + w];
    base += w < wv ? v : 0u;
    total += v;
  }
  CSA2_TOPK_TS(6);
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool f = kr[k] >= T;                     // T is a real key, so f implies nonzero
    const uint64_t mask = __ballot(f);
    const uint32_t pos = base + lanes_below(mask);
    s_sel[(f && pos < (uint32_t)len) ? pos : len + lane] = ids[k];
    base += (uint32_t)__popcll(mask);
  }
  for (int j = (int)total + t; j < len; j += 256) s_sel[j] = -1;
  __syncthreads();
  CSA2_TOPK_TS(7);
  if (out)
    for (int j = t; j < len; j += 256) out[j] = s_sel[j];
}

// Top r of the list s_keys[0..m) (LDS, 0 = empty entry, m <= 256 * KPT):
// the chosen entries' s_ids, in list order, go to s_sel (LDS, len +
// SEL_PAD entries) and, unless out is NULL, to out[0..len), -1 padded.  All
// 256 threads; wave w takes the contiguous quarter of the list
// select_top_regs expects; s_hist holds TOPK_HIST_BINS counters.
template <int KPT>
__device__ __forceinline__ void select_top(const uint64_t *s_keys, const int32_t *s_ids, int m, int r, int32_t *out,
                           int32_t *s_sel, int len, uint32_t *s_hist, uint64_t *s_state,
                           uint32_t *s_wave) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t kr[KPT];
  float sc[KPT];
  int32_t ids[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int e = 64 * KPT * wv + 64 * k + lane;
    const int j = min(e, m - 1);
    kr[k] = e < m ? s_keys[j] : 0ull;
    sc[k] = unord_key((uint32_t)(kr[k] >> 32));
    ids[k] = s_ids[j];
  }
  select_top_regs<KPT>(kr, sc, ids, s_keys, m, r, out, s_sel, len, s_hist, s_state, s_wave);
}

// Runtime dispatch on the list length (up to 8,192 entries).
__device__ __forceinline__ void select_in_lds(const uint64_t *s_keys, const int32_t *s_ids, int m, int r, int32_t *out,
                              int32_t *s_sel, int len, uint32_t *s_hist, uint64_t *s_state,
                              uint32_t *s_wave) {
  if (m <= 2048)
    select_top<8>(s_keys, s_ids, m, r, out, s_sel, len, s_hist, s_state, s_wave);
  else
    select_top<32>(s_keys, s_ids, m, r, out, s_sel, len, s_hist, s_state, s_wave);
}

// Threshold of a top-r choice over the LDS list s_keys[0..m) (0 = empty
// entry; keys distinct), for any workgroup of up to 16 waves: T such that
// exactly min(r, #nonzero) nonzero keys are >= T (0 when r >= #nonzero, ~0
// when r <= 0).  Thread t holds entries t + nt k, k < KPT (m <= nt KPT).
// The block top-k's method without its compaction: one pass of RADIX_BINS
// linear bins over the keys' score range, the threshold bin found by every
// wave alone, its members ranked pairwise (four workgroup barriers); a NaN
// or infinite score, a degenerate range or a crowded bin falls back to the
// radix select.  s_hist holds TOPK_HIST_BINS counters.
struct LinearLds {
  uint32_t red[3 * 16];   // per wave: valid count, min key - 1, max key
  uint32_t ntie;
  uint64_t tie[TIE_MAX];
};
__device__ __forceinline__ LinearLds &linear_lds() {
  __shared__ LinearLds s;   // one object, whatever KPT the caller picks
  return s;
}

template <int KPT>
__device__ __forceinline__ uint64_t threshold_linear(const uint64_t *s_keys, int m, int r, uint32_t *s_hist,
                                                     uint64_t *s_state, uint32_t *s_wave) {
  LinearLds &L = linear_lds();
  uint32_t *s_red = L.red;
  uint32_t &s_nt = L.ntie;
  uint64_t *s_tie = L.tie;
  const int t = threadIdx.x, nt = blockDim.x, lane = t & 63, wv = t >> 6, nw = nt >> 6;
  uint64_t kr[KPT];
  uint32_t hmax = 0u, hmin1 = 0xFFFFFFFFu, cnt = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    kr[k] = t + nt * k < m ? s_keys[t + nt * k] : 0ull;
    const uint32_t h = (uint32_t)(kr[k] >> 32);
    hmax = max(hmax, h);
    hmin1 = min(hmin1, h - 1u);                    // an empty entry (0) wraps to the top
    cnt += (uint32_t)__popcll(__ballot(kr[k] != 0));
  }
  for (int j = t; j < TOPK_HIST_BINS; j += nt) s_hist[j] = 0;
  if (t == 0) s_nt = 0;
  hmax = wave_umax(hmax);
  hmin1 = wave_umin(hmin1);
  if (lane == 0) { s_red[wv] = cnt; s_red[16 + wv] = hmin1; s_red[32 + wv] = hmax; }
  __syncthreads();
  uint32_t nvalid = 0, umin = 0xFFFFFFFFu, umax = 0u;
  for (int w = 0; w < nw; ++w) {
    nvalid += s_red[w];
    umin = min(umin, s_red[16 + w]);
    umax = max(umax, s_red[32 + w]);
  }
  umin += 1u;
  r = min(r, (int)nvalid);
  if (r <= 0 || r == (int)nvalid) {
    __syncthreads();                               // every wave has read s_red: a next call may write it
    return r <= 0 ? ~0ull : 0ull;
  }
  const float lo = unord_key(umin), hi = unord_key(umax);
  const float inv = (float)RADIX_BINS * __builtin_amdgcn_rcpf(hi - lo);
  if (umin >= umax || umin <= 0x007FFFFFu || umax >= 0xFF800000u || !(inv < __builtin_huge_valf()) ||
      !(inv > 0.f))
    return radix_threshold(s_keys, m, r, 63, s_hist, s_state, s_wave);
  uint32_t bin[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const float sc = unord_key((uint32_t)(kr[k] >> 32));
    const int bf = min(RADIX_BINS - 1, (int)((sc - lo) * inv));
    bin[k] = kr[k] != 0 ? (uint32_t)bf : (uint32_t)(RADIX_BINS + lane);
    atomicAdd(&s_hist[bin[k]], 1u);
  }
  __syncthreads();
  uint32_t bstar, rem, cbin, binned;
  const bool ok = find_threshold_bin(s_hist, r, &bstar, &rem, &cbin, &binned);
  if (!ok || cbin > (uint32_t)TIE_MAX)             // uniform: every wave read the same bins
    return radix_threshold(s_keys, m, r, 63, s_hist, s_state, s_wave);
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    if (bin[k] == bstar) s_tie[atomicAdd(&s_nt, 1u)] = kr[k];
  __syncthreads();
  if (t < (int)cbin) {
    const uint64_t k = s_tie[t];
    uint32_t gt = 0, ge = 0;
    for (uint32_t i2 = 0; i2 < cbin; ++i2) {
      const uint64_t o = s_tie[i2];
      gt += o > k ? 1u : 0u;
      ge += o >= k ? 1u : 0u;
    }
    if (gt < rem && rem <= ge) s_state[0] = k;  // k is the rem-th largest of the bin
  }
  __syncthreads();
  const uint64_t T = s_state[0];
  __syncthreads();                                 // s_state and s_hist are free again
  return T;
}

// Threshold only, over an LDS list of up to MAXK * blockDim entries
// (MAXK = 16 or 32): the fewest registers per thread that hold it.
template <int MAXK>
__device__ __forceinline__ uint64_t threshold_in_lds(const uint64_t *s_keys, int m, int r, uint32_t *s_hist,
                                                     uint64_t *s_state, uint32_t *s_wave) {
  static_assert(MAXK == 16 || MAXK == 32, "list size class");
  const int nt = blockDim.x;
  if (m <= 4 * nt) return threshold_linear<4>(s_keys, m, r, s_hist, s_state, s_wave);
  if (m <= 8 * nt) return threshold_linear<8>(s_keys, m, r, s_hist, s_state, s_wave);
  if (MAXK == 16 || m <= 16 * nt) return threshold_linear<16>(s_keys, m, r, s_hist, s_state, s_wave);
  return threshold_linear<MAXK>(s_keys, m, r, s_hist, s_state, s_wave);
}

__global__ void __launch_bounds__(SCAN_THREADS) select_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint64_t s_keys[];                 // lds_keys
  __shared__ int32_t s_ids[LDS_KEYS];
  __shared__ int32_t s_sel[CSA2_TOPK_MAX + SEL_PAD];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[TOPK_HIST_BINS];   // also 64-bit keys (radix_select_keys)
  __shared__ uint64_t s_state[2];
  __shared__ uint32_t s_wave[16];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  Ctrl *ctrl = a.ctrl + b;
  const int t = threadIdx.x, nt = blockDim.x;
  const int64_t n = clamp_len(a.seq_len[b], a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;
  const float *scores = a.scores + (int64_t)b * a.score_stride;
  uint32_t *bm = a.bitmap + (int64_t)b * a.nwords;
  uint64_t *cands = a.cands + (int64_t)b * CAND_COPIES * a.cand_stride;
  uint32_t *gh = a.hist + (int64_t)b * HIST_COPIES * HIST_BINS;
  CSA2_TS(8);
  // This wave's scores (up to PRE chunks of 64 blocks), requested together
  // with the histogram copies: one memory round trip for both.
  constexpr int PRE = 4;
  const int chunks = a.nwords / 2;
  const uint32_t wx = wg_x();
  const int ch0 = wx * 4 + wv, chs = gridDim.x * 4;
  float sv[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int64_t id = (int64_t)(ch0 + k * chs) * 64 + lane;
    sv[k] = scores[id < nblk ? id : 0];
  }
  // Threshold digit, found by every workgroup from the scan's copies:
  // thread t owns bins HIST_BINS-1-(4t+j), j = 0..3 (top thread first).
  constexpr int PER = HIST_BINS / SCAN_THREADS;
  uint32_t hv[PER][HIST_COPIES];
#pragma unroll
  for (int j = 0; j < PER; ++j)
#pragma unroll
    for (int k = 0; k < HIST_COPIES; ++k) hv[j][k] = gh[k * HIST_BINS + (HIST_BINS - 1 - (PER * t + j))];
  __builtin_amdgcn_sched_barrier(0);
  const bool all = (int64_t)a.R >= nblk;
  uint32_t thr = 0, need = 0;
  {
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      c[j] = 0;
#pragma unroll
      for (int k = 0; k < HIST_COPIES; ++k) c[j] += hv[j][k];
      sum += c[j];
    }
    uint32_t total;
    const uint32_t above = block_exclusive_scan(sum, &total, s_wave);
    const uint32_t R = (uint32_t)a.R;
    if (t == 0) s_state[0] = 0;
    __syncthreads();
    if (!all && above < R && R <= above + sum) {
      uint32_t acc = above;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (acc < R && R <= acc + c[j])
          s_state[0] = ((uint64_t)(HIST_BINS - 1 - (PER * t + j)) << 32) | (uint64_t)(R - acc);
        acc += c[j];
      }
    }
    __syncthreads();
    thr = (uint32_t)(s_state[0] >> 32);
    need = (uint32_t)s_state[0];
  }
  // 64 ids per chunk: the ballot of ids above the tie digit is OR-ed into
  // the (zeroed) bitmap; ids in the tie digit go to one of 8 lists, with one
  // counter reservation per wave for all its chunks
  uint64_t *mylist = cands + (wx % CAND_COPIES) * a.cand_stride;
  uint32_t *mycount = &ctrl->ncand[wx % CAND_COPIES];
  for (int base_ch = ch0; base_ch < chunks; base_ch += PRE * chs) {
    if (base_ch != ch0) {
#pragma unroll
      for (int k = 0; k < PRE; ++k) {
        const int64_t id = (int64_t)(base_ch + k * chs) * 64 + lane;
        sv[k] = scores[id < nblk ? id : 0];
      }
    }
    uint64_t m_tie[PRE];
    uint32_t key_hi[PRE];
    uint32_t ntie = 0;
#pragma unroll
    for (int k = 0; k < PRE; ++k) {
      const int ch = base_ch + k * chs;
      const int64_t id = (int64_t)ch * 64 + lane;
      key_hi[k] = ord_key(sv[k]);
      const uint32_t dg = key_hi[k] >> HIST_SHIFT;
      const bool valid = ch < chunks && id < nblk;
      const bool in = valid && (all || dg > thr);
      const bool tie = valid && !all && dg == thr;
      const uint64_t m_in = __ballot(in);
      if (lane == 0 && (uint32_t)m_in) atomicOr(bm + 2 * ch, (uint32_t)m_in);
      if (lane == 1 && (uint32_t)(m_in >> 32)) atomicOr(bm + 2 * ch + 1, (uint32_t)(m_in >> 32));
      m_tie[k] = __ballot(tie);
      ntie += (uint32_t)__popcll(m_tie[k]);
    }
    if (ntie) {
      uint32_t base = 0;
      if (lane == 0) base = atomic_add_agent(mycount, ntie);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int k = 0; k < PRE; ++k) {
        if ((m_tie[k] >> lane) & 1ull) {
          const uint32_t rank = base + (uint32_t)__popcll(m_tie[k] & ((1ull << lane) - 1));
          const int64_t id = (int64_t)(base_ch + k * chs) * 64 + lane;
          st_agent(mylist + rank, ((uint64_t)key_hi[k] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id));
        }
        base += (uint32_t)__popcll(m_tie[k]);
      }
    }
  }
  CSA2_TS(9);
  if (!arrive_last(ctrl->sel_grp, &ctrl->sel_top, gridDim.x)) return;

  // ---- finisher: one workgroup per sequence ----
  CSA2_TS(10);
  if (!all && nblk > 0) {
    uint32_t cnt[CAND_COPIES], off[CAND_COPIES + 1];
    off[0] = 0;
#pragma unroll
    for (int k = 0; k < CAND_COPIES; ++k) {
      cnt[k] = ld_agent(&ctrl->ncand[k]);
      off[k + 1] = off[k] + cnt[k];
    }
    const int c = (int)off[CAND_COPIES];
    if (c <= a.lds_keys) {
      // flat index over the 8 lists, 16 loads in flight per thread (one
      // round trip up to 4,096 candidates)
      constexpr int U = 16;
      for (int j0 = t; j0 < c; j0 += nt * U) {
        uint64_t kv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = min(j0 + u * nt, c - 1);        // clamped: no branch
          int k = 0;
#pragma unroll
          for (int kk = 1; kk < CAND_COPIES; ++kk) k += (j >= (int)off[kk]) ? 1 : 0;
          kv[u] = ld_agent(cands + k * a.cand_stride + (j - (int)off[k]));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * nt;
          if (j < c) s_keys[j] = kv[u];
        }
      }
      __syncthreads();
      CSA2_TS(11);
      // the candidates share the top 10 key bits (the tie digit)
      const uint64_t T = threshold_in_lds<32>(s_keys, c, (int)need, s_hist, s_state, s_wave);
      CSA2_TS(12);
      for (int j = t; j < c; j += nt) {
        uint64_t k = s_keys[j];
        if (k >= T) {
          uint32_t id = 0xFFFFFFFFu - (uint32_t)k;
          atomicOr(&bm[id >> 5], 1u << (id & 31));
        }
      }
    } else {
      // rare: the tie digit holds more keys than LDS; select through global
      // memory one 8-bit digit at a time (same rule, slower)
      uint64_t prefix = 0, pmask = 0;
      int remaining = (int)need;
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int j = t; j < 256; j += nt) s_hist[j] = 0;
        __syncthreads();
        for (int k = 0; k < CAND_COPIES; ++k)
          for (int j = t; j < (int)cnt[k]; j += nt) {
            uint64_t key = ld_agent(cands + k * a.cand_stride + j);
            if ((key & pmask) == prefix) atomicAdd(&s_hist[(uint32_t)(key >> shift) & 255u], 1u);
          }
        __syncthreads();
        if (t == 0) {
          uint32_t acc = 0;
          for (int d = 255; d >= 0; --d) {
            if (acc + s_hist[d] >= (uint32_t)remaining) {
              s_state[0] = prefix | ((uint64_t)d << shift);
              uint32_t rem = (uint32_t)remaining - acc;
              s_state[1] = (uint64_t)rem | ((rem == s_hist[d]) ? (1ull << 63) : 0ull);
              break;
            }
            acc += s_hist[d];
          }
        }
        __syncthreads();
        prefix = s_state[0];
        pmask |= 0xFFull << shift;
        uint64_t st = s_state[1];
        __syncthreads();
        remaining = (int)(uint32_t)st;
        if (st >> 63) break;
      }
      for (int k = 0; k < CAND_COPIES; ++k)
        for (int j = t; j < (int)cnt[k]; j += nt) {
          uint64_t key = ld_agent(cands + k * a.cand_stride + j);
          if (key >= prefix) {
            uint32_t id = 0xFFFFFFFFu - (uint32_t)key;
            atomicOr(&bm[id >> 5], 1u << (id & 31));
          }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  int32_t *first = a.first_out + (int64_t)b * a.R;
  CSA2_TS(13);
  compact_bitmap(bm, a.nwords, first, s_ids, a.R, s_wave);
  __syncthreads();
  CSA2_TS(14);
  if (a.pool_scores) {
    // the chosen list's scores in list order (-1 entries get any value):
    // the attention kernel takes the layer's top-k from them
    constexpr int U = 8;
    const int m = a.R;
    float *ps = a.pool_scores + (int64_t)b * m;
    for (int j0 = t; j0 < m; j0 += nt * U) {
      float sv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t id = s_ids[min(j0 + u * nt, m - 1)];
        sv[u] = scores[id >= 0 ? id : 0];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (j0 + u * nt < m) ps[j0 + u * nt] = sv[u];
    }
  }
  if (a.topk > 0) {
    // top-k inside the pool: keys of the pool members, in pool order
    constexpr int U = 8;
    const int m = a.R;
    for (int j0 = t; j0 < m; j0 += nt * U) {
      float sv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t id = s_ids[min(j0 + u * nt, m - 1)];
        sv[u] = scores[id >= 0 ? id : 0];               // unconditional: no branch
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * nt;
        if (j < m) {
          const int32_t id = s_ids[j];
          s_keys[j] = id >= 0 ? make_key(sv[u], (uint32_t)id) : 0ull;
        }
      }
    }
    __syncthreads();
    select_in_lds(s_keys, s_ids, m, a.topk, a.idx_out + (int64_t)b * a.topk, s_sel, a.topk,
                  s_hist, s_state, s_wave);
  }
  CSA2_TS(15);
  __syncthreads();
  // leave the row clean for the next call (read only by later kernels):
  // bitmap, tie counters, the scan's histogram copies and work counters
  for (int j = t; j < a.nwords; j += nt) bm[j] = 0;
  for (int j = t; j < HIST_COPIES * HIST_BINS; j += nt) gh[j] = 0;
  if (t < CAND_COPIES) ctrl->ncand[t] = 0;
  if (t < SCAN_GROUPS) ctrl->work[t * 32] = 0;
}

// ---- select: classification by every workgroup, ranking by the last ------
//
// The same choice as select_kernel (pool or top-k by (score desc, id asc),
// ids ascending, -1 padded).  Every workgroup (1,024 threads) takes 4,096
// consecutive blocks, finds the threshold digit from the scan's histogram
// and writes the keys of its blocks at or above that digit into its own
// region of a key list (no shared counter); the last workgroup to arrive
// loads the regions into LDS (R plus the digit's blocks: about 5K keys at a
// 1M-position context), takes the threshold inside the digit by radix
// digits, marks the chosen ids in an LDS bitmap and writes every chosen
// block at its rank in ascending id order, its score recovered from the
// key (the order-preserving score bits invert exactly), so the scores are
// read once.  One workgroup cannot stream the whole score row fast enough
// (about 26 GB/s from one compute unit, measured), hence the split.  When
// the regions hold more keys than LDS, the digits are counted from the
// regions in global memory (one pass per digit).
constexpr int SEL2_THREADS = 1024;
constexpr int SEL2_KEYS = 8192;      // region keys ranked in LDS
constexpr int SEL2_WORDS = 8192;     // bitmap words in LDS: up to 262,144 blocks
constexpr int SEL2_U = 4;            // scores per thread
constexpr int SEL2_SPAN = SEL2_THREADS * SEL2_U;       // blocks per workgroup
constexpr int SEL2_MAXG = SEL2_WORDS * 32 / SEL2_SPAN;  // workgroups per sequence
static_assert(SEL2_THREADS == HIST_BINS, "one histogram bin per thread");

// The finisher's LDS key capacity for a bitmap of nwords words: what fits in
// SEL2_LDS_BYTES of dynamic LDS beside the bitmap and its word prefix sums
// (a multiple of 1,024; at least SEL2_KEYS for nwords <= SEL2_WORDS).
constexpr int64_t SEL2_LDS_BYTES = 136 * 1024;
inline int select2_keys(int nwords) {
  const int64_t k = (SEL2_LDS_BYTES - 2 * (int64_t)sizeof(uint32_t) * nwords) / (int64_t)sizeof(uint64_t);
  return (int)(k / 1024 * 1024);
}
static_assert((SEL2_LDS_BYTES - 8 * SEL2_WORDS) / 8 >= SEL2_KEYS, "finisher capacity");

// Dynamic LDS bytes of select2_kernel: the keys, the bitmap and its word
// prefix sums.
inline size_t select2_lds(int nwords) {
  return sizeof(uint64_t) * (size_t)select2_keys(nwords) + 2 * sizeof(uint32_t) * (size_t)nwords;
}

// Digit step of a radix select: s_hist[0..nb) counts the keys under the
// current prefix by their digit at bit lo; the digit holding the
// remaining-th largest key is added to *prefix, *remaining becomes the rank
// inside it and *bucket (if given) that digit's key count.  Returns true
// when that digit's keys are all taken (the threshold is then the prefix
// itself).  All threads call.
__device__ __forceinline__ bool radix_pick(const uint32_t *s_hist, int nb, int lo, uint64_t *prefix,
                                           int *remaining, uint64_t *s_state, uint32_t *s_wave,
                                           uint32_t *bucket = nullptr) {
  const int t = threadIdx.x, nt = blockDim.x;
  const int per = (nb + nt - 1) / nt;
  uint32_t sum = 0;
  for (int j = 0; j < per; ++j) {
    const int bin = nb - 1 - (per * t + j);
    sum += bin >= 0 ? s_hist[bin] : 0u;
  }
  uint32_t total;
  const uint32_t above = block_exclusive_scan(sum, &total, s_wave);
  const uint32_t r = (uint32_t)*remaining;
  if (above < r && r <= above + sum) {
    uint32_t acc = above;
    for (int j = 0; j < per; ++j) {
      const int bin = nb - 1 - (per * t + j);
      const uint32_t c = bin >= 0 ? s_hist[bin] : 0u;
      if (acc + c >= r) {
        s_state[0] = *prefix | ((uint64_t)bin << lo);
        const uint32_t rem = r - acc;
        s_state[1] = (uint64_t)rem | ((uint64_t)c << 32) | ((rem == c) ? (1ull << 63) : 0ull);
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  *prefix = s_state[0];
  const uint64_t st = s_state[1];
  __syncthreads();
  *remaining = (int)(uint32_t)st;
  if (bucket) *bucket = (uint32_t)(st >> 32) & 0x7FFFFFFFu;
  return (st >> 63) != 0;
}

// The key T such that exactly r of the keys get(0..m) that match `prefix`
// on the bits of `pmask` (the bits above hi) are >= T; 11-bit digits from
// bit hi down (keys distinct, 1 <= r <= matching keys).  Once a digit's
// bucket holds at most one key per thread (and no more than s_hist holds as
// 64-bit keys), its keys are gathered and ranked pairwise instead of taking
// further digits.  All threads call.
template <class F>
__device__ __forceinline__ uint64_t radix_select_keys(F get, int m, int r, uint64_t prefix, uint64_t pmask,
                                                      int hi, uint32_t *s_hist, uint64_t *s_state,
                                                      uint32_t *s_wave) {
  const int t = threadIdx.x, nt = blockDim.x;
  constexpr int TIE_CAP = RADIX_BINS / 2;     // 64-bit keys that fit in s_hist
  __shared__ uint32_t s_ntie;
  int remaining = r;
  for (; hi >= 0; hi -= 11) {
    const int lo = hi >= 10 ? hi - 10 : 0;
    const int nb = 1 << (hi - lo + 1);
    for (int j = t; j < nb; j += nt) s_hist[j] = 0;
    __syncthreads();
    constexpr int U = 8;
    for (int j0 = 0; j0 < m; j0 += nt * U) {
      uint64_t kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) kv[u] = get(min(j0 + u * nt + t, m - 1));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (j0 + u * nt + t < m && (kv[u] & pmask) == prefix)
          atomicAdd(&s_hist[(uint32_t)(kv[u] >> lo) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t bucket = 0;
    const bool whole = radix_pick(s_hist, nb, lo, &prefix, &remaining, s_state, s_wave, &bucket);
    pmask |= ((2ull << hi) - 1) & ~((1ull << lo) - 1);
    if (whole || lo == 0) break;
    if ((int)bucket <= min(nt, TIE_CAP)) {
      // the bucket's keys into s_hist (as 64-bit keys), then each one's rank
      uint64_t *s_tie = reinterpret_cast<uint64_t *>(s_hist);
      if (t == 0) s_ntie = 0;
      __syncthreads();
      for (int j0 = 0; j0 < m; j0 += nt * 8) {
        uint64_t kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = get(min(j0 + u * nt + t, m - 1));
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j0 + u * nt + t < m && (kv[u] & pmask) == prefix) {
            const uint32_t k = atomicAdd(&s_ntie, 1u);
            CSA2_CHECK(k < (uint32_t)min(nt, TIE_CAP));
            s_tie[k] = kv[u];
          }
      }
      __syncthreads();
      if (t < (int)bucket) {
        const uint64_t k = s_tie[t];
        uint32_t gt = 0;
        for (uint32_t i2 = 0; i2 < bucket; ++i2) gt += s_tie[i2] > k ? 1u : 0u;
        if (gt == (uint32_t)remaining - 1) s_state[0] = k;   // the remaining-th largest
      }
      __syncthreads();
      prefix = s_state[0];
      __syncthreads();
      break;
    }
  }
  return prefix;
}

// grid (ceil(blocks / SEL2_SPAN) <= SEL2_MAXG, batch), SEL2_THREADS threads;
// nwords <= SEL2_WORDS, R <= SEL2_KEYS; select2_lds(nwords) bytes of
// dynamic LDS.  Regions live in `cands` (region g at entry g * SEL2_SPAN:
// it holds keys of its own blocks only, so it stays inside the sequence's
// cand_stride >= blocks entries); region sizes in the first words of
// `bitmap` (zero at entry, left zero).
__global__ void __launch_bounds__(SEL2_THREADS) select2_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint64_t s_dyn[];
  uint64_t *s_keys = s_dyn;                                            // [lds_keys]
  uint32_t *s_bm = reinterpret_cast<uint32_t *>(s_dyn + a.lds_keys);  // [nwords]
  uint32_t *s_wpre = s_bm + a.nwords;                                  // [nwords]
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[TOPK_HIST_BINS];   // also 64-bit keys (radix_select_keys)
  __shared__ uint32_t s_off[SEL2_MAXG + 1];
  __shared__ uint64_t s_state[2];
  __shared__ uint32_t s_wave[16];
  __shared__ uint32_t s_cnt;
  const int b = blockIdx.y, g = wg_x(), G = gridDim.x;
  const int t = threadIdx.x, nt = SEL2_THREADS;
  Ctrl *ctrl = a.ctrl + b;
  const float *scores = a.scores + (int64_t)b * a.score_stride;
  uint32_t *gh = a.hist + (int64_t)b * HIST_COPIES * HIST_BINS;
  uint64_t *keys_g = a.cands + (int64_t)b * CAND_COPIES * a.cand_stride;
  uint32_t *counts = a.bitmap + (int64_t)b * a.nwords;
  const uint32_t R = (uint32_t)a.R;
  CSA2_TS(8);
  // one batch of requests: this thread's histogram bin (8 copies), its
  // scores, the length
  const int bin = HIST_BINS - 1 - t;
  uint32_t hv[HIST_COPIES];
#pragma unroll
  for (int k = 0; k < HIST_COPIES; ++k) hv[k] = gh[k * HIST_BINS + bin];
  const int id0 = g * SEL2_SPAN + t;
  float sv[SEL2_U];
#pragma unroll
  for (int u = 0; u < SEL2_U; ++u) sv[u] = scores[min(id0 + u * nt, (int)a.score_stride - 1)];
  const int64_t n = clamp_len(a.seq_len[b], a.limit);
  const int nblk = (int)((n + BLOCK - 1) / BLOCK);
  if (t == 0) { s_cnt = 0; s_state[0] = 0; }
  const bool all = R >= (uint32_t)nblk;
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < HIST_COPIES; ++k) c += hv[k];
  uint32_t total;
  const uint32_t above = block_exclusive_scan(c, &total, s_wave);    // barriers: s_cnt is clear
  if (!all && above < R && R <= above + c) s_state[0] = ((uint64_t)bin << 32) | (uint64_t)(R - above);
  __syncthreads();
  const uint32_t thr = (uint32_t)(s_state[0] >> 32), need = (uint32_t)s_state[0];
  // keys of this workgroup's blocks at or above the threshold digit (every
  // block when R >= blocks)
  uint64_t *region = keys_g + (int64_t)g * SEL2_SPAN;
#pragma unroll
  for (int u = 0; u < SEL2_U; ++u) {
    const int id = id0 + u * nt;
    const uint32_t kh = ord_key(sv[u]);
    if (id < nblk && (all || (kh >> HIST_SHIFT) >= thr)) {
      const uint32_t pos = atomicAdd(&s_cnt, 1u);
      st_agent(region + pos, ((uint64_t)kh << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id));
    }
  }
  __syncthreads();
  if (t == 0) st_agent(counts + g, s_cnt);
  CSA2_TS(9);
  if (!arrive_last(ctrl->sel_grp, &ctrl->sel_top, G)) return;

  // ---- the last workgroup: rank the regions' keys ----
  CSA2_TS(10);
  // One batch of requests: every region's key count and, speculatively, its
  // first SU * tpr entries (tpr threads per region); entries past a count
  // are dropped, and a longer region's remaining entries are read after.
  int lg = 0;
  while ((1 << lg) < G) ++lg;                  // G <= SEL2_MAXG
  const int tpr = SEL2_THREADS >> lg;          // threads per region
  const int rg = t / tpr, rl = t - rg * tpr;
  const int64_t rbase = (int64_t)rg * SEL2_SPAN;
  const int64_t rlim = rg < G ? min((int64_t)SEL2_SPAN, a.cand_stride - rbase) : 1;   // >= 1: inside the row
  constexpr int SU = 8;
  const uint32_t rc = (rg < G && rl == 0) ? ld_agent(counts + rg) : 0u;
  uint64_t kv[SU];
#pragma unroll
  for (int u = 0; u < SU; ++u)
    kv[u] = rg < G ? ld_agent(keys_g + rbase + min((int64_t)(rl + u * tpr), rlim - 1)) : 0ull;
  if (rg < G && rl == 0) { s_off[rg] = rc; counts[rg] = 0; }
  for (int j = t; j < a.nwords; j += nt) s_bm[j] = 0;
  __syncthreads();
  if (t < 64) {                                // region offsets: exclusive prefix of the counts
    const uint32_t c = t < G ? s_off[t] : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (t < G) s_off[t] = incl - c;
    if (t == 63) s_off[G] = incl;
  }
  __syncthreads();
  const int cap = a.lds_keys;
  const uint32_t E = s_off[G];
  // entry j of the concatenated regions
  auto key_at = [&](int j) -> uint64_t {
    int lo = 0, hi = G - 1;                    // largest k with s_off[k] <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= (uint32_t)j) lo = mid; else hi = mid - 1;
    }
    return ld_agent(keys_g + (int64_t)lo * SEL2_SPAN + (j - (int)s_off[lo]));
  };
  const int m = (int)E;
  const bool in_lds = m <= cap;
  const bool fast = in_lds && m <= 16 * SEL2_THREADS;   // within the linear threshold's registers
  if (in_lds && rg < G) {
    const uint32_t off = s_off[rg], cnt = s_off[rg + 1] - off;
#pragma unroll
    for (int u = 0; u < SU; ++u)
      if ((uint32_t)(rl + u * tpr) < cnt) s_keys[off + rl + u * tpr] = kv[u];
    for (uint32_t j = (uint32_t)(SU * tpr + rl); j < cnt; j += (uint32_t)tpr)
      s_keys[off + j] = ld_agent(keys_g + rbase + j);
  }
  __syncthreads();
  auto get_lds = [&](int j) -> uint64_t { return s_keys[j]; };
  CSA2_TS(11);
  // threshold: need-th largest key inside the digit (every entry when R >= blocks)
  uint64_t T = 1ull;                           // keys are never 0
  if (!all && need > 0 && (uint32_t)m > R) {
    const uint64_t prefix = (uint64_t)thr << (32 + HIST_SHIFT);
    const uint64_t pmask = ~((1ull << (32 + HIST_SHIFT)) - 1);
    // one digit of the radix select inside the threshold digit (its keys
    // alone) leaves a bucket small enough to rank; the linear threshold
    // over every key measured no faster here (8,700-10,200 cycles at 1M)
    T = in_lds ? radix_select_keys(get_lds, m, (int)need, prefix, pmask, 31 + HIST_SHIFT, s_hist, s_state, s_wave)
               : radix_select_keys(key_at, m, (int)need, prefix, pmask, 31 + HIST_SHIFT, s_hist, s_state, s_wave);
  }
  CSA2_TS(12);
  // chosen ids (keys >= Tc) -> ranks in ascending id order -> out[rank]
  auto emit = [&](uint64_t Tc, int32_t *out, float *out_scores, int len) {
    for (int j0 = 0; j0 < m; j0 += nt) {
      const int j = j0 + t;
      if (j < m) {
        const uint64_t k = in_lds ? s_keys[j] : key_at(j);
        if (k >= Tc) {
          const uint32_t id = 0xFFFFFFFFu - (uint32_t)k;
          atomicOr(&s_bm[id >> 5], 1u << (id & 31));
        }
      }
    }
    __syncthreads();
    const int per = (a.nwords + nt - 1) / nt;
    const int w0 = min(a.nwords, t * per), w1 = min(a.nwords, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(s_bm[w]);
    uint32_t tot;
    uint32_t off = block_exclusive_scan(cnt, &tot, s_wave);
    CSA2_CHECK(tot <= (uint32_t)len);   // the threshold admits at most len keys
    for (int w = w0; w < w1; ++w) {
      s_wpre[w] = off;
      off += __popc(s_bm[w]);
    }
    __syncthreads();
    for (int j0 = 0; j0 < m; j0 += nt) {
      const int j = j0 + t;
      if (j < m) {
        const uint64_t k = in_lds ? s_keys[j] : key_at(j);
        if (k >= Tc) {
          const uint32_t id = 0xFFFFFFFFu - (uint32_t)k;
          const uint32_t rank = s_wpre[id >> 5] + __popc(s_bm[id >> 5] & ((1u << (id & 31)) - 1u));
          if (rank < (uint32_t)len) {
            out[rank] = (int32_t)id;
            if (out_scores) out_scores[rank] = unord_key((uint32_t)(k >> 32));
          }
        }
      }
    }
    for (int j = (int)tot + t; j < len; j += nt) out[j] = -1;
    __syncthreads();
    for (int j = t; j < a.nwords; j += nt) s_bm[j] = 0;
    __syncthreads();
  };
  const uint32_t chosen = min(R, (uint32_t)m);
  emit(T, a.first_out + (int64_t)b * R, a.pool_scores ? a.pool_scores + (int64_t)b * R : nullptr, (int)R);
  CSA2_TS(13);
  if (a.topk > 0) {
    // the top-k of the chosen list is the top-k of every entry
    uint64_t T2 = T;
    if ((uint32_t)a.topk < chosen)
      // no digit is known here: linear bins over the keys' range (11,000
      // cycles at 1M against 34,500 for a radix select from the top bit)
      T2 = fast ? threshold_in_lds<16>(s_keys, m, a.topk, s_hist, s_state, s_wave)
           : in_lds ? radix_select_keys(get_lds, m, a.topk, 0ull, 0ull, 63, s_hist, s_state, s_wave)
                    : radix_select_keys(key_at, m, a.topk, 0ull, 0ull, 63, s_hist, s_state, s_wave);
    emit(T2, a.idx_out + (int64_t)b * a.topk, nullptr, a.topk);
  }
  CSA2_TS(14);
  // leave the row clean for the next call: the scan's histogram copies and
  // work counters (the region sizes were cleared above)
  for (int j = t; j < HIST_COPIES * HIST_BINS; j += nt) gh[j] = 0;
  if (t < SCAN_GROUPS) ctrl->work[t * 32] = 0;
}

// ---- rescoring of a candidate list (pool) + top-k --------------------------

struct RescoreArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const int64_t *seq_len;
  int64_t capacity;
  int64_t limit;
  const float *q;
  int32_t heads;
  const int32_t *cand;      // [batch][n_cand]
  int32_t n_cand;
  float *scores;            // [batch][score_stride]
  int64_t score_stride;
  Ctrl *ctrl;
  int32_t topk;
  int32_t *idx_out;         // [batch][topk]; NULL = scores only
};

// Selection keys of a scored candidate list into LDS (all threads call):
// s_ids[j] = cand[j]; s_keys[j] = key of (scores[j], cand[j]), 0 for an id
// outside [0, nblk).  AGENT: other workgroups of the running kernel wrote
// the scores.
template <bool AGENT>
__device__ __forceinline__ void cand_keys_to_lds(const int32_t *cand, const float *scores, int m, int64_t nblk,
                                                 uint64_t *s_keys, int32_t *s_ids) {
  const int t = threadIdx.x, nt = blockDim.x;
  constexpr int U = 8;
  for (int j0 = t; j0 < m; j0 += nt * U) {
    int32_t idv[U];
    float sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = min(j0 + u * nt, m - 1);         // clamped: no branch
      idv[u] = cand[jj];
      sv[u] = AGENT ? ld_agent(scores + jj) : scores[jj];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j0 + u * nt;
      if (jj < m) {
        const bool ok = idv[u] >= 0 && idv[u] < nblk;
        s_ids[jj] = idv[u];
        s_keys[jj] = ok ? make_key(sv[u], (uint32_t)idv[u]) : 0ull;
      }
    }
  }
  __syncthreads();
}

template <bool SELECT>
__global__ void __launch_bounds__(SCAN_THREADS) rescore_kernel(RescoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint64_t s_keys[];
  __shared__ float s_qbar[D];
  __shared__ int32_t s_ids[SELECT ? LDS_KEYS : 1];
  __shared__ int32_t s_sel[SELECT ? CSA2_TOPK_MAX + SEL_PAD : 1];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[SELECT ? TOPK_HIST_BINS : 1];
  __shared__ uint64_t s_state[2];
  __shared__ uint32_t s_wave[16];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane >> 4, i = lane & 15;
  const int64_t cap_blocks = a.capacity / BLOCK;   // loads stay inside the cache
  const uint8_t *codes = a.codes + (int64_t)b * a.capacity * CODE_BYTES;
  const uint8_t *scales = a.scales + (int64_t)b * a.capacity * SCALE_BYTES;
  const int32_t *cand = a.cand + (int64_t)b * a.n_cand;
  float *scores = a.scores + (int64_t)b * a.score_stride;
  const int iters = (a.n_cand + BLOCKS_PER_ITER - 1) / BLOCKS_PER_ITER;
  // first group's candidate ids and rows are requested before the query sum
  int it = wg_x();
  int j = it * BLOCKS_PER_ITER + wv * 4 + slot;
  int32_t blk = cand[min(j, a.n_cand - 1)];          // unconditional: no branch
  if (!(it < iters && j < a.n_cand)) blk = -1;
  BlockRows cur;
  {
    // unconditional (an id outside the cache reads block 0, dropped later),
    // so the rows and the query loads below form one batch
    const int64_t lb = (blk >= 0 && blk < cap_blocks) ? blk : 0;
    load_block(cur, codes + lb * BLOCK * CODE_BYTES, scales + lb * BLOCK * SCALE_BYTES, i);
  }
  CSA2_TS(0);
  compute_qbar<64>(a.q, a.heads, b, s_qbar);
  // the length only masks: read after the first rows and the query sum
  const int64_t n = clamp_len(a.seq_len[b], a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;
  CSA2_TS(1);
  const float *qb = s_qbar + 32 * i;
  for (; it < iters; it += gridDim.x) {
    if (j < a.n_cand) {
      if (blk >= 0 && blk < nblk) {
        const int cnt = (int)min((int64_t)BLOCK, n - (int64_t)blk * BLOCK);
        float s = block_score(cur, cnt, qb);
        if (i == 0) { if (SELECT) st_agent(scores + j, s); else scores[j] = s; }
      } else if (i == 0) {
        if (SELECT) st_agent(scores + j, -__builtin_huge_valf()); else scores[j] = -__builtin_huge_valf();
        if (blk >= nblk) raise_flag(FLAG_BAD_INDEX);
      }
    }
    const int it_next = it + gridDim.x;
    j = it_next * BLOCKS_PER_ITER + wv * 4 + slot;
    blk = cand[min(j, a.n_cand - 1)];
    if (!(it_next < iters && j < a.n_cand)) blk = -1;
    if (it_next < iters) {
      const int64_t lb = (blk >= 0 && blk < cap_blocks) ? blk : 0;
      load_block(cur, codes + lb * BLOCK * CODE_BYTES, scales + lb * BLOCK * SCALE_BYTES, i);
    }
  }
  CSA2_TS(2);
  if (!SELECT) return;
  Ctrl *ctrl = a.ctrl + b;
  if (!arrive_last(ctrl->sel_grp, &ctrl->sel_top, gridDim.x)) return;
  CSA2_TS(3);
  cand_keys_to_lds<true>(cand, scores, a.n_cand, nblk, s_keys, s_ids);
  CSA2_TS(4);
  select_in_lds(s_keys, s_ids, a.n_cand, a.topk, a.idx_out + (int64_t)b * a.topk, s_sel, a.topk,
                s_hist, s_state, s_wave);
  CSA2_TS(5);
}

// Pool rescoring without selection (the decode step's later layers): the
// full scan's 32-lane layout (lane j owns scale group j), 8 waves of two
// blocks, so a lane dequantises 8 x 16 values per block instead of the
// 16-lane layout's 8 x 32.  Thread t forms Qbar channel t (heads in order;
// 64 head requests per batch).  Same arithmetic, same order.
constexpr int RESCORE32_THREADS = 512;
constexpr int RESCORE32_BLOCKS = RESCORE32_THREADS / 32;   // blocks per round
__global__ void __launch_bounds__(RESCORE32_THREADS) rescore32_kernel(RescoreArgs a) {
  __shared__ __attribute__((aligned(16))) float s_qbar[D];   // qbar32_index layout
  const int b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int half = lane >> 5, j = lane & 31;
  const int64_t cap_blocks = a.capacity / BLOCK;   // loads stay inside the cache
  const uint8_t *codes = a.codes + (int64_t)b * a.capacity * CODE_BYTES;
  const uint8_t *scales = a.scales + (int64_t)b * a.capacity * SCALE_BYTES;
  const int32_t *cand = a.cand + (int64_t)b * a.n_cand;
  float *scores = a.scores + (int64_t)b * a.score_stride;
  const int iters = (a.n_cand + RESCORE32_BLOCKS - 1) / RESCORE32_BLOCKS;
  CSA2_CHECK(a.n_cand <= a.score_stride);
  // rounds it, it + grid, ...: the ids of the first two rounds and the rows
  // of the first are requested before the query sum; afterwards each round's
  // rows are requested as the previous round's rows are consumed and the ids
  // run one round further ahead (a batch gives a workgroup many rounds)
  auto id_of = [&](int r, int &jr) {
    jr = r * RESCORE32_BLOCKS + 2 * wv + half;
    int32_t v = cand[min(jr, a.n_cand - 1)];           // unconditional: no branch
    if (!(r < iters && jr < a.n_cand)) v = -1;
    return v;
  };
  auto rows_of = [&](int32_t blkv) {
    return (blkv >= 0 && blkv < cap_blocks) ? (int64_t)blkv : (int64_t)0;   // block 0 always exists
  };
  int it = wg_x();
  int jj, jj1;
  int32_t blk = id_of(it, jj);
  int32_t blk1 = id_of(it + (int)gridDim.x, jj1);
  BlockRows32 cur;
  {
    const int64_t lb = rows_of(blk);
    load_block32(cur, codes + lb * BLOCK * CODE_BYTES, scales + lb * BLOCK * SCALE_BYTES, j);
  }
  CSA2_TS(0);
  {
    const float *qp = a.q + (int64_t)b * a.heads * D + t;
    float acc = 0.f;
    constexpr int HB = 64;
    for (int h0 = 0; h0 < a.heads; h0 += HB) {
      float v[HB];
#pragma unroll
      for (int u = 0; u < HB; ++u) v[u] = qp[(int64_t)min(h0 + u, a.heads - 1) * D];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < HB; ++u) {
        const int h = h0 + u;
        if (h == 0) acc = v[u];
        else if (h < a.heads) acc = acc + v[u];
      }
    }
    if (!__builtin_isfinite(acc)) raise_flag(FLAG_NONFINITE_Q);
    s_qbar[qbar32_index(t)] = acc;
  }
  __syncthreads();
  // the length only masks: read after the first rows and the query sum
  const int64_t n = clamp_len(a.seq_len[b], a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;
  CSA2_TS(1);
  const float *qb = s_qbar + qbar32_base(j);
  for (; it < iters; it += gridDim.x) {
    const bool more = it + (int)gridDim.x < iters;              // uniform
    const int64_t nb = rows_of(blk1);
    const bool ok = blk >= 0 && blk < nblk;
    const int cnt = ok ? (int)min((int64_t)BLOCK, n - (int64_t)blk * BLOCK) : 1;
    float sc;
    if (more)
      sc = block_score32<true>(cur, cnt, qb, codes + nb * BLOCK * CODE_BYTES, scales + nb * BLOCK * SCALE_BYTES, j);
    else
      sc = block_score32<false>(cur, cnt, qb, nullptr, nullptr, j);
    if (jj < a.n_cand && j == 0) {
      if (ok) {
        scores[jj] = sc;
      } else {
        scores[jj] = -__builtin_huge_valf();
        if (blk >= nblk) raise_flag(FLAG_BAD_INDEX);
      }
    }
    int jj2;
    const int32_t blk2 = id_of(it + 2 * (int)gridDim.x, jj2);
    blk = blk1; jj = jj1;
    blk1 = blk2; jj1 = jj2;
  }
  CSA2_TS(2);
}

// Reuse: idx_out = prior (grid-stride copy).
__global__ void __launch_bounds__(256) copy_idx_kernel(const int32_t *__restrict__ src,
                                                       int32_t *__restrict__ dst, int64_t n) {
  for (int64_t j = (int64_t)wg_x() * blockDim.x + threadIdx.x; j < n;
       j += (int64_t)gridDim.x * blockDim.x)
    dst[j] = src[j];
}

// Explicit instantiations used by the host layer.
template __global__ void scan_kernel<true>(ScanArgs);
template __global__ void scan_kernel<false>(ScanArgs);
template __global__ void rescore_kernel<true>(RescoreArgs);

}  // namespace csa2
