// FP4 quantiser / packer of the global-KV cache (gfx950).
//
// One position is the 512-channel latent stored as E2M1 codes with one E4M3
// scale per 16 channels (ailily.cc "890 bytes per token", section 二; the
// representable maximum 448 x 6 = 2688 of section 三 leaves no room for a
// second, per-tensor scale).  Rows sit at a fixed stride so a kernel finds
// a position from its index (yomxxx.com long-form post, section 五).
//
// Rounding (the pages give none): scale = E4M3 nearest to amax/6, ties to
// the even code, saturating at 448; code = E2M1 nearest to |x|/scale, ties
// to even, saturating at 6; the sign bit is kept (-0 -> 0x8).  Both
// decisions are made exactly by comparing against exact products:
//   amax <> 6 * (midpoint of two E4M3 values)   (<= 8 significant bits)
//   |x|  <> scale * (midpoint of two E2M1 values) (<= 7 significant bits)
// so no division is ever rounded.
//
// Both the bulk row quantiser and the decode-step append run the same
// per-group routine (quantize_group): one lane per 16-channel group reads
// the group's 64 bytes, finds its scale once and packs its 8 code bytes.
#include "common.hpp"

namespace csa2 {

__device__ uint32_t g_flags = 0;
#ifdef CSA2_CHECKED
__device__ uint32_t g_wg_salt = 0;   // workgroup-order salt of the checked build
#endif

// E4M3 value of a non-negative code 0..126.
__device__ __forceinline__ float e4m3_pos(uint32_t c) { return e4m3_to_f32(c); }

// Exact E4M3 code of RNE(amax / 6), saturating.  amax >= 0, finite.
__device__ __forceinline__ uint32_t scale_code(float amax) {
  // 6 * midpoint(416, 448) = 2592: anything at or above rounds to 448 (0x7E, even)
  if (amax >= 2592.0f) return 0x7Eu;
  // estimate from y ~ amax/6 (at most one code off), then fix exactly
  float y = amax * (1.0f / 6.0f);
  uint32_t c;
  if (y < 0.015625f) {
    c = (uint32_t)__builtin_rintf(y * 512.0f);          // subnormal codes 0..8
  } else {
    uint32_t u = __float_as_uint(y);
    int e = (int)(u >> 23) - 127;                        // -6 .. 8
    c = (uint32_t)(((e + 7) << 3) | ((u >> 20) & 7u));
    c = c > 126u ? 126u : c;
  }
  // threshold between codes k and k+1, times 6: 3 * (v_k + v_{k+1}), exact
  while (c < 126u) {
    float t = 3.0f * (e4m3_pos(c) + e4m3_pos(c + 1));
    if (amax > t || (amax == t && ((c + 1) & 1u) == 0)) ++c; else break;
  }
  while (c > 0u) {
    float t = 3.0f * (e4m3_pos(c - 1) + e4m3_pos(c));
    if (amax < t || (amax == t && (c & 1u))) --c; else break;
  }
  return c;
}

// E2M1 magnitude code of RNE(a / s) from t[k] = s * midpoint_k, with the
// tie rule folded into the comparisons: a tie at an odd midpoint (0.75,
// 1.75, 3.5) goes up to the even code (>=), at an even one (0.25, 1.25,
// 2.5, 5) it stays down (>).  Same result as mag_code.
__device__ __forceinline__ uint32_t mag_code_ties(float a, const float *t) {
  return (uint32_t)(a > t[0]) + (uint32_t)(a >= t[1]) + (uint32_t)(a > t[2]) + (uint32_t)(a >= t[3]) +
         (uint32_t)(a > t[4]) + (uint32_t)(a >= t[5]) + (uint32_t)(a > t[6]);
}

// One 16-channel group f[0..15] -> its 8 code bytes (w0: channels 0..7,
// w1: channels 8..15, channel 2j in the low nibble of byte j) and its scale
// byte.  Returns false for a group holding NaN or Inf, which is written as
// zero codes and scale 0.
__device__ __forceinline__ bool quantize_group(const float *f, uint32_t &w0, uint32_t &w1, uint32_t &sc) {
  // |x| as bits: finite magnitudes order like their bit patterns, and any
  // infinity or NaN is at least 0x7f800000
  uint32_t mb = 0;
#pragma unroll
  for (int e = 0; e < 16; e += 2)
    mb = max(mb, max(__float_as_uint(f[e]) & 0x7fffffffu, __float_as_uint(f[e + 1]) & 0x7fffffffu));
  w0 = w1 = sc = 0;
  if (mb >= 0x7f800000u) return false;
  sc = scale_code(__uint_as_float(mb));
  const float sv = e4m3_pos(sc);
  uint32_t nib[16];
  if (sv == 0.0f) {
    // magnitudes all round to 0; keep the signs
#pragma unroll
    for (int e = 0; e < 16; ++e) nib[e] = (__float_as_uint(f[e]) >> 31) << 3;
  } else {
    const float t[7] = {sv * 0.25f, sv * 0.75f, sv * 1.25f, sv * 1.75f, sv * 2.5f, sv * 3.5f, sv * 5.0f};
    // one value's comparisons at a time: hoisting all 112 of them ahead of
    // their sums runs out of scalar mask registers
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      nib[e] = mag_code_ties(fabsf(f[e]), t) | ((__float_as_uint(f[e]) >> 31) << 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    w0 |= nib[e] << (4 * e);
    w1 |= nib[8 + e] << (4 * e);
  }
  return true;
}

// rows x 512 floats -> codes/scales rows dst_row[r] (or r), one lane per
// 16-channel group: the lane reads the group's 64 bytes, finds the group's
// scale once (no cross-lane exchange) and writes its 8 code bytes with one
// store.  Each thread takes GU groups per round, a grid stride apart, and
// requests all of them (and their destination rows) before quantising any.
constexpr int GU = 1;
__global__ void __launch_bounds__(256) quantize_rows_kernel(
    const float *__restrict__ x, int64_t rows, const int64_t *__restrict__ dst_row,
    int64_t dst_rows, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  const int64_t total = rows * NGROUPS;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const float4 *x4 = reinterpret_cast<const float4 *>(x);
  for (int64_t g0 = (int64_t)wg_x() * blockDim.x + threadIdx.x; g0 < total; g0 += stride * GU) {
    float4 v[GU][4];
    int64_t d[GU];
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int64_t gi = min(g0 + u * stride, total - 1);     // clamped: no branch
#pragma unroll
      for (int j = 0; j < 4; ++j) v[u][j] = x4[gi * 4 + j];
      d[u] = dst_row ? dst_row[gi / NGROUPS] : gi / NGROUPS;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int64_t gi = g0 + u * stride;
      if (gi >= total) break;
      const int grp = (int)(gi % NGROUPS);
      if (d[u] < 0 || d[u] >= dst_rows) {
        if (grp == 0) raise_flag(FLAG_CAPACITY);
        continue;
      }
      const float *f = reinterpret_cast<const float *>(v[u]);
      uint32_t w0, w1, sc;
      if (!quantize_group(f, w0, w1, sc)) raise_flag(FLAG_NONFINITE_KV);   // written as zeros
      *reinterpret_cast<uint2 *>(codes + d[u] * CODE_BYTES + 8 * grp) = uint2{w0, w1};
      scales[d[u] * SCALE_BYTES + grp] = (uint8_t)sc;
    }
  }
}

// ---- FP8 rows of the sliding-window (SWA) cache -------------------------
//
// The local branch's KV stays FP8 because it is more sensitive to
// quantisation (rebasdaily.com "DeepSeek-V4.1-Flash KV compression",
// section "same notes, many layers").  Reading (the pages give no layout):
// E4M3FN codes with one float32 scale per row, s = fl(amax / 448), code =
// E4M3 nearest to fl(x / s) (ties to even; |x / s| <= 448 by construction),
// sign kept; s == 0 leaves only the signs.  Both divisions are IEEE
// (correctly rounded), the E4M3 rounding is the hardware's RNE converter.

// Codes of 4 values (bytes in channel order) for scale s.
__device__ __forceinline__ uint32_t fp8_encode4(float4 v, float s) {
  if (s > 0.0f) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(v.x, s), __fdiv_rn(v.y, s), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(v.z, s), __fdiv_rn(v.w, s), w, true);
    return (uint32_t)w;
  }
  return ((__float_as_uint(v.x) >> 31) << 7) | ((__float_as_uint(v.y) >> 31) << 15) |
         ((__float_as_uint(v.z) >> 31) << 23) | ((__float_as_uint(v.w) >> 31) << 31);
}

__device__ __forceinline__ bool finite4(float4 v) {
  return __builtin_isfinite(v.x) && __builtin_isfinite(v.y) && __builtin_isfinite(v.z) &&
         __builtin_isfinite(v.w);
}

__device__ __forceinline__ uint32_t amax_bits4(float4 v) {
  // non-negative floats order like their bit patterns
  return max(max(__float_as_uint(fabsf(v.x)), __float_as_uint(fabsf(v.y))),
             max(__float_as_uint(fabsf(v.z)), __float_as_uint(fabsf(v.w))));
}

// The largest magnitude the attention can stage as fp16, and the flag bit a
// larger SWA row raises.
constexpr float SWA_FP16_MAX = 65504.0f;
constexpr uint32_t FLAG_SWA_RANGE = 16;

// rows x 512 floats -> codes [dst][512], scales [dst]: one wave per row,
// 8 channels (two float4) per lane; rows grid-strided.
__global__ void __launch_bounds__(256) fp8_quantize_kernel(
    const float *__restrict__ x, int64_t rows, const int64_t *__restrict__ dst_row,
    int64_t dst_rows, uint8_t *__restrict__ codes, float *__restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t r = (int64_t)wg_x() * (blockDim.x >> 6) + (threadIdx.x >> 6); r < rows; r += waves) {
    const float4 *src = reinterpret_cast<const float4 *>(x + r * D) + 2 * lane;
    const float4 v0 = src[0], v1 = src[1];
    const int64_t d = dst_row ? dst_row[r] : r;
    const bool bad = __builtin_amdgcn_ballot_w64(!(finite4(v0) && finite4(v1))) != 0;
    const float amax = __uint_as_float(wave_umax(max(amax_bits4(v0), amax_bits4(v1))));
    if (d < 0 || d >= dst_rows) {
      if (lane == 0) raise_flag(FLAG_CAPACITY);
      continue;
    }
    float s = bad ? 0.0f : __fdiv_rn(amax, 448.0f);
    uint32_t c0 = 0, c1 = 0;
    if (!bad) { c0 = fp8_encode4(v0, s); c1 = fp8_encode4(v1, s); }
    reinterpret_cast<uint2 *>(codes + d * D)[lane] = uint2{c0, c1};
    if (lane == 0) {
      scales[d] = s;
      if (bad) raise_flag(FLAG_NONFINITE_KV);
      else if (amax > SWA_FP16_MAX) raise_flag(FLAG_SWA_RANGE);
    }
  }
}

// Caches appended in one launch (decode step: one row per sequence each):
// the FP4 global caches of the Full layers, then the FP8 SWA rings.
struct AppendArgs {
  uint8_t *codes[16];
  uint8_t *scales[16];
  int64_t *seq_len[16];
  int64_t capacity[16];
};
constexpr int MAX_SWA_RINGS = 64;
struct SwaRings {
  uint8_t *codes[MAX_SWA_RINGS];     // [batch][slots][512]
  float *scales[MAX_SWA_RINGS];      // [batch][slots]
  int64_t *seq_len[MAX_SWA_RINGS];   // [batch]
  const float *rows[MAX_SWA_RINGS];  // [batch][512]
  int32_t slots[MAX_SWA_RINGS];      // ring positions
};

// The indexer's query sum of one layer, computed in the same launch as the
// appends (it only reads the query): Qbar[b] = heads added in order.
constexpr int QBAR_SLICES = D / 128;   // query-sum workgroups per sequence in append_kernel

struct QbarJob {
  const float *q;           // [batch][heads][512]; NULL = none
  int32_t heads;
  float *qbar;              // [batch][512]
};

// grid (batch, n_caches + n_rings [+ QBAR_SLICES]), 128 threads.  y <
// n_caches: x[y][b][512] -> position seq_len[b] of cache y.  Then ring y -
// n_caches: rows[b] -> position seq_len[b], slot seq_len[b] % slots.  The
// last QBAR_SLICES rows of workgroups (when qj.q is set) sum the query heads
// of sequence b, 128 channels each.
__global__ void __launch_bounds__(128) append_kernel(AppendArgs a, SwaRings r, const float *__restrict__ x,
                                                     int32_t batch, int32_t n_caches, int32_t n_rings,
                                                     QbarJob qj) {
  const int b = wg_x(), c = blockIdx.y;
  const int q = threadIdx.x;
  if (c >= n_caches + n_rings) {
    // query sum: slice k of QBAR_SLICES owns channels 128k..128k+127, one
    // per thread, heads added in order; the heads of a batch of 64 are
    // requested together (one memory round trip for 64 heads)
    const int ch = 128 * (c - n_caches - n_rings) + q;
    constexpr int HB = 64;
    const float *qp = qj.q + (int64_t)b * qj.heads * D + ch;
    float acc = 0.f;
    for (int h0 = 0; h0 < qj.heads; h0 += HB) {
      float v[HB];
#pragma unroll
      for (int j = 0; j < HB; ++j) v[j] = qp[(int64_t)min(h0 + j, qj.heads - 1) * D];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int h = h0 + j;
        if (h == 0) acc = v[j];
        else if (h < qj.heads) acc = acc + v[j];
      }
    }
    if (!__builtin_isfinite(acc)) raise_flag(FLAG_NONFINITE_Q);
    qj.qbar[(int64_t)b * D + ch] = acc;
    return;
  }
  if (c >= n_caches) {
    __shared__ uint32_t s_red[2];
    const int i = c - n_caches;
    int64_t *len = r.seq_len[i] + b;
    const int64_t pos = *len;
    const float4 v = reinterpret_cast<const float4 *>(r.rows[i] + (int64_t)b * D)[q];
    const bool bad_w = __builtin_amdgcn_ballot_w64(!finite4(v)) != 0;
    const uint32_t am = wave_umax(amax_bits4(v));
    if ((q & 63) == 0) s_red[q >> 6] = am | (bad_w ? 0x80000000u : 0u);   // |x| bits have no sign
    __syncthreads();
    const uint32_t both = max(s_red[0] & 0x7fffffffu, s_red[1] & 0x7fffffffu);
    const bool bad = ((s_red[0] | s_red[1]) & 0x80000000u) != 0;
    if (pos < 0) {
      if (q == 0) raise_flag(FLAG_CAPACITY);
      return;
    }
    const float amax = __uint_as_float(both);
    const float s = bad ? 0.0f : __fdiv_rn(amax, 448.0f);
    const int64_t row = (int64_t)b * r.slots[i] + pos % r.slots[i];
    reinterpret_cast<uint32_t *>(r.codes[i] + row * D)[q] = bad ? 0u : fp8_encode4(v, s);
    if (q == 0) {
      r.scales[i][row] = s;
      if (bad) raise_flag(FLAG_NONFINITE_KV);
      else if (amax > SWA_FP16_MAX) raise_flag(FLAG_SWA_RANGE);
    }
    __syncthreads();
    if (q == 0) *len = pos + 1;
    return;
  }
  // FP4 cache row: lane g < 32 quantises group g with the row quantiser's
  // routine (the other lanes only wait for the length update)
  int64_t *len = a.seq_len[c] + b;
  const int64_t pos = *len;
  uint32_t w0 = 0, w1 = 0, sb = 0;
  bool ok = true;
  if (q < NGROUPS) {
    const float4 *src = reinterpret_cast<const float4 *>(x + ((int64_t)c * batch + b) * D) + 4 * q;
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = src[j];
    ok = quantize_group(reinterpret_cast<const float *>(v), w0, w1, sb);
  }
  if (pos < 0 || pos >= a.capacity[c]) {
    if (q == 0) raise_flag(FLAG_CAPACITY);
    return;
  }
  if (q < NGROUPS) {
    if (!ok) raise_flag(FLAG_NONFINITE_KV);
    const int64_t row = (int64_t)b * a.capacity[c] + pos;
    *reinterpret_cast<uint2 *>(a.codes[c] + row * CODE_BYTES + 8 * q) = uint2{w0, w1};
    a.scales[c][row * SCALE_BYTES + q] = (uint8_t)sb;
  }
  __syncthreads();
  if (q == 0) *len = pos + 1;
}

// Zero fill (graph-safe replacement for memset).
__global__ void __launch_bounds__(256) zero_kernel(uint32_t *__restrict__ p, int64_t words) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)wg_x() * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0;
}

}  // namespace csa2
