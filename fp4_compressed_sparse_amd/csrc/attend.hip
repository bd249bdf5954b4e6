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
//  * A workgroup (4 waves) takes a range of "stages" of SP gathered
//    positions.  Per stage the 256 threads load the FP4 codes and E4M3
//    scales of the SP positions and write code*scale as fp16 rows into LDS
//    (exact: at most 6 significant bits, range 2^-10..2688).
//  * Each wave owns 16 heads (one MFMA tile) and 32-position sub-tiles:
//      S^T = K Q^T   v_mfma_f32_16x16x32_f16, K rows read from LDS (b128),
//                    Q in registers (fp16), 16 k-steps over 512 channels;
//      online softmax in registers (exp2 domain);
//      O^T += V^T P^T  32 channel tiles, V^T read straight from the
//                    row-major LDS tile with ds_read_b64_tr_b16, P^T from
//                    the S^T accumulators (lane layout already matches).
//  * Each wave writes its (max, sum, O) partial; a combine kernel merges the
//    partials of every head (split-K over positions).
//
// MFMA 16x16x32 f16 lane layout (checked on gfx950): A row = lane%16 with
// k = 8*(lane/16)..+7; B column = lane%16, same k; C column = lane%16,
// rows 4*(lane/16)..+3.  ds_read_b64_tr_b16: within each 16-lane group,
// result lane i, element r comes from element i%4 of the 8 bytes addressed
// by lane 4r + i/4.
#include "common.hpp"

namespace csa2 {

constexpr int ATT_THREADS = 256;
constexpr int ROW_HALVES = D + 8;                 // LDS row stride: 1040 bytes

struct AttendArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const int64_t *seq_len;
  int64_t capacity;
  int64_t limit;            // min(capacity, max_len)
  const float *q;           // [batch][heads][512]
  const int32_t *idx;       // [batch][topk]
  int32_t topk;
  float scale_log2;         // scale * log2(e)
  int32_t n_stages;         // ceil(topk*8 / SP)
  int32_t splits;           // workgroups per sequence
  float *part_o;            // [batch][splits][4 waves][32 tiles][64 lanes][4]: the O^T
                            // accumulators in lane order (contiguous stores)
  float *part_ml;           // [batch][splits][4 waves][16 heads][2]
};

template <int HT>   // head tiles of 16: 1, 2 or 4
__global__ void __launch_bounds__(ATT_THREADS) attend_partial_kernel(AttendArgs a) {
  constexpr int WPT = 4 / HT;                     // waves per head tile
  constexpr int NSUB = (HT == 4) ? 2 : 1;         // 32-position sub-tiles per wave per stage
  constexpr int SP = 32 * NSUB * WPT;             // positions per stage: 64, 64, 128
  extern __shared__ _Float16 s_v[];               // [SP][ROW_HALVES]
  __shared__ uint8_t s_ok[SP];

  const int b = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ht = wv % HT, wsub = wv / HT;
  const int n16 = lane & 15, g = lane >> 4;
  const int64_t n = clamp_len(a.seq_len[b], a.limit);
  const int64_t nblk = (n + BLOCK - 1) / BLOCK;
  const int32_t *idx = a.idx + (int64_t)b * a.topk;
  const uint8_t *codes = a.codes + (int64_t)b * a.capacity * CODE_BYTES;
  const uint8_t *scales = a.scales + (int64_t)b * a.capacity * SCALE_BYTES;
  const int total_pos = a.topk * BLOCK;

  // stage range of this workgroup
  const int st0 = (int)((int64_t)a.n_stages * split / a.splits);
  const int st1 = (int)((int64_t)a.n_stages * (split + 1) / a.splits);

  // ---- gathered rows of a stage: block ids, then rows (two round trips) --
  constexpr int PASSES = SP / 16;         // rows per thread per stage
  const int i16 = tid & 15;               // this thread's 16-byte column of a row
  int64_t posv[PASSES];
  bool okv[PASSES];
  u32x4 wr[PASSES];
  uint32_t scr[PASSES];
  auto fetch_stage = [&](int st) {
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int pp = (tid >> 4) + 16 * k;
      const int j = st * SP + pp;
      const int32_t blk = j < total_pos ? idx[j >> 3] : -1;
      posv[k] = (int64_t)blk * BLOCK + (j & 7);
      okv[k] = blk >= 0 && blk < nblk && posv[k] < n;
      if (blk >= nblk && i16 == 0 && (j & 7) == 0) raise_flag(FLAG_BAD_INDEX);
    }
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      if (okv[k]) {
        wr[k] = *reinterpret_cast<const u32x4 *>(codes + posv[k] * CODE_BYTES + 16 * i16);
        scr[k] = *reinterpret_cast<const uint16_t *>(scales + posv[k] * SCALE_BYTES + 2 * i16);
      } else {
        wr[k] = u32x4{0u, 0u, 0u, 0u};
        scr[k] = 0u;
      }
    }
  };
  // the first stage's rows are requested before the query is staged
  if (st0 < st1) fetch_stage(st0);

  // Q^T operand: head ht*16 + n16, channels 32*kc + 8*g + 0..7.  q is staged
  // through LDS (coalesced float4 loads issued 16 per thread at a time,
  // stored as fp16 rows in the space the stages use later), then each lane
  // reads its 16 operand chunks.
  f16x8 qop[16];
  {
    constexpr int NV = 16 * HT * D / 4 / ATT_THREADS;       // float4 per thread: 8*HT
    constexpr int BATCH = NV < 16 ? NV : 16;
    const float4 *src = reinterpret_cast<const float4 *>(a.q + (int64_t)b * (16 * HT) * D);
#pragma unroll
    for (int u0 = 0; u0 < NV; u0 += BATCH) {
      float4 v[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) v[u] = src[tid + (u0 + u) * ATT_THREADS];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int e = tid + (u0 + u) * ATT_THREADS;        // float4 index: head e/128, channels 4*(e%128)
        f16x2 lo = {(_Float16)v[u].x, (_Float16)v[u].y}, hi = {(_Float16)v[u].z, (_Float16)v[u].w};
        *reinterpret_cast<u32x2 *>(s_v + (e >> 7) * ROW_HALVES + 4 * (e & 127)) =
            u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
    }
    __syncthreads();
    const _Float16 *qrow = s_v + (ht * 16 + n16) * ROW_HALVES + 8 * g;
#pragma unroll
    for (int kc = 0; kc < 16; ++kc) qop[kc] = *reinterpret_cast<const f16x8 *>(qrow + 32 * kc);
  }

  f32x4 acc[32];
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf();   // running max of this lane's head (log2 domain)
  float l_run = 0.f;                      // this lane's share of the softmax sum

#pragma unroll 1
  for (int st = st0; st < st1; ++st) {
    __syncthreads();                      // query / previous stage fully consumed
    if (st != st0) fetch_stage(st);
    // ---- dequantise the stage's rows into LDS as fp16 (16 threads per row) ----
#pragma unroll
    for (int k = 0; k < PASSES; ++k) {
      const int pp = (tid >> 4) + 16 * k;
      const _Float16 s0 = (_Float16)e4m3_to_f32(scr[k] & 0xffu);
      const _Float16 s1 = (_Float16)e4m3_to_f32(scr[k] >> 8);
      const f16x2 sv0 = {s0, s0}, sv1 = {s1, s1};
      u32x4 *dst = reinterpret_cast<u32x4 *>(s_v + pp * ROW_HALVES + 32 * i16);
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        const f16x2 sv = dw < 2 ? sv0 : sv1;
        f16x2 h0 = e2m1x2_to_f16<0>(wr[k][dw]) * sv;
        f16x2 h1 = e2m1x2_to_f16<1>(wr[k][dw]) * sv;
        f16x2 h2 = e2m1x2_to_f16<2>(wr[k][dw]) * sv;
        f16x2 h3 = e2m1x2_to_f16<3>(wr[k][dw]) * sv;
        dst[dw] = u32x4{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                        __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
      }
      if (i16 == 0) s_ok[pp] = okv[k] ? 1 : 0;
    }
    __syncthreads();

    // ---- this wave's 32-position sub-tiles of the stage (kept as a loop:
    // every dispatch starts with a cold instruction cache) ----
#pragma unroll 1
    for (int sub = 0; sub < NSUB; ++sub) {
      const int base = 32 * (wsub * NSUB + sub);          // first row of the sub-tile
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const _Float16 *krow = s_v + (base + 16 * t + n16) * ROW_HALVES + 8 * g;
#pragma unroll
        for (int kc = 0; kc < 16; ++kc) {
          f16x8 kop = *reinterpret_cast<const f16x8 *>(krow + 32 * kc);
          sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[kc], sacc[t], 0, 0, 0);
        }
      }
      // lane (head n16, group g) holds logits of rows 4g..4g+3 of tiles 0 and 1:
      // positions base + 4g + r and base + 16 + 4g + r
      float z[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = s_ok[base + 4 * g + r] ? sacc[0][r] * a.scale_log2 : -__builtin_huge_valf();
        z[4 + r] = s_ok[base + 16 + 4 * g + r] ? sacc[1][r] * a.scale_log2 : -__builtin_huge_valf();
      }
      float mx = z[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) mx = fmaxf(mx, z[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      float corr = 1.f;
      _Float16 ph[8];
      if (m_new == -__builtin_huge_valf()) {
#pragma unroll
        for (int r = 0; r < 8; ++r) ph[r] = (_Float16)0.f;
      } else {
        corr = __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          ph[r] = (_Float16)__builtin_amdgcn_exp2f(z[r] - m_new);
          psum += (float)ph[r];
        }
        l_run = l_run * corr + psum;
        m_run = m_new;
      }
      if (corr != 1.f) {
#pragma unroll
        for (int ct = 0; ct < 32; ++ct) acc[ct] *= corr;
      }
      const f16x8 pop = {ph[0], ph[1], ph[2], ph[3], ph[4], ph[5], ph[6], ph[7]};
      // V^T operand rows (k) = positions base + 4g + 0..3 then base + 16 + 4g + 0..3;
      // source lane s = 4r + q points at row k0 + r, channel n0 + 32q, so row
      // m of O^T tile ct holds channel 128*(ct/8) + 4*(ct%8) + 32*(m/4) + m%4
      // (groups of 4 lanes read 8 bytes 64 bytes apart: no LDS bank conflict)
      const int r_src = n16 >> 2, q_src = n16 & 3;
      const _Float16 *v0 = s_v + (base + 4 * g + r_src) * ROW_HALVES + 32 * q_src;
      const _Float16 *v1 = v0 + 16 * ROW_HALVES;
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) {
        const int n0 = 128 * (ct >> 3) + 4 * (ct & 7);
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(v0 + n0));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(v1 + n0));
        f16x8 vop = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop, acc[ct], 0, 0, 0);
      }
    }
  }

  // ---- write this wave's partial: O^T rows 4g..4g+3 of every tile ----
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t slot = ((int64_t)b * a.splits + split) * 4 + wv;
  f32x4 *po = reinterpret_cast<f32x4 *>(a.part_o + slot * (16 * D)) + lane;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) po[ct * 64] = acc[ct];
  if (g == 0) {
    float *pm = a.part_ml + (slot * 16 + n16) * 2;
    pm[0] = m_run;
    pm[1] = l_tot;
  }
}

struct CombineArgs {
  const float *part_o;
  const float *part_ml;
  int32_t splits;
  int32_t heads;
  float *out;               // [batch][heads][512]
};

// grid (heads, batch), 128 threads x 4 channels: merge every partial of a
// head.  The (max, sum) of every slot go through LDS first (vector loads;
// uniform-address loads would become serialised scalar loads), then each
// thread reads its 4 channels of every slot, 8 slots per batch.
constexpr int MAX_SLOTS = 1024;
__global__ void __launch_bounds__(128) attend_combine_kernel(CombineArgs a) {
  __shared__ float s_m[MAX_SLOTS], s_l[MAX_SLOTS];
  constexpr int U = 8;
  const int hh = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int HT = a.heads / 16, ht = hh / 16, n16 = hh % 16;
  const int WPT = 4 / HT;
  const int nslots = a.splits * WPT;
  auto slot_of = [&](int s) -> int64_t {
    return ((int64_t)b * a.splits + s / WPT) * 4 + ht + HT * (s % WPT);
  };
  float M = -__builtin_huge_valf();
  for (int s = t; s < nslots; s += 128) {
    const float2 ml = reinterpret_cast<const float2 *>(a.part_ml)[slot_of(s) * 16 + n16];
    s_m[s] = ml.x;
    s_l[s] = ml.y;
  }
  __syncthreads();
  for (int s = 0; s < nslots; ++s) M = fmaxf(M, s_m[s]);
  // channels 4t..4t+3 live in tile ct, lane 16g + n16 of the wave's partial
  const int ct = 8 * (t >> 5) + (t & 7), g = (t >> 3) & 3;
  const int64_t within = (int64_t)(ct * 64 + 16 * g + n16) * 4;
  float L = 0.f;
  float4 o = {0.f, 0.f, 0.f, 0.f};
  if (M != -__builtin_huge_valf()) {
#pragma unroll 1
    for (int s0 = 0; s0 < nslots; s0 += U) {
      float4 ov[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        ov[u] = (s0 + u < nslots) ? *reinterpret_cast<const float4 *>(a.part_o + slot_of(s0 + u) * (16 * D) + within)
                                  : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u >= nslots) break;
        const float m = s_m[s0 + u];
        if (m == -__builtin_huge_valf()) continue;
        const float e = __builtin_amdgcn_exp2f(m - M);
        L += e * s_l[s0 + u];
        o.x += e * ov[u].x; o.y += e * ov[u].y; o.z += e * ov[u].z; o.w += e * ov[u].w;
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
  reinterpret_cast<float4 *>(a.out + ((int64_t)b * a.heads + hh) * D)[t] = o;
}

template __global__ void attend_partial_kernel<1>(AttendArgs);
template __global__ void attend_partial_kernel<2>(AttendArgs);
template __global__ void attend_partial_kernel<4>(AttendArgs);

}  // namespace csa2
