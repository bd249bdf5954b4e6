// Device-side helpers shared by the CSA2 kernels (gfx950, wave64).
//
// Format facts used here: FP4 E2M1 element codes with one E4M3 scale per 16
// channels of the 512-channel latent (ailily.cc "890 bytes per token",
// section 二 and 三); fixed-stride rows addressed by position index
// (yomxxx.com long-form post, section 五).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int D = 512;            // latent channels
constexpr int BLOCK = 8;          // positions per block
constexpr int CODE_BYTES = 256;   // FP4 bytes per position
constexpr int SCALE_BYTES = 32;   // E4M3 scales per position
constexpr int GROUP = 16;         // channels per scale
constexpr int NGROUPS = 32;
constexpr int WAVE = 64;

constexpr int HIST_BINS = 1024;   // first radix digit: top 10 bits of the score key
constexpr int HIST_SHIFT = 22;
constexpr int HIST_COPIES = 8;    // histogram copies (workgroup x adds to copy x % 8)
constexpr int CAND_COPIES = 8;    // tie-candidate lists, likewise
constexpr int MAX_GRID_X = 2048;  // workgroups per grid row of a hand-off kernel

// Device flag bits (mirrors include/csa2.h).
constexpr uint32_t FLAG_NONFINITE_KV = 1, FLAG_CAPACITY = 2, FLAG_NONFINITE_Q = 4,
                   FLAG_BAD_INDEX = 8, FLAG_Q_RANGE = 32, FLAG_CHECK = 64;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Per-sequence control words of a workspace (1 KB of arrival/tie counters,
// then 8 KB of full-scan work counters).
constexpr int SCAN_GROUPS = 64;         // full-scan workgroup groups sharing a work counter

struct Ctrl {
  uint32_t sel_grp[MAX_GRID_X / 32];    // select / rescore arrivals per group of 32 workgroups
  uint32_t sel_top;                     // groups complete
  uint32_t ncand[CAND_COPIES];          // tie candidates collected per list
  uint32_t pad[256 - (MAX_GRID_X / 32) - 1 - CAND_COPIES];
  uint32_t work[SCAN_GROUPS * 32];      // full-scan work counters, one per 128-byte line
};

// E4M3FN byte -> float (exact).  gfx950 decodes the OCP FN variant.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Two E2M1 codes of byte `sel` (0..3) of w -> floats, low nibble first.
// The hardware applies only the exponent of its scale operand, so it is
// always called with 1.0 and the E4M3 scale is applied by the caller.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f16x2 e2m1x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Valid positions of a sequence: seq_len clamped to [0, limit], where
// limit = min(capacity, host max_len), so a bad length can never move an
// access outside the cache.
__device__ __forceinline__ int64_t clamp_len(int64_t n, int64_t limit) {
  return n < 0 ? 0 : (n > limit ? limit : n);
}

// Order-preserving map of a float (no NaN) onto uint32.
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Phase timestamps for profiling builds only (compiled with
// -DCSA2_PHASE_TIMING; the normal build compiles the hook away).  Thread 0
// of each workgroup records s_memrealtime (100 MHz) after its wave's memory
// operations complete; with -DCSA2_PHASE_TIMING_LIGHT it records the
// core-clock counter (s_memtime) as the wave reaches the hook, without
// waiting for outstanding memory operations (progress, not arrival).
#ifdef CSA2_PHASE_TIMING
constexpr int TS_SLOTS = 32;
__device__ unsigned long long g_phase_ts[4096][TS_SLOTS];
#ifdef CSA2_PHASE_TIMING_LIGHT
#define CSA2_TS(k)                                                                     \
  do {                                                                                 \
    const unsigned wg_ = blockIdx.x + blockIdx.y * gridDim.x;                          \
    if (threadIdx.x == 0 && wg_ < 4096) g_phase_ts[wg_][k] = __builtin_amdgcn_s_memtime(); \
  } while (0)
#else
#define CSA2_TS(k)                                                                     \
  do {                                                                                 \
    __builtin_amdgcn_s_waitcnt(0);                                                     \
    const unsigned wg_ = blockIdx.x + blockIdx.y * gridDim.x;                          \
    if (threadIdx.x == 0 && wg_ < 4096) g_phase_ts[wg_][k] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#endif
#else
#define CSA2_TS(k) \
  do {             \
  } while (0)
#endif

// Device-wide flag word; read and cleared by csa2_device_error.
extern __device__ uint32_t g_flags;
__device__ __forceinline__ void raise_flag(uint32_t bit) {
  __hip_atomic_fetch_or(&g_flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- checked build (-DCSA2_CHECKED: libcsa2_checked.so) -------------------
//
// Two debugging aids that the product library compiles away:
// * wg_x(), the workgroup's logical index along x, from which every kernel
//   derives the work it takes.  The product build returns blockIdx.x.  The
//   checked build returns (blockIdx.x * p + salt) mod gridDim.x, with p the
//   first of three primes that does not divide gridDim.x (a bijection), so
//   the hardware's in-order dispatch hands the work to other physical
//   workgroups and every cross-workgroup hand-off sees another arrival
//   order.  The salt is the CSA2_WG_ORDER environment variable, read at the
//   library's first call on a device (0 keeps the identity order).
// * CSA2_CHECK(cond): an index bound that a kernel's memory accesses rely
//   on.  The checked build raises FLAG_CHECK when it does not hold; it only
//   records (the access still goes ahead), so it is for runs on valid
//   inputs, whose flag word must stay zero.
#ifdef CSA2_CHECKED
extern __device__ uint32_t g_wg_salt;
__device__ __forceinline__ uint32_t wg_x() {
  const uint32_t n = gridDim.x, salt = g_wg_salt;
  if (salt == 0 || n < 2) return blockIdx.x;
  const uint32_t p = (n % 65521u) ? 65521u : (n % 40009u) ? 40009u : 7919u;
  return (uint32_t)(((uint64_t)blockIdx.x * p + salt) % n);
}
#define CSA2_CHECK(cond)                         \
  do {                                           \
    if (!(cond)) raise_flag(::csa2::FLAG_CHECK); \
  } while (0)
#else
__device__ __forceinline__ uint32_t wg_x() { return blockIdx.x; }
#define CSA2_CHECK(cond) \
  do {                   \
  } while (0)
#endif

// Load of a value another workgroup of the same kernel wrote (after the
// arrive_last hand-off): agent-scope atomic load, coherent across XCDs.
template <typename T>
__device__ __forceinline__ T ld_agent(const T *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// "Last workgroup" hand-off without device-scope fences.
//
// On gfx950 a release fence per workgroup (an L2 write-back) followed by an
// arrival on one counter costs about 75 ns per workgroup, serialised (77 us
// for 1024 workgroups, measured), and same-address atomics serialise at
// about 12 ns each.  So: every value the last workgroup reads is written
// with a device-scope store or atomic (st_agent, atomic_add_agent: written
// through to the device coherence point, not left in an XCD's L2); each
// wave waits for all of its memory operations to
// complete (s_waitcnt 0) before the workgroup barrier; the arrival counts on
// two levels (groups of 32 workgroups, then groups), so no address sees more
// than 64 contending atomics; the last workgroup reads with device-scope
// atomic loads.  Counters reset themselves.  All threads of the workgroup
// call this once; exactly one workgroup per grid row gets true.
__device__ __forceinline__ bool arrive_last(uint32_t *grp, uint32_t *top, uint32_t nwg) {
  __shared__ uint32_t s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t g = blockIdx.x >> 5;
    const uint32_t gsize = min(32u, nwg - 32u * g);
    const uint32_t ngroups = (nwg + 31) >> 5;
    uint32_t last = 0;
    if (__hip_atomic_fetch_add(grp + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gsize - 1) {
      __hip_atomic_store(grp + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = 1;
      }
    }
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

// Agent-scope store: written through to the device coherence point (a plain
// store with the device-scope cache bit), so a later ld_agent on another XCD
// sees it once the writer's vmcnt has drained.
template <typename T>
__device__ __forceinline__ void st_agent(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- wave64 primitives on DPP lane moves (no LDS round trip) --------------
// update_dpp(old, src, ctrl, row_mask, bank_mask, bound_ctrl): lanes whose
// source is outside the 16-lane row, or whose row is masked off, keep `old`.
#define CSA2_DPP(x, ctrl, rmask) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x), (ctrl), (rmask), 0xf, false))

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each row
// (shift right 1, 2, 4, 8), then row 0's total into row 1 and row 2's into
// row 3 (broadcast of lane 15), then lane 31's into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += CSA2_DPP(x, 0x111, 0xf);
  x += CSA2_DPP(x, 0x112, 0xf);
  x += CSA2_DPP(x, 0x114, 0xf);
  x += CSA2_DPP(x, 0x118, 0xf);
  x += CSA2_DPP(x, 0x142, 0xa);
  x += CSA2_DPP(x, 0x143, 0xc);
  return x;
}

// Minimum / maximum over the wave, uniform: butterflies inside each row
// (quad swaps, then rotations by 4 and 8), then the four row results.
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x124, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x128, 0xf, 0xf, false));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x124, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x128, 0xf, 0xf, false));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return max(max(a, b), max(c, d));
}

// Lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace csa2
