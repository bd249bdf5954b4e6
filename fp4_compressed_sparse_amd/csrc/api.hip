// Host side of the CSA2 C ABI: validation, workspace layout, launches and
// the layer-stack driver.  The kernel sources are compiled in this single
// translation unit so the device flag word has one definition.
//
// Modes and the hierarchical pool follow rebasdaily.com "DeepSeek-V4.1-Flash
// KV compression", section "same notes, many layers" (Full / Reindex /
// Reuse; the first Full layer scans everything into a pool that later layers
// search) and the mode table of ailily.cc "890 bytes per token", section 二.
#include "quantize.hip"
#include "index.hip"
#include "headmax.hip"
#include "attend.hip"

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "csa2.h"

using namespace csa2;

// The library's own workspace for csa2_decode_step_noalloc (callers that
// cannot allocate): one copy per device, held until the process ends.  Host
// code never uses this name as an address: the device address comes from
// hipGetSymbolAddress, per device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_WORKSPACE_BYTES];

namespace {

thread_local std::string t_last_error;
thread_local hipEvent_t t_scan_before = nullptr, t_scan_after = nullptr;

csa2_status fail(csa2_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return s;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

csa2_status launched(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CSA2_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return CSA2_OK;
}

// One-time per-device setup: architecture check and LDS limits.
csa2_status device_ready() {
  static std::mutex mu;
  static int state[64] = {0};   // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CSA2_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(CSA2_E_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(CSA2_E_HIP, "hipGetDeviceProperties failed");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      state[dev] = 2;
    } else {
      const int big = 160 * 1024 - 16 * 1024;
      for (const void *k : {reinterpret_cast<const void *>(&attend64_kernel),
                            reinterpret_cast<const void *>(&attend_partial_kernel<false, false>),
                            reinterpret_cast<const void *>(&attend_partial_kernel<true, false>),
                            reinterpret_cast<const void *>(&attend_partial_kernel<false, true>),
                            reinterpret_cast<const void *>(&attend_partial_kernel<true, true>)})
        (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, big);
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, big);
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&select2_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, big);
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&rescore_kernel<true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, big);
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&select_cand_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, big);
      (void)hipGetLastError();
#ifdef CSA2_CHECKED
      {
        // checked build: the workgroup-order salt (a blocking copy, once per
        // device; this build is not meant for graph capture)
        const char *env = getenv("CSA2_WG_ORDER");
        const uint32_t salt = env ? (uint32_t)strtoul(env, nullptr, 10) : 0u;
        const hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_wg_salt), &salt, sizeof salt, 0, hipMemcpyHostToDevice);
        if (e != hipSuccess) return fail(CSA2_E_HIP, "set workgroup order: %s", hipGetErrorString(e));
      }
#endif
      state[dev] = 1;
    }
  }
  if (state[dev] == 2) return fail(CSA2_E_UNSUPPORTED, "device %d is not gfx950", dev);
  return CSA2_OK;
}

// ---- workspace layout ----------------------------------------------------

int att_splits(int workgroup_rows, int n_stages) {
  int want = (int)ceil_div(512, workgroup_rows);
  if (want < 1) want = 1;
  if (want > MAX_SPLITS) want = MAX_SPLITS;
  return n_stages < want ? n_stages : want;
}

struct Layout {
  size_t ctrl, hist, scores, bitmap, cands, qbar, part_o, part_ml, cscores, total;
  int64_t score_stride, cand_stride;
  int32_t nwords;
  int32_t att_stages, att_splits;
};

bool make_layout(int32_t batch, int32_t heads, int64_t max_len, int32_t pool, int32_t topk, Layout *L) {
  if (batch < 1 || max_len < 0 || topk < 1 || topk > CSA2_MAX_TOPK || pool < 0 || pool > CSA2_MAX_POOL)
    return false;
  if (heads < 1 || heads > CSA2_MAX_HEADS) return false;
  const int64_t nblk = ceil_div(max_len, BLOCK);
  L->score_stride = ceil_div(nblk > CSA2_MAX_POOL ? nblk : CSA2_MAX_POOL, 64) * 64;
  L->nwords = (int32_t)(ceil_div(nblk > 0 ? nblk : 1, 64) * 2);
  L->cand_stride = nblk > 0 ? nblk : 1;
  size_t off = 0;
  L->ctrl = off;   off = align256(off + sizeof(Ctrl) * batch);
  L->hist = off;   off = align256(off + sizeof(uint32_t) * HIST_COPIES * HIST_BINS * (size_t)batch);
  L->scores = off; off = align256(off + sizeof(float) * (size_t)L->score_stride * batch);
  L->bitmap = off; off = align256(off + sizeof(uint32_t) * (size_t)L->nwords * batch);
  L->cands = off;  off = align256(off + sizeof(uint64_t) * CAND_COPIES * (size_t)L->cand_stride * batch);
  L->qbar = off;   off = align256(off + sizeof(float) * D * (size_t)batch);
  L->cscores = off; off = align256(off + sizeof(float) * (size_t)(pool > 0 ? pool : 1) * batch);
  L->att_stages = L->att_splits = 0;
  L->part_o = L->part_ml = off;
  if (heads == 16 || heads == 32 || heads == 64) {
    L->att_stages = (int32_t)ceil_div((int64_t)topk * BLOCK, ATT_SP);
    L->att_splits = att_splits(batch * (heads / 16), L->att_stages);
    // partials for the most splits any call may use: a local branch adds up
    // to CSA2_MAX_WINDOW / ATT_SP stages; one split normalises in-kernel
    const int cap = att_splits(batch * (heads / 16), L->att_stages + CSA2_MAX_WINDOW / ATT_SP);
    const size_t slots = cap > 1 ? (size_t)batch * cap * (heads / 16) * 16 : 0;
    L->part_o = off;  off = align256(off + sizeof(_Float16) * slots * D);
    L->part_ml = off; off = align256(off + sizeof(float) * slots * 2);
  }
  L->total = off;
  return true;
}

csa2_status check_kv(const csa2_kv *kv) {
  if (!kv) return fail(CSA2_E_ARG, "kv is NULL");
  if (!kv->codes || !kv->scales || !kv->seq_len) return fail(CSA2_E_ARG, "kv has a NULL pointer");
  if (!aligned(kv->codes, 256) || !aligned(kv->scales, 256))
    return fail(CSA2_E_ARG, "kv codes/scales must be 256-byte aligned");
  if (!aligned(kv->seq_len, 8)) return fail(CSA2_E_ARG, "kv seq_len must be 8-byte aligned");
  if (kv->batch < 1 || kv->batch > 65535) return fail(CSA2_E_ARG, "kv batch %d out of range", kv->batch);
  if (kv->capacity < BLOCK || kv->capacity % BLOCK)
    return fail(CSA2_E_SHAPE, "kv capacity %lld must be a positive multiple of 8", (long long)kv->capacity);
  if (kv->max_len < 0 || kv->max_len > kv->capacity)
    return fail(CSA2_E_CAPACITY, "kv max_len %lld outside [0, capacity %lld]", (long long)kv->max_len,
                (long long)kv->capacity);
  return CSA2_OK;
}

static_assert(MAX_SWA_RINGS == CSA2_MAX_SWA_LAYERS, "ring table size");

// Ring positions of an SWA view (0 means as many as the window).
inline int32_t swa_slots(const csa2_swa *swa) { return swa->slots ? swa->slots : swa->window; }

csa2_status check_swa(const csa2_swa *swa, int32_t batch) {
  if (!swa->codes || !swa->scales || !swa->seq_len) return fail(CSA2_E_ARG, "swa has a NULL pointer");
  if (!aligned(swa->codes, 16) || !aligned(swa->scales, 4) || !aligned(swa->seq_len, 8))
    return fail(CSA2_E_ARG, "swa codes/scales/seq_len misaligned");
  if (swa->window < 1 || swa->window > CSA2_MAX_WINDOW)
    return fail(CSA2_E_SHAPE, "swa window %d outside [1, %d]", swa->window, CSA2_MAX_WINDOW);
  if (swa->slots != 0 && (swa->slots < swa->window || swa->slots > CSA2_MAX_SWA_SLOTS))
    return fail(CSA2_E_SHAPE, "swa slots %d outside [window %d, %d]", swa->slots, swa->window, CSA2_MAX_SWA_SLOTS);
  if (swa->batch != batch) return fail(CSA2_E_ARG, "swa batch %d != %d", swa->batch, batch);
  return CSA2_OK;
}

csa2_status check_ws(void *ws, size_t ws_bytes, const Layout &L) {
  if (!ws) return fail(CSA2_E_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(CSA2_E_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(CSA2_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  return CSA2_OK;
}

// The words that must be zero when a call starts (control words, digit
// counts, the fallback selection's bitmap) sit at offsets that depend on the
// call's bounds, and every call leaves only its own ones zero.  So the
// library remembers, per workspace, where the last call's were; a call
// whose layout differs zero-fills [0, cands) first (a kernel on its stream).
// A workspace seen for the first time is taken as zero-filled, as the ABI
// requires; csa2_workspace_init forgets it.
struct WsStamp {
  const void *ws;
  int32_t batch, nwords;
  size_t ctrl, hist, scores, bitmap, cands;
};
std::mutex g_ws_mu;
WsStamp g_ws_tab[256];
int g_ws_next = 0;

void ws_forget(const void *ws) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (WsStamp &e : g_ws_tab)
    if (e.ws == ws) e.ws = nullptr;
}

csa2_status ws_ready(void *ws, int32_t batch, const Layout &L, hipStream_t s) {
  const WsStamp now{ws, batch, L.nwords, L.ctrl, L.hist, L.scores, L.bitmap, L.cands};
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (WsStamp &e : g_ws_tab) {
    if (e.ws != ws) continue;
    if (e.batch == now.batch && e.nwords == now.nwords && e.ctrl == now.ctrl && e.hist == now.hist &&
        e.scores == now.scores && e.bitmap == now.bitmap && e.cands == now.cands)
      return CSA2_OK;
    const int64_t words = (int64_t)(L.cands / sizeof(uint32_t));
    zero_kernel<<<(int)std::min<int64_t>(2048, ceil_div(words, 256)), 256, 0, s>>>(static_cast<uint32_t *>(ws),
                                                                                    words);
    if (csa2_status st = launched("workspace re-zero")) return st;
    e = now;
    return CSA2_OK;
  }
  g_ws_tab[g_ws_next] = now;
  g_ws_next = (g_ws_next + 1) % (int)(sizeof(g_ws_tab) / sizeof(g_ws_tab[0]));
  return CSA2_OK;
}

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

// Workgroups per grid row: about `target` in total over the batch, at most
// one per item and at most MAX_GRID_X (the hand-off counters' capacity).
int grid_for(int64_t items, int batch, int target) {
  int64_t want = ceil_div(target, batch);
  if (want < 1) want = 1;
  if (items < want) want = items;
  if (want > MAX_GRID_X) want = MAX_GRID_X;
  return (int)(want < 1 ? 1 : want);
}

// ---- launches (arguments already validated) -----------------------------

// Per-head score rule: tile sizes and grid (headmax.hip; 4 waves of 128
// channels, about 190 registers: two workgroups per compute unit).  The full
// scan gives each of 512 workgroups 16 blocks at a time; the candidate
// rescoring gives each workgroup one tile of 4 candidates, so a 2,048-block
// pool spreads over 512 workgroups.
constexpr int HM_SCAN_NT = 16;
constexpr int HM_SCAN_GRID = 512;
constexpr int HM_CAND_NT = 4;

HeadmaxArgs headmax_args(const csa2_kv *kv, const float *q, int32_t heads, const int32_t *cand,
                         int32_t n_cand, float *scores, int64_t score_stride) {
  HeadmaxArgs ha;
  memset(&ha, 0, sizeof ha);
  ha.codes = kv->codes; ha.scales = kv->scales; ha.seq_len = kv->seq_len; ha.capacity = kv->capacity;
  ha.limit = kv->max_len;
  ha.q = q; ha.heads = heads; ha.cand = cand; ha.n_cand = n_cand;
  ha.scores = scores; ha.score_stride = score_stride;
  return ha;
}

csa2_status run_select(const csa2_kv *kv, int32_t R, int32_t *first_out, int32_t topk2, int32_t *idx_out,
                       void *ws, const Layout &L, hipStream_t s, float *pool_scores);

// qbar_ready: the query sum is already in the workspace (computed in the
// decode step's append launch for this same query).
csa2_status run_scan_select(const csa2_kv *kv, const float *q, int32_t heads, int32_t R,
                            int32_t *first_out, int32_t topk2, int32_t *idx_out, void *ws,
                            const Layout &L, hipStream_t s, float *pool_scores = nullptr,
                            bool qbar_ready = false, int32_t rule = CSA2_SCORE_SUM) {
  const int B = kv->batch;
  const int64_t nblk_grid = ceil_div(kv->max_len, BLOCK);
  if (rule == CSA2_SCORE_HEADMAX) {
    // per-head scores and their digit counts, then the same selection
    HeadmaxArgs ha = headmax_args(kv, q, heads, nullptr, 0, at<float>(ws, L.scores), L.score_stride);
    ha.nblk_grid = (int32_t)nblk_grid;
    ha.hist = at<uint32_t>(ws, L.hist);
    if (t_scan_before) (void)hipEventRecord(t_scan_before, s);
    const int64_t tiles = ceil_div(nblk_grid > 0 ? nblk_grid : 1, HM_SCAN_NT);
    headmax_kernel<4, HM_SCAN_NT, false, true><<<dim3(grid_for(tiles, B, HM_SCAN_GRID), B), 256, 0, s>>>(ha);
    if (csa2_status st = launched("headmax scan")) return st;
    if (t_scan_after) (void)hipEventRecord(t_scan_after, s);
    return run_select(kv, R, first_out, topk2, idx_out, ws, L, s, pool_scores);
  }
  ScanArgs sa;
  sa.codes = kv->codes; sa.scales = kv->scales; sa.seq_len = kv->seq_len; sa.capacity = kv->capacity;
  sa.limit = kv->max_len;
  sa.q = q; sa.heads = heads; sa.nblk_grid = (int32_t)nblk_grid;
  sa.scores = at<float>(ws, L.scores); sa.score_stride = L.score_stride;
  sa.ctrl = at<Ctrl>(ws, L.ctrl); sa.hist = at<uint32_t>(ws, L.hist);
  sa.R = R; sa.fill_invalid = 0;
  sa.qbar = at<float>(ws, L.qbar);
  if (!qbar_ready) {
    qbar_kernel<<<B, SCAN_THREADS, 0, s>>>(q, heads, at<float>(ws, L.qbar));
    if (csa2_status st = launched("qbar")) return st;
  }
  // a workgroup scores 8 blocks per round (4 waves x 2).  512 workgroups
  // (two per compute unit) stream the cache faster than more: at 1M, cold,
  // 56.6 us against 61.8 with 1,536 (six waves per SIMD) and 60.2 with
  // 1,024; 384 or 256 leave compute units idle (62.7, 77.8 us).  A batch
  // runs over its chunks laid end to end (scan_flat_kernel, 768 workgroups:
  // 279 us at batch 64 against 285 with 1,280 and 301 with 512), so ragged
  // lengths leave no slot idle (batch of 64, 32K-128K: 382 -> 288 us
  // against a per-sequence split).  Beyond its limits a batch gets 128
  // workgroups per sequence, which the dispatcher moves from short
  // sequences to long ones as they finish.
  const int64_t rounds = ceil_div(nblk_grid > 0 ? nblk_grid : 1, 8);
  dim3 g1(grid_for(rounds, B, B > 1 ? 128 * B : 512), B);
  if (t_scan_before) (void)hipEventRecord(t_scan_before, s);
  if (B > 1 && B <= SCAN_FLAT_MAXB && (int64_t)B * ((nblk_grid + 1) / 2) < ((int64_t)1 << 31))
    scan_flat_kernel<<<768, SCAN_THREADS, 0, s>>>(sa, B);
  else
    scan_kernel<true><<<g1, SCAN_THREADS, 0, s>>>(sa);
  if (csa2_status st = launched("scan")) return st;
  if (t_scan_after) (void)hipEventRecord(t_scan_after, s);
  return run_select(kv, R, first_out, topk2, idx_out, ws, L, s, pool_scores);
}

// Selection of the top-R scored blocks (and their top-topk2) from the
// workspace's scores and digit counts, as the full scan left them.
csa2_status run_select(const csa2_kv *kv, int32_t R, int32_t *first_out, int32_t topk2, int32_t *idx_out,
                       void *ws, const Layout &L, hipStream_t s, float *pool_scores) {
  const int B = kv->batch;
  const int64_t nblk_grid = ceil_div(kv->max_len, BLOCK);
  SelectArgs se;
  se.seq_len = kv->seq_len; se.limit = kv->max_len; se.scores = at<float>(ws, L.scores);
  se.score_stride = L.score_stride;
  se.ctrl = at<Ctrl>(ws, L.ctrl); se.bitmap = at<uint32_t>(ws, L.bitmap); se.nwords = L.nwords;
  se.cands = at<uint64_t>(ws, L.cands); se.cand_stride = L.cand_stride;
  se.R = R; se.first_out = first_out; se.topk = topk2; se.idx_out = idx_out;
  int lk = R > 4096 ? R : 4096;
  se.lds_keys = lk;
  se.pool_scores = pool_scores;
  se.hist = at<uint32_t>(ws, L.hist);
  if (L.nwords <= SEL2_WORDS && R <= SEL2_KEYS) {
    // the chosen ids' bitmap fits in one workgroup's LDS
    dim3 g2(std::max<int64_t>(1, ceil_div(nblk_grid, SEL2_SPAN)), B);
    se.lds_keys = select2_keys(L.nwords);
    select2_kernel<<<g2, SEL2_THREADS, select2_lds(L.nwords), s>>>(se);
    return launched("select");
  }
  dim3 g2(grid_for(ceil_div(L.nwords / 2, 4), B, 256), B);
  select_kernel<<<g2, SCAN_THREADS, (size_t)lk * sizeof(uint64_t), s>>>(se);
  return launched("select");
}

csa2_status run_rescore(const csa2_kv *kv, const float *q, int32_t heads, const int32_t *cand,
                        int32_t n_cand, int32_t topk, int32_t *idx_out, float *scores,
                        int64_t score_stride, Ctrl *ctrl, hipStream_t s, int32_t rule = CSA2_SCORE_SUM) {
  const int B = kv->batch;
  if (rule == CSA2_SCORE_HEADMAX) {
    // per-head scores of the list (one tile per workgroup), then, when a
    // selection is wanted, its top-k in one workgroup per sequence
    HeadmaxArgs ha = headmax_args(kv, q, heads, cand, n_cand, scores, score_stride);
    headmax_kernel<4, HM_CAND_NT, true, false><<<dim3((int)ceil_div(n_cand, HM_CAND_NT), B), 256, 0, s>>>(ha);
    if (csa2_status st = launched("headmax rescore")) return st;
    if (!idx_out) return CSA2_OK;
    RescoreArgs ra;
    memset(&ra, 0, sizeof ra);
    ra.seq_len = kv->seq_len; ra.limit = kv->max_len; ra.cand = cand; ra.n_cand = n_cand;
    ra.scores = scores; ra.score_stride = score_stride; ra.topk = topk; ra.idx_out = idx_out;
    select_cand_kernel<<<dim3(1, B), SCAN_THREADS, (size_t)n_cand * sizeof(uint64_t), s>>>(ra);
    return launched("candidate select");
  }
  RescoreArgs ra;
  ra.codes = kv->codes; ra.scales = kv->scales; ra.seq_len = kv->seq_len; ra.capacity = kv->capacity;
  ra.limit = kv->max_len;
  ra.q = q; ra.heads = heads; ra.cand = cand; ra.n_cand = n_cand;
  ra.scores = scores; ra.score_stride = score_stride; ra.ctrl = ctrl;
  ra.topk = topk; ra.idx_out = idx_out;
  dim3 g(grid_for(ceil_div(n_cand, BLOCKS_PER_ITER), B, 512), B);
  if (idx_out) {
    rescore_kernel<true><<<g, SCAN_THREADS, (size_t)n_cand * sizeof(uint64_t), s>>>(ra);
  } else {
    rescore32_kernel<<<g, RESCORE32_THREADS, 0, s>>>(ra);
  }
  return launched("rescore");
}

// idx given: attend over it.  idx NULL: take the top-k of (cand,
// cand_scores) inside the attention kernel and write it to idx_out.
csa2_status run_attend(const csa2_kv *kv, const float *q, int32_t heads, const int32_t *idx,
                       int32_t topk, float scale, float *out, void *ws, const Layout &L,
                       hipStream_t s, const int32_t *cand = nullptr, const float *cand_scores = nullptr,
                       int32_t n_cand = 0, int32_t *idx_out = nullptr, const csa2_swa *swa = nullptr) {
  const int B = kv->batch;
  AttendArgs aa;
  aa.codes = kv->codes; aa.scales = kv->scales; aa.seq_len = kv->seq_len; aa.capacity = kv->capacity;
  aa.limit = kv->max_len;
  aa.q = q; aa.idx = idx; aa.topk = topk;
  aa.scale_log2 = scale * 1.4426950408889634f;
  aa.n_sparse = L.att_stages;
  aa.window = swa ? swa->window : 0;
  aa.swa_slots = swa ? swa_slots(swa) : 1;
  aa.swa_stride = 1;
  aa.win_at_query = 0;
  aa.swa_codes = swa ? swa->codes : kv->codes;
  aa.swa_scales = swa ? swa->scales : reinterpret_cast<const float *>(kv->scales);
  aa.swa_len = swa ? swa->seq_len : kv->seq_len;
  aa.n_stages = L.att_stages + (int32_t)ceil_div(aa.window, ATT_SP);
  // window stages add workgroups only up to the next multiple of 64 splits
  // (the combine merges up to 64 in one load batch); beyond that they are
  // spread over the existing splits (<= the layout's capacity either way)
  const int base = att_splits(B * (heads / 16), aa.n_sparse);
  const int room = (int)ceil_div(base, 64) * 64;
  int splits = att_splits(B * (heads / 16), aa.n_stages);
  if (splits > room) splits = room;
  aa.splits = splits;
  aa.part_o = at<_Float16>(ws, L.part_o); aa.part_ml = at<float>(ws, L.part_ml);
  aa.heads = heads;
  aa.cand = cand; aa.cand_scores = cand_scores; aa.n_cand = n_cand; aa.idx_out = idx_out;
  aa.seq_stride = kv->capacity; aa.len_add = 0; aa.out = out;
  dim3 g(splits * (heads / 16), B);
  const size_t lds = (size_t)ATT_SP * ROW_HALVES * sizeof(_Float16);
  if (idx && swa)
    attend_partial_kernel<false, true><<<g, ATT_THREADS, lds, s>>>(aa);
  else if (idx)
    attend_partial_kernel<false, false><<<g, ATT_THREADS, lds, s>>>(aa);
  else if (swa)
    attend_partial_kernel<true, true><<<g, ATT_THREADS, lds, s>>>(aa);
  else
    attend_partial_kernel<true, false><<<g, ATT_THREADS, lds, s>>>(aa);
  if (csa2_status st = launched("attend")) return st;
  if (splits == 1) return CSA2_OK;
  CombineArgs ca;
  ca.part_o = aa.part_o; ca.part_ml = aa.part_ml; ca.splits = splits; ca.heads = heads; ca.out = out;
  // up to 8 splits (batches): one wave per output tile merges them all;
  // more: four waves of 8 or 16 splits each (one wave idles less than four)
  if (splits <= 8)
    attend_combine_regs_kernel<1, 8><<<dim3((heads / 16) * 32, B), 64, 0, s>>>(ca);
  else if (splits <= 32)
    attend_combine_regs_kernel<4, 8><<<dim3((heads / 16) * 32, B), 256, 0, s>>>(ca);
  else if (splits <= 64)
    attend_combine_regs_kernel<4, 16><<<dim3((heads / 16) * 32, B), 256, 0, s>>>(ca);
  else
    attend_combine_kernel<2><<<dim3((heads / 16) * 32, B), 128, 0, s>>>(ca);
  return launched("combine");
}

csa2_status check_select_args(int32_t topk, int32_t pool) {
  if (topk < 1 || topk > CSA2_MAX_TOPK) return fail(CSA2_E_SHAPE, "topk %d outside [1, %d]", topk, CSA2_MAX_TOPK);
  if (pool < 0 || pool > CSA2_MAX_POOL) return fail(CSA2_E_SHAPE, "pool %d outside [0, %d]", pool, CSA2_MAX_POOL);
  if (pool > 0 && pool < topk) return fail(CSA2_E_ARG, "pool %d < topk %d", pool, topk);
  return CSA2_OK;
}

// Attention-only layout of the prefill entry: partials only with more
// than one split.
// window > 0: the local branch adds ceil(window / 64) stages and runs on
// the per-head-tile kernel; without it 64 heads take one workgroup per
// (query, split) for all four head tiles.  att_stages counts the gathered
// stages only.
bool prefill_layout(int32_t n_q, int32_t heads, int32_t topk, int32_t window, Layout *L) {
  if (n_q < 1 || n_q > 65535 || topk < 1 || topk > CSA2_MAX_TOPK) return false;
  if (heads != 16 && heads != 32 && heads != 64) return false;
  memset(L, 0, sizeof *L);
  L->att_stages = (int32_t)ceil_div((int64_t)topk * BLOCK, ATT_SP);
  const int wstages = (int)ceil_div(window, ATT_SP);
  L->att_splits = att_splits(heads == 64 && window == 0 ? n_q : n_q * (heads / 16), L->att_stages + wstages);
  const size_t slots = L->att_splits > 1 ? (size_t)n_q * L->att_splits * (heads / 16) * 16 : 0;
  size_t off = 0;
  L->part_o = off;  off = align256(off + sizeof(_Float16) * slots * D);
  L->part_ml = off; off = align256(off + sizeof(float) * slots * 2);
  L->total = slots ? off : 0;
  return true;
}

}  // namespace

namespace csa2 {
// Plain streaming read (the read-rate yardstick for the full scan): four
// 16-byte loads per thread per round, grid-stride over 512 workgroups.
__global__ void __launch_bounds__(256) read_probe_kernel(const u32x4 *__restrict__ p, int64_t n,
                                                         uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; i < n; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[min(i + 256 * u, n - 1)];   // clamped: one batch, in bounds
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= (i + 256 * u < n) ? (v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]) : 0u;
  }
  sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace csa2

extern "C" {

const char *csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_E_ARG: return "invalid argument";
    case CSA2_E_SHAPE: return "unsupported shape";
    case CSA2_E_WORKSPACE: return "workspace too small";
    case CSA2_E_CAPACITY: return "capacity exceeded";
    case CSA2_E_HIP: return "HIP error";
    case CSA2_E_UNSUPPORTED: return "unsupported device";
    default: return "unknown status";
  }
}

const char *csa2_last_error(void) { return t_last_error.c_str(); }

csa2_status csa2_set_scan_events(void *before, void *after) {
  t_last_error.clear();
  if ((before == nullptr) != (after == nullptr)) return fail(CSA2_E_ARG, "set both events or neither");
  t_scan_before = reinterpret_cast<hipEvent_t>(before);
  t_scan_after = reinterpret_cast<hipEvent_t>(after);
  return CSA2_OK;
}

size_t csa2_workspace_bytes(int32_t batch, int32_t heads, int64_t max_len, int32_t pool, int32_t topk) {
  Layout L;
  if (!make_layout(batch, heads, max_len, pool, topk, &L)) return 0;
  return L.total;
}

csa2_status csa2_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  t_last_error.clear();
  if (!ws || !aligned(ws, 256) || ws_bytes % 4) return fail(CSA2_E_ARG, "workspace must be non-NULL, 256-byte aligned, size a multiple of 4");
  if (csa2_status st = device_ready()) return st;
  if (ws_bytes == 0) return CSA2_OK;
  const int64_t words = (int64_t)(ws_bytes / 4);
  const int grid = (int)(ceil_div(words, 256) < 2048 ? ceil_div(words, 256) : 2048);
  zero_kernel<<<grid, 256, 0, as_stream(stream)>>>(static_cast<uint32_t *>(ws), words);
  ws_forget(ws);
  return launched("workspace_init");
}

csa2_status fp4_quantize_kv(const float *x, int64_t rows, const int64_t *dst_row, int64_t dst_rows,
                            uint8_t *codes, uint8_t *scales, void *stream) {
  t_last_error.clear();
  if (rows < 0) return fail(CSA2_E_ARG, "rows %lld < 0", (long long)rows);
  if (rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return fail(CSA2_E_ARG, "NULL pointer");
  if (!aligned(x, 16)) return fail(CSA2_E_ARG, "x must be 16-byte aligned");
  if (!aligned(codes, 8)) return fail(CSA2_E_ARG, "codes must be 8-byte aligned (a group's 8 code bytes are one store)");
  if (dst_row && !aligned(dst_row, 8)) return fail(CSA2_E_ARG, "dst_row must be 8-byte aligned");
  if (dst_rows < 0 || (!dst_row && dst_rows < rows))
    return fail(CSA2_E_CAPACITY, "dst_rows %lld too small for %lld rows", (long long)dst_rows, (long long)rows);
  if (csa2_status st = device_ready()) return st;
  const int64_t groups = rows * NGROUPS;
  const int64_t want = ceil_div(groups, 256 * GU);    // one round of GU groups per thread
  // one group per thread and no grid-stride rounds up to 8M rows: a fuller
  // grid outran every capped grid that loops (465 vs 503-541 us at 1M rows)
  const int grid = (int)(want < (1 << 20) ? want : (1 << 20));
  quantize_rows_kernel<<<grid, 256, 0, as_stream(stream)>>>(x, rows, dst_row, dst_rows, codes, scales);
  return launched("quantize");
}

csa2_status csa2_append_kv(const csa2_kv *kv, const float *x, void *stream) {
  t_last_error.clear();
  if (csa2_status st = check_kv(kv)) return st;
  if (!x || !aligned(x, 16)) return fail(CSA2_E_ARG, "x must be non-NULL and 16-byte aligned");
  if (csa2_status st = device_ready()) return st;
  AppendArgs aa;
  memset(&aa, 0, sizeof aa);
  aa.codes[0] = kv->codes; aa.scales[0] = kv->scales; aa.seq_len[0] = kv->seq_len; aa.capacity[0] = kv->capacity;
  SwaRings rr;
  memset(&rr, 0, sizeof rr);
  append_kernel<<<dim3(kv->batch, 1), 128, 0, as_stream(stream)>>>(aa, rr, x, kv->batch, 1, 0, QbarJob{});
  return launched("append");
}

csa2_status fp8_quantize_kv(const float *x, int64_t rows, const int64_t *dst_row, int64_t dst_rows,
                            uint8_t *codes, float *scales, void *stream) {
  t_last_error.clear();
  if (rows < 0) return fail(CSA2_E_ARG, "rows %lld < 0", (long long)rows);
  if (rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return fail(CSA2_E_ARG, "NULL pointer");
  if (!aligned(x, 16)) return fail(CSA2_E_ARG, "x must be 16-byte aligned");
  if (!aligned(codes, 8) || !aligned(scales, 4)) return fail(CSA2_E_ARG, "codes/scales misaligned");
  if (dst_row && !aligned(dst_row, 8)) return fail(CSA2_E_ARG, "dst_row must be 8-byte aligned");
  if (dst_rows < 0 || (!dst_row && dst_rows < rows))
    return fail(CSA2_E_CAPACITY, "dst_rows %lld too small for %lld rows", (long long)dst_rows, (long long)rows);
  if (csa2_status st = device_ready()) return st;
  const int64_t want = ceil_div(rows, 4);            // one row per wave
  const int grid = (int)(want < 4096 ? want : 4096);
  fp8_quantize_kernel<<<grid, 256, 0, as_stream(stream)>>>(x, rows, dst_row, dst_rows, codes, scales);
  return launched("fp8 quantize");
}

csa2_status csa2_swa_append(const csa2_swa *swa, const float *x, void *stream) {
  t_last_error.clear();
  if (!swa) return fail(CSA2_E_ARG, "swa is NULL");
  if (swa->batch < 1 || swa->batch > 65535) return fail(CSA2_E_ARG, "swa batch %d out of range", swa->batch);
  if (csa2_status st = check_swa(swa, swa->batch)) return st;
  if (!x || !aligned(x, 16)) return fail(CSA2_E_ARG, "x must be non-NULL and 16-byte aligned");
  if (csa2_status st = device_ready()) return st;
  AppendArgs aa;
  memset(&aa, 0, sizeof aa);
  SwaRings rr;
  memset(&rr, 0, sizeof rr);
  rr.codes[0] = swa->codes; rr.scales[0] = swa->scales; rr.seq_len[0] = swa->seq_len;
  rr.rows[0] = x; rr.slots[0] = swa_slots(swa);
  append_kernel<<<dim3(swa->batch, 1), 128, 0, as_stream(stream)>>>(aa, rr, nullptr, swa->batch, 0, 1,
                                                                     QbarJob{});
  return launched("swa append");
}

csa2_status csa2_index_topk(int32_t mode, const csa2_kv *kv, const float *q, int32_t heads,
                            const int32_t *cand, int32_t n_cand, int32_t topk, int32_t *idx_out,
                            int32_t pool, int32_t *pool_out, const int32_t *prior_idx, void *ws,
                            size_t ws_bytes, void *stream) {
  t_last_error.clear();
  const int32_t rule = (mode & CSA2_MODE_HEADMAX) ? CSA2_SCORE_HEADMAX : CSA2_SCORE_SUM;
  mode &= ~CSA2_MODE_HEADMAX;
  if (mode != CSA2_FULL && mode != CSA2_REINDEX && mode != CSA2_REUSE)
    return fail(CSA2_E_ARG, "mode %d is not Full/Reindex/Reuse (optionally | CSA2_MODE_HEADMAX)", mode);
  if (!idx_out || !aligned(idx_out, 4)) return fail(CSA2_E_ARG, "idx_out must be non-NULL");
  if (topk < 1 || topk > CSA2_MAX_TOPK) return fail(CSA2_E_SHAPE, "topk %d outside [1, %d]", topk, CSA2_MAX_TOPK);
  hipStream_t s = as_stream(stream);
  if (mode == CSA2_REUSE) {
    if (!prior_idx) return fail(CSA2_E_ARG, "Reuse needs prior_idx");
    if (!kv || kv->batch < 1) return fail(CSA2_E_ARG, "Reuse needs kv for the batch size");
    if (csa2_status st = device_ready()) return st;
    if (prior_idx == idx_out) return CSA2_OK;
    const int64_t nidx = (int64_t)kv->batch * topk;
    copy_idx_kernel<<<(int)ceil_div(nidx, 256), 256, 0, s>>>(prior_idx, idx_out, nidx);
    return launched("reuse copy");
  }
  if (csa2_status st = check_kv(kv)) return st;
  if (!q || !aligned(q, 16)) return fail(CSA2_E_ARG, "q must be non-NULL and 16-byte aligned");
  if (heads < 1 || heads > CSA2_MAX_HEADS) return fail(CSA2_E_SHAPE, "heads %d outside [1, 64]", heads);
  if (csa2_status st = check_select_args(topk, pool)) return st;
  Layout L;
  if (!make_layout(kv->batch, heads, kv->max_len, pool, topk, &L)) return fail(CSA2_E_SHAPE, "bad sizes");
  if (csa2_status st = check_ws(ws, ws_bytes, L)) return st;
  if (csa2_status st = device_ready()) return st;
  if (csa2_status st = ws_ready(ws, kv->batch, L, s)) return st;
  if (cand) {
    if (pool != 0) return fail(CSA2_E_ARG, "pool must be 0 with a candidate list");
    if (n_cand < 1 || n_cand > CSA2_MAX_POOL) return fail(CSA2_E_SHAPE, "n_cand %d outside [1, %d]", n_cand, CSA2_MAX_POOL);
    if (!aligned(cand, 4)) return fail(CSA2_E_ARG, "cand misaligned");
    return run_rescore(kv, q, heads, cand, n_cand, topk, idx_out, at<float>(ws, L.scores),
                       L.score_stride, at<Ctrl>(ws, L.ctrl), s, rule);
  }
  if (pool > 0) {
    if (!pool_out || !aligned(pool_out, 4)) return fail(CSA2_E_ARG, "pool > 0 needs pool_out");
    return run_scan_select(kv, q, heads, pool, pool_out, topk, idx_out, ws, L, s, nullptr, false, rule);
  }
  return run_scan_select(kv, q, heads, topk, idx_out, 0, nullptr, ws, L, s, nullptr, false, rule);
}

csa2_status csa2_sparse_attend(const csa2_kv *kv, const float *q, int32_t heads, const int32_t *idx,
                               int32_t topk, float scale, const csa2_swa *swa, float *out, void *ws,
                               size_t ws_bytes, void *stream) {
  t_last_error.clear();
  if (csa2_status st = check_kv(kv)) return st;
  if (swa) {
    if (csa2_status st = check_swa(swa, kv->batch)) return st;
  }
  if (!q || !aligned(q, 16) || !out || !aligned(out, 16))
    return fail(CSA2_E_ARG, "q/out must be non-NULL and 16-byte aligned");
  if (!idx || !aligned(idx, 4)) return fail(CSA2_E_ARG, "idx must be non-NULL");
  if (heads != 16 && heads != 32 && heads != 64)
    return fail(CSA2_E_SHAPE, "attention heads must be 16, 32 or 64 (got %d)", heads);
  if (topk < 1 || topk > CSA2_MAX_TOPK) return fail(CSA2_E_SHAPE, "topk %d outside [1, %d]", topk, CSA2_MAX_TOPK);
  if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
    return fail(CSA2_E_ARG, "scale must be finite");
  Layout L;
  if (!make_layout(kv->batch, heads, kv->max_len, 0, topk, &L)) return fail(CSA2_E_SHAPE, "bad sizes");
  if (csa2_status st = check_ws(ws, ws_bytes, L)) return st;
  if (csa2_status st = device_ready()) return st;
  return run_attend(kv, q, heads, idx, topk, scale, out, ws, L, as_stream(stream), nullptr, nullptr, 0,
                    nullptr, swa);
}

size_t csa2_prefill_workspace_bytes(int32_t n_q, int32_t heads, int32_t topk) {
  Layout L0, L1;                          // without and with the largest local branch
  if (!prefill_layout(n_q, heads, topk, 0, &L0) || !prefill_layout(n_q, heads, topk, CSA2_MAX_WINDOW, &L1))
    return 0;
  return L0.total > L1.total ? L0.total : L1.total;
}

csa2_status csa2_prefill_attend(const csa2_kv *kv, int32_t seq, const float *q, int32_t n_q,
                                int32_t heads, const int64_t *qpos, const int32_t *idx,
                                int32_t topk, float scale, const csa2_swa *swa, float *out,
                                void *ws, size_t ws_bytes, void *stream) {
  t_last_error.clear();
  if (csa2_status st = check_kv(kv)) return st;
  if (seq < 0 || seq >= kv->batch) return fail(CSA2_E_ARG, "seq %d outside [0, %d)", seq, kv->batch);
  if (swa) {
    if (csa2_status st = check_swa(swa, kv->batch)) return st;
  }
  if (!q || !aligned(q, 16) || !out || !aligned(out, 16))
    return fail(CSA2_E_ARG, "q/out must be non-NULL and 16-byte aligned");
  if (!qpos || !aligned(qpos, 8) || !idx || !aligned(idx, 4)) return fail(CSA2_E_ARG, "qpos/idx must be non-NULL");
  if (heads != 16 && heads != 32 && heads != 64)
    return fail(CSA2_E_SHAPE, "attention heads must be 16, 32 or 64 (got %d)", heads);
  if (topk < 1 || topk > CSA2_MAX_TOPK) return fail(CSA2_E_SHAPE, "topk %d outside [1, %d]", topk, CSA2_MAX_TOPK);
  if (n_q < 1 || n_q > 65535) return fail(CSA2_E_SHAPE, "n_q %d outside [1, 65535]", n_q);
  if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
    return fail(CSA2_E_ARG, "scale must be finite");
  Layout L;
  const int32_t window = swa ? swa->window : 0;
  if (!prefill_layout(n_q, heads, topk, window, &L)) return fail(CSA2_E_SHAPE, "bad sizes");
  if (L.total) {
    if (csa2_status st = check_ws(ws, ws_bytes, L)) return st;
  }
  if (csa2_status st = device_ready()) return st;
  hipStream_t s = as_stream(stream);
  AttendArgs aa;
  memset(&aa, 0, sizeof aa);
  aa.codes = kv->codes + (int64_t)seq * kv->capacity * CODE_BYTES;
  aa.scales = kv->scales + (int64_t)seq * kv->capacity * SCALE_BYTES;
  aa.seq_len = qpos; aa.len_add = 1; aa.seq_stride = 0;      // every row b is a query of one sequence
  aa.capacity = kv->capacity; aa.limit = kv->max_len;
  aa.q = q; aa.idx = idx; aa.topk = topk; aa.heads = heads;
  aa.scale_log2 = scale * 1.4426950408889634f;
  aa.n_sparse = L.att_stages;
  aa.n_stages = L.att_stages + (int32_t)ceil_div(window, ATT_SP);
  aa.splits = L.att_splits;
  aa.window = window;
  if (swa) {
    // every query reads the ring of sequence seq, its window ending at its own position
    const int32_t slots = swa_slots(swa);
    aa.swa_slots = slots; aa.swa_stride = 0; aa.win_at_query = 1;
    aa.swa_codes = swa->codes + (int64_t)seq * slots * D;
    aa.swa_scales = swa->scales + (int64_t)seq * slots;
    aa.swa_len = swa->seq_len + seq;
  } else {
    aa.swa_slots = 1; aa.swa_stride = 0; aa.win_at_query = 0;
    aa.swa_codes = aa.codes; aa.swa_scales = nullptr; aa.swa_len = qpos;
  }
  aa.part_o = L.total ? at<_Float16>(ws, L.part_o) : nullptr;
  aa.part_ml = L.total ? at<float>(ws, L.part_ml) : nullptr;
  aa.out = out;
  const size_t lds = (size_t)ATT_SP * ROW_HALVES * sizeof(_Float16);
  const dim3 g16(L.att_splits * (heads / 16), n_q);
  if (swa)
    attend_partial_kernel<false, true><<<g16, ATT_THREADS, lds, s>>>(aa);
  else if (heads == 64)
    attend64_kernel<<<dim3(L.att_splits, n_q), ATT64_THREADS, ATT64_LDS, s>>>(aa);
  else
    attend_partial_kernel<false, false><<<g16, ATT_THREADS, lds, s>>>(aa);
  if (csa2_status st = launched("prefill attend")) return st;
  if (L.att_splits == 1) return CSA2_OK;
  CombineArgs ca;
  ca.part_o = aa.part_o; ca.part_ml = aa.part_ml; ca.splits = L.att_splits; ca.heads = heads; ca.out = out;
  if (L.att_splits <= 32)
    attend_combine_regs_kernel<4, 8><<<dim3((heads / 16) * 32, n_q), 256, 0, s>>>(ca);
  else if (L.att_splits <= 64)
    attend_combine_regs_kernel<4, 16><<<dim3((heads / 16) * 32, n_q), 256, 0, s>>>(ca);
  else
    attend_combine_kernel<2><<<dim3((heads / 16) * 32, n_q), 128, 0, s>>>(ca);
  return launched("prefill combine");
}

csa2_status csa2_block_scores(const csa2_kv *kv, const float *q, int32_t heads, const int32_t *cand,
                              int32_t n_cand, float *scores, int32_t score_rule, void *stream) {
  t_last_error.clear();
  if (score_rule != CSA2_SCORE_SUM && score_rule != CSA2_SCORE_HEADMAX)
    return fail(CSA2_E_ARG, "score_rule %d is not CSA2_SCORE_SUM or CSA2_SCORE_HEADMAX", score_rule);
  if (csa2_status st = check_kv(kv)) return st;
  if (!q || !aligned(q, 16) || !scores || !aligned(scores, 4))
    return fail(CSA2_E_ARG, "q/scores must be non-NULL and aligned");
  if (heads < 1 || heads > CSA2_MAX_HEADS) return fail(CSA2_E_SHAPE, "heads %d outside [1, 64]", heads);
  if (csa2_status st = device_ready()) return st;
  hipStream_t s = as_stream(stream);
  if (cand) {
    if (n_cand < 1 || n_cand > CSA2_MAX_POOL) return fail(CSA2_E_SHAPE, "n_cand %d outside [1, %d]", n_cand, CSA2_MAX_POOL);
    return run_rescore(kv, q, heads, cand, n_cand, 0, nullptr, scores, n_cand, nullptr, s, score_rule);
  }
  const int64_t nblk_grid = ceil_div(kv->max_len, BLOCK);
  if (nblk_grid == 0) return CSA2_OK;
  if (score_rule == CSA2_SCORE_HEADMAX) {
    HeadmaxArgs ha = headmax_args(kv, q, heads, nullptr, 0, scores, nblk_grid);
    ha.nblk_grid = (int32_t)nblk_grid;
    ha.fill_invalid = 1;
    const int64_t tiles = ceil_div(nblk_grid, HM_SCAN_NT);
    headmax_kernel<4, HM_SCAN_NT, false, false>
        <<<dim3(grid_for(tiles, kv->batch, HM_SCAN_GRID), kv->batch), 256, 0, s>>>(ha);
    return launched("headmax scores");
  }
  ScanArgs sa;
  sa.codes = kv->codes; sa.scales = kv->scales; sa.seq_len = kv->seq_len; sa.capacity = kv->capacity;
  sa.limit = kv->max_len;
  sa.q = q; sa.heads = heads; sa.nblk_grid = (int32_t)nblk_grid;
  sa.scores = scores; sa.score_stride = nblk_grid; sa.ctrl = nullptr; sa.hist = nullptr;
  sa.R = 0; sa.fill_invalid = 1; sa.qbar = nullptr;
  dim3 g(grid_for(ceil_div(nblk_grid, BLOCKS_PER_ITER), kv->batch, 512), kv->batch);
  scan_kernel<false><<<g, SCAN_THREADS, 0, s>>>(sa);
  return launched("scores");
}

csa2_status csa2_decode_step(const csa2_step *st, void *stream) {
  t_last_error.clear();
  if (!st) return fail(CSA2_E_ARG, "step is NULL");
  if (!st->caches || st->n_caches < 1 || st->n_caches > CSA2_MAX_CACHES)
    return fail(CSA2_E_ARG, "n_caches %d outside [1, %d]", st->n_caches, CSA2_MAX_CACHES);
  if (!st->layers || st->n_layers < 1) return fail(CSA2_E_ARG, "no layers");
  const int B = st->caches[0].batch;
  int64_t max_len = 0;
  for (int c = 0; c < st->n_caches; ++c) {
    if (csa2_status e = check_kv(&st->caches[c])) return e;
    if (st->caches[c].batch != B) return fail(CSA2_E_ARG, "caches differ in batch");
    if (st->caches[c].max_len > max_len) max_len = st->caches[c].max_len;
  }
  if (st->heads != 16 && st->heads != 32 && st->heads != 64)
    return fail(CSA2_E_SHAPE, "heads must be 16, 32 or 64");
  if (csa2_status e = check_select_args(st->topk, st->pool)) return e;
  if (st->pool > 0 && (!st->pool_out || !aligned(st->pool_out, 4))) return fail(CSA2_E_ARG, "pool > 0 needs pool_out");
  if (st->new_rows && !aligned(st->new_rows, 16)) return fail(CSA2_E_ARG, "new_rows misaligned");
  const int32_t rule = st->score_rule;
  if (rule != CSA2_SCORE_SUM && rule != CSA2_SCORE_HEADMAX)
    return fail(CSA2_E_ARG, "score_rule %d is not CSA2_SCORE_SUM or CSA2_SCORE_HEADMAX", rule);
  // mode pattern: layer 0 Full; Reindex/Reuse use the latest Full cache
  int latest = -1, n_rings = 0;
  for (int l = 0; l < st->n_layers; ++l) {
    const csa2_layer &ly = st->layers[l];
    if (ly.mode != CSA2_FULL && ly.mode != CSA2_REINDEX && ly.mode != CSA2_REUSE)
      return fail(CSA2_E_ARG, "layer %d: bad mode %d", l, ly.mode);
    if (ly.cache < 0 || ly.cache >= st->n_caches) return fail(CSA2_E_ARG, "layer %d: cache %d out of range", l, ly.cache);
    if (ly.mode == CSA2_FULL) latest = ly.cache;
    else if (latest < 0) return fail(CSA2_E_ARG, "layer %d: no earlier Full layer", l);
    else if (ly.cache != latest) return fail(CSA2_E_ARG, "layer %d: must use the latest Full cache %d", l, latest);
    if (!ly.q || !aligned(ly.q, 16) || !ly.out || !aligned(ly.out, 16) || !ly.idx || !aligned(ly.idx, 4))
      return fail(CSA2_E_ARG, "layer %d: q/out/idx missing or misaligned", l);
    if (ly.swa) {
      if (csa2_status e = check_swa(ly.swa, B)) return e;
      if (ly.swa_row && !aligned(ly.swa_row, 16)) return fail(CSA2_E_ARG, "layer %d: swa_row misaligned", l);
      if (ly.swa_row && ++n_rings > CSA2_MAX_SWA_LAYERS)
        return fail(CSA2_E_SHAPE, "more than %d layers append SWA rows", CSA2_MAX_SWA_LAYERS);
      // two appends into one ring would race on its slot and length
      if (ly.swa_row)
        for (int k = 0; k < l; ++k) {
          const csa2_layer &o = st->layers[k];
          if (o.swa && o.swa_row && (o.swa->seq_len == ly.swa->seq_len || o.swa->codes == ly.swa->codes))
            return fail(CSA2_E_ARG, "layers %d and %d append into the same SWA ring", k, l);
        }
    }
  }
  Layout L;
  if (!make_layout(B, st->heads, max_len, st->pool, st->topk, &L)) return fail(CSA2_E_SHAPE, "bad sizes");
  if (csa2_status e = check_ws(st->ws, st->ws_bytes, L)) return e;
  if (csa2_status e = device_ready()) return e;
  hipStream_t s = as_stream(stream);
  if (csa2_status e = ws_ready(st->ws, B, L, s)) return e;

  bool qbar_ready = false;                // layer 0's query sum is in the workspace
  if (st->new_rows || n_rings) {
    // one launch: the Full caches' rows, then every layer's SWA row
    AppendArgs aa;
    memset(&aa, 0, sizeof aa);
    const int nc = st->new_rows ? st->n_caches : 0;
    for (int c = 0; c < nc; ++c) {
      aa.codes[c] = st->caches[c].codes; aa.scales[c] = st->caches[c].scales;
      aa.seq_len[c] = st->caches[c].seq_len; aa.capacity[c] = st->caches[c].capacity;
    }
    SwaRings rr;
    memset(&rr, 0, sizeof rr);
    int nr = 0;
    for (int l = 0; l < st->n_layers; ++l) {
      const csa2_layer &ly = st->layers[l];
      if (!ly.swa || !ly.swa_row) continue;
      rr.codes[nr] = ly.swa->codes; rr.scales[nr] = ly.swa->scales; rr.seq_len[nr] = ly.swa->seq_len;
      rr.rows[nr] = ly.swa_row; rr.slots[nr] = swa_slots(ly.swa);
      ++nr;
    }
    // the first layer (Full) scans all blocks: its query sum rides along
    // (the summed score rule only)
    QbarJob qj{st->layers[0].q, st->heads, at<float>(st->ws, L.qbar)};
    const int slices = rule == CSA2_SCORE_SUM ? QBAR_SLICES : 0;
    if (nc + nr + slices > 0) {
      append_kernel<<<dim3(B, nc + nr + slices), 128, 0, s>>>(aa, rr, st->new_rows, B, nc, nr, qj);
      if (csa2_status e = launched("append")) return e;
    }
    qbar_ready = slices > 0;
  }
  bool pool_built = false;
  const int32_t *prev_idx = nullptr;
  for (int l = 0; l < st->n_layers; ++l) {
    const csa2_layer &ly = st->layers[l];
    const csa2_kv *kv = &st->caches[ly.cache];
    csa2_status e = CSA2_OK;
    if (ly.mode == CSA2_REUSE) {
      if (!prev_idx) return fail(CSA2_E_ARG, "layer %d: Reuse with no earlier selection", l);
      if (prev_idx != ly.idx) {
        const int64_t nidx = (int64_t)B * st->topk;
        copy_idx_kernel<<<(int)ceil_div(nidx, 256), 256, 0, s>>>(prev_idx, ly.idx, nidx);
        e = launched("reuse copy");
      }
    } else if (st->pool > 0 && st->pool <= SEL_CAND_MAX) {
      // the pool's top-k is taken inside the attention kernel: the index
      // kernels stop at the scored candidate list (no hand-off to a single
      // finishing workgroup, no re-read of the selection)
      float *cs = at<float>(st->ws, L.cscores);
      if (!pool_built) {
        e = run_scan_select(kv, ly.q, st->heads, st->pool, st->pool_out, 0, nullptr, st->ws, L, s, cs,
                            qbar_ready && l == 0, rule);
        pool_built = true;
      } else {
        e = run_rescore(kv, ly.q, st->heads, st->pool_out, st->pool, 0, nullptr, cs, st->pool, nullptr, s, rule);
      }
      if (e) return e;
      e = run_attend(kv, ly.q, st->heads, nullptr, st->topk, st->scale, ly.out, st->ws, L, s,
                     st->pool_out, cs, st->pool, ly.idx, ly.swa);
      if (e) return e;
      prev_idx = ly.idx;
      continue;
    } else if (st->pool > 0 && !pool_built) {
      e = run_scan_select(kv, ly.q, st->heads, st->pool, st->pool_out, st->topk, ly.idx, st->ws, L, s,
                          nullptr, qbar_ready && l == 0, rule);
      pool_built = true;
    } else if (st->pool > 0) {
      e = run_rescore(kv, ly.q, st->heads, st->pool_out, st->pool, st->topk, ly.idx,
                      at<float>(st->ws, L.scores), L.score_stride, at<Ctrl>(st->ws, L.ctrl), s, rule);
    } else {
      e = run_scan_select(kv, ly.q, st->heads, st->topk, ly.idx, 0, nullptr, st->ws, L, s, nullptr,
                          qbar_ready && l == 0, rule);
    }
    if (e) return e;
    e = run_attend(kv, ly.q, st->heads, ly.idx, st->topk, st->scale, ly.out, st->ws, L, s, nullptr,
                   nullptr, 0, nullptr, ly.swa);
    if (e) return e;
    prev_idx = ly.idx;
  }
  return CSA2_OK;
}

csa2_status csa2_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
  t_last_error.clear();
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4))
    return fail(CSA2_E_ARG, "read probe: NULL or misaligned pointer");
  if (bytes <= 0 || bytes % 16 != 0) return fail(CSA2_E_ARG, "read probe: bytes %lld not a positive multiple of 16",
                                                 (long long)bytes);
  if (csa2_status st = device_ready()) return st;
  csa2::read_probe_kernel<<<512, 256, 0, as_stream(stream)>>>(static_cast<const u32x4 *>(buf), bytes / 16, sink);
  return launched("read probe");
}

#ifdef CSA2_PHASE_TIMING
// Profiling builds only: copy the phase timestamps to the host.
int csa2_debug_phase_ts(void *host, size_t bytes) {
  if (bytes > sizeof(g_phase_ts)) bytes = sizeof(g_phase_ts);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_ts), bytes, 0, hipMemcpyDeviceToHost);
}
int csa2_debug_phase_clear(void) {
  static unsigned long long zero[4096][TS_SLOTS];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_phase_ts), zero, sizeof(zero), 0, hipMemcpyHostToDevice);
}
#endif

// Device address of this device's scratch array, found once per device
// (with that device current) and zero-filled then on `stream` by a kernel;
// every call leaves the workspace's control words zero again, so later calls
// need no clearing.
static csa2_status noalloc_scratch(void **out, hipStream_t s) {
  static std::mutex mu;
  static void *addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CSA2_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(CSA2_E_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(CSA2_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const int64_t words = (int64_t)(CSA2_NOALLOC_WORKSPACE_BYTES / 4);
    zero_kernel<<<2048, 256, 0, s>>>(static_cast<uint32_t *>(p), words);
    if (csa2_status st = launched("scratch init")) return st;
    addr[dev] = p;
  }
  *out = addr[dev];
  return CSA2_OK;
}

csa2_status csa2_decode_step_noalloc(const csa2_step *st, void *stream) {
  t_last_error.clear();
  if (!st) return fail(CSA2_E_ARG, "step is NULL");
  if (!st->caches || st->n_caches < 1 || st->n_caches > CSA2_MAX_CACHES)
    return fail(CSA2_E_ARG, "n_caches %d outside [1, %d]", st->n_caches, CSA2_MAX_CACHES);
  int64_t max_len = 0;
  for (int c = 0; c < st->n_caches; ++c) {
    if (csa2_status e = check_kv(&st->caches[c])) return e;
    if (st->caches[c].max_len > max_len) max_len = st->caches[c].max_len;
  }
  Layout L;
  if (!make_layout(st->caches[0].batch, st->heads, max_len, st->pool, st->topk, &L))
    return fail(CSA2_E_SHAPE, "bad sizes");
  if (L.total > (size_t)CSA2_NOALLOC_WORKSPACE_BYTES)
    return fail(CSA2_E_WORKSPACE, "this step needs a %zu-byte workspace, more than the %zu-byte scratch of "
                "csa2_decode_step_noalloc (use csa2_decode_step with a workspace)",
                L.total, (size_t)CSA2_NOALLOC_WORKSPACE_BYTES);
  if (csa2_status e = device_ready()) return e;
  void *ws = nullptr;
  if (csa2_status e = noalloc_scratch(&ws, as_stream(stream))) return e;
  csa2_step own = *st;
  own.ws = ws;
  own.ws_bytes = CSA2_NOALLOC_WORKSPACE_BYTES;
  return csa2_decode_step(&own, stream);
}

csa2_status csa2_device_error(int32_t *flags_host, void *stream) {
  t_last_error.clear();
  if (!flags_host) return fail(CSA2_E_ARG, "flags_host is NULL");
  if (csa2_status st = device_ready()) return st;
  hipError_t e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return fail(CSA2_E_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  uint32_t v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_flags), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(CSA2_E_HIP, "read flags: %s", hipGetErrorString(e));
  const uint32_t zero = 0;
  e = hipMemcpyToSymbol(HIP_SYMBOL(g_flags), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(CSA2_E_HIP, "clear flags: %s", hipGetErrorString(e));
  *flags_host = (int32_t)v;
  return CSA2_OK;
}

}  // extern "C"
