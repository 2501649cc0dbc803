// C ABI of the CSA2 gfx950 library: host-side validation, workspace layout, launch
// sequencing and optional per-kernel event timing.  Validation runs before any HIP call,
// so every error path is reachable without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/csa2.h"
#include "csa2_internal.h"

using namespace csa2;

namespace csa2 {
thread_local hipEvent_t g_launch_events[2] = {nullptr, nullptr};

// The device property cache: compute units per device ordinal, each queried once.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCus;
  std::call_once(once[dev], [dev] {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                    hipSuccess && n > 0) ? n : kDefaultCus;
  });
  return cus[dev];
}
}

namespace csa2 {
bool side_create(Side* sd) {
  *sd = Side{};
  const unsigned fl = hipEventDisableTiming | hipEventDisableSystemFence;
  if (hipStreamCreateWithFlags(&sd->s, hipStreamNonBlocking) != hipSuccess) sd->s = nullptr;
  if (sd->s && hipEventCreateWithFlags(&sd->fork, fl) != hipSuccess) sd->fork = nullptr;
  if (sd->fork && hipEventCreateWithFlags(&sd->join, fl) != hipSuccess) sd->join = nullptr;
  if (!sd->join) {                                   // partial failure: release, no side
    if (sd->fork) (void)hipEventDestroy(sd->fork);
    if (sd->s) (void)hipStreamDestroy(sd->s);
    *sd = Side{};
    return false;
  }
  sd->ok = true;
  return true;
}
}  // namespace csa2

namespace {

thread_local std::string g_err;

csa2_status fail(csa2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

constexpr size_t kWsAlign = 256;
size_t round_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// ---------------------------------------------------------------- kernel timing
struct TimedLaunch {
  const char* name;
  hipEvent_t e0, e1;
};
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<TimedLaunch> pending;
  std::vector<std::string> names;
  std::vector<int64_t> launches;
  std::vector<double> ms;
};
Timing g_timing;

hipEvent_t timing_event() {
  if (g_timing.used == g_timing.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_timing.pool.push_back(e);
  }
  return g_timing.pool[g_timing.used++];
}

// Launch `fn` (returning hipError_t, one kernel launch) on `s`; while timing is on, the
// launch itself records a start and a stop event, so the pair brackets the kernel alone.
// With kernel timing off: an event that the next launch records as it completes (set to
// fork the side stream off a kernel without a separate event packet in the stream).
thread_local hipEvent_t g_stop_next = nullptr;
// Set with g_stop_next when the side stream is idle at the fork (the call's first): the
// per-row scoring then forks off all but its last round (score_fork_blocks).
thread_local bool g_fork_early = false;

template <class F>
csa2_status timed(const char* name, hipStream_t s, F&& fn) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (g_timing.on) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    e0 = timing_event();
    e1 = timing_event();
  }
  (void)s;
  if (e0 && e1) {
    csa2::g_launch_events[0] = e0;
    csa2::g_launch_events[1] = e1;
  } else if (g_stop_next) {
    csa2::g_launch_events[1] = g_stop_next;
    g_stop_next = nullptr;
  }
  hipError_t err = fn();
  csa2::g_launch_events[0] = csa2::g_launch_events[1] = nullptr;
  if (err != hipSuccess) return fail(CSA2_ERR_HIP, "%s launch: %s", name, hipGetErrorString(err));
  if (e0 && e1) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.pending.push_back({name, e0, e1});
  }
  return CSA2_OK;
}

// ---------------------------------------------------------------- side stream
// The SWA branch depends only on its own inputs, so it runs on a library-owned stream of
// the current device (default priority), forked from and joined back into the caller's
// stream with events.  Both are capturable, so a caller may record the calls in a graph.
// This is the library's one piece of state besides the device property cache: one side
// stream and event pair per host thread and device, created on first use and kept (a
// pool of one) for the life of the thread.  If creating them fails, whatever was created
// is destroyed and the branch runs on the caller's stream instead.  The events only order
// work between two streams of one device and are never inspected from the host, so they
// skip the system-scope fence on record (its cache write-back measured about 1% of a
// decode step); device-scope visibility comes from the kernels' own completion.
Side* side_for_current_device() {
  thread_local std::map<int, Side> sides;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  Side& sd = sides[dev];
  if (!sd.ok && !side_create(&sd)) return nullptr;
  return &sd;
}

// Make `side` wait for everything issued to `s` so far.
csa2_status fork_to(Side* sd, hipStream_t s) {
  hipError_t e = hipEventRecord(sd->fork, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(sd->s, sd->fork, 0);
  if (e != hipSuccess) return fail(CSA2_ERR_HIP, "side stream fork: %s", hipGetErrorString(e));
  return CSA2_OK;
}

// Make `s` wait for everything issued to the side stream so far.
csa2_status join_from(Side* sd, hipStream_t s) {
  hipError_t e = hipEventRecord(sd->join, sd->s);
  if (e == hipSuccess) e = hipStreamWaitEvent(s, sd->join, 0);
  if (e != hipSuccess) return fail(CSA2_ERR_HIP, "side stream join: %s", hipGetErrorString(e));
  return CSA2_OK;
}

// ---------------------------------------------------------------- validation helpers
#define REQ(ptr, what)                                                    \
  do {                                                                    \
    if (!(ptr)) return fail(CSA2_ERR_NULL, "%s: %s is NULL", fn, what);   \
    if (misaligned(ptr))                                                  \
      return fail(CSA2_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, what); \
  } while (0)

#define FORBID(ptr, what)                                                          \
  do {                                                                             \
    if (ptr) return fail(CSA2_ERR_MODE, "%s: %s must be NULL here", fn, what);     \
  } while (0)

constexpr int64_t kMaxPagesTotal = (int64_t(1) << 25) - 1;   // physical rows fit in int32

// Main-KV row layout: 0 (dense planes) or a multiple of 16 that holds the entry's codes,
// rope and scales (400 bytes, 416 with E4M3 scales), at most CSA2_MAX_ROW_BYTES.
csa2_status check_row_bytes(const char* fn, int32_t row_bytes, int32_t fmt) {
  if (row_bytes == 0) return CSA2_OK;
  const int need = kLatBytes + 2 * kRope + (fmt == CSA2_KV_FP4_E4M3 ? 2 * kScl : kScl);
  if (row_bytes < need || row_bytes > CSA2_MAX_ROW_BYTES || row_bytes % 16 != 0)
    return fail(CSA2_ERR_SHAPE, "%s: row bytes %d must be 0 or a multiple of 16 in [%d, %d]",
                fn, row_bytes, need, CSA2_MAX_ROW_BYTES);
  return CSA2_OK;
}

csa2_status check_paging(const char* fn, int32_t B, int32_t max_pages, int32_t n_pages) {
  if (B < 1) return fail(CSA2_ERR_SHAPE, "%s: B=%d must be >= 1", fn, B);
  if (max_pages < 1 || (int64_t)max_pages * CSA2_PAGE > INT32_MAX)
    return fail(CSA2_ERR_SHAPE, "%s: max_pages=%d out of range", fn, max_pages);
  if (n_pages < 1 || n_pages > kMaxPagesTotal)
    return fail(CSA2_ERR_SHAPE, "%s: n_pages=%d out of range [1, %lld]", fn, n_pages,
                (long long)kMaxPagesTotal);
  return CSA2_OK;
}

// Row-tiled rows long enough select through sampled candidates (see kCandMinKeys).
bool cand_path(int32_t T, int64_t E) {
  return T >= kIdxGemmMinRows && E >= kCandMinKeys && !topk_chunked(T, E);
}

// Keys [T, E]; for the chunked Top-K also row histograms [T, kCkHistWords], per-chunk
// counts [T, chunks], per-row digits [T, 8] and candidate keys and indices [T, E] each.
size_t index_ws_bytes(int32_t T, int32_t max_pages) {
  const int64_t E = (int64_t)max_pages * CSA2_PAGE;
  size_t b = round_up((size_t)T * (size_t)E * sizeof(uint32_t));
  if (topk_chunked(T, E))
    b += round_up((size_t)T * kCkHistWords * sizeof(uint32_t)) +
         round_up((size_t)T * topk_chunks(E) * sizeof(uint32_t)) +
         round_up((size_t)T * 8 * sizeof(uint32_t)) +
         2 * round_up((size_t)T * (size_t)E * sizeof(uint32_t));
  if (T >= kIdxGemmMinRows) b += round_up(1024);   // the row-tiled scoring's store sink
  if (cand_path(T, E)) b += 2 * round_up((size_t)T * sizeof(uint32_t));   // thresholds, flags
  return b;
}

size_t attn_ws_bytes(int32_t T, int32_t H, int32_t K) {
  int S, per;
  attn_plan(T, H, K, &S, &per, device_cus());   // the most splits any plan below uses
  if (S <= 1) return 0;
  return round_up((size_t)T * S * H * CSA2_D_LAT * sizeof(float)) +
         round_up((size_t)T * S * H * sizeof(float));
}

csa2_status check_ws(const char* fn, void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return CSA2_OK;
  if (!ws) return fail(CSA2_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign)
    return fail(CSA2_ERR_WORKSPACE, "%s: workspace must be %zu-byte aligned", fn, kWsAlign);
  if (ws_bytes < need)
    return fail(CSA2_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  return CSA2_OK;
}

// ---------------------------------------------------------------- index + top-k
csa2_status validate_index(const csa2_index_args* a) {
  const char* fn = "csa2_index_topk";
  if (!a) return fail(CSA2_ERR_NULL, "%s: args is NULL", fn);
  if (a->T < 0) return fail(CSA2_ERR_SHAPE, "%s: T=%d < 0", fn, a->T);
  if (a->H_I < 1 || a->H_I > CSA2_MAX_H_I)
    return fail(CSA2_ERR_SHAPE, "%s: H_I=%d outside [1, %d]", fn, a->H_I, CSA2_MAX_H_I);
  if (a->K < 1 || a->K > CSA2_MAX_K)
    return fail(CSA2_ERR_SHAPE, "%s: K=%d outside [1, %d]", fn, a->K, CSA2_MAX_K);
  csa2_status st = check_paging(fn, a->B, a->max_pages, a->n_pages);
  if (st) return st;
  const int64_t E = (int64_t)a->max_pages * CSA2_PAGE;
  if (topk_chunked(a->T, E) && topk_chunks(E) > kCkMaxChunks)
    return fail(CSA2_ERR_UNSUPPORTED, "%s: %d rows of up to %lld entries: at most %d rows "
                "longer than 65536 entries support up to %lld entries", fn, a->T,
                (long long)E, kCkMaxRows, (long long)kCkMaxChunks * kCkKeys);
  if (a->T == 0) return CSA2_OK;
  REQ(a->q_idx, "q_idx");
  REQ(a->w_idx, "w_idx");
  REQ(a->k_idx, "k_idx");
  REQ(a->page_table, "page_table");
  REQ(a->seq_id, "seq_id");
  REQ(a->n_vis, "n_vis");
  REQ(a->idx_out, "idx_out");
  return CSA2_OK;
}

// Indexer scoring, then Top-K; `between` runs after the scoring launch.
// fuse_swa: a small SWA branch of the same rows, run inside the per-row scoring's launch
// (swa_blocks workgroups) instead of on the side stream.
template <class Between>
csa2_status run_index_split(const csa2_index_args* a, void* ws, hipStream_t s, Between&& between,
                            const SwaParams* fuse_swa = nullptr, int swa_blocks = 0) {
  if (a->T == 0) return between();
  const int64_t E = (int64_t)a->max_pages * CSA2_PAGE;
  IdxScoreParams sp;
  sp.T = a->T;
  sp.H_I = a->H_I;
  sp.max_pages = a->max_pages;
  // per-row scoring: 8 pages per wave, or 4 when the rows' 2048-entry chunks would leave
  // the CUs short of four workgroups each (few long rows: twice the waves, each with its
  // next page in flight)
  const int64_t full_blocks = (int64_t)a->T * ((E + kIdxChunk - 1) / kIdxChunk);
  sp.ppw = (full_blocks < 4 * (int64_t)device_cus()) ? 4 : 8;
  sp.chunks = (int)((E + 256 * sp.ppw - 1) / (256 * sp.ppw));
  sp.key_stride = E;
  sp.q_idx = static_cast<const uint16_t*>(a->q_idx);
  sp.w_idx = a->w_idx;
  sp.k_idx = static_cast<const uint16_t*>(a->k_idx);
  sp.page_table = a->page_table;
  sp.seq_id = a->seq_id;
  sp.n_vis = a->n_vis;
  sp.keys = static_cast<uint32_t*>(ws);
  // the chunked Top-K keeps row histograms right after the keys; scoring zeroes them
  const bool chunked = topk_chunked(a->T, E);
  uint32_t* ck = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) +
                                             round_up((size_t)a->T * (size_t)E * sizeof(uint32_t)));
  sp.clear = chunked ? ck : nullptr;
  sp.clear_words = chunked ? a->T * kCkHistWords : 0;
  sp.trash = (a->T >= kIdxGemmMinRows) ? ck : nullptr;   // chunked and row-tiled never meet
  TopkParams tp;
  tp.T = a->T;
  tp.K = a->K;
  tp.key_stride = E;
  tp.keys = sp.keys;
  tp.n_vis = a->n_vis;
  tp.idx_out = a->idx_out;
  tp.ck_hist = tp.ck_counts = tp.ck_sel = tp.ck_ckey = nullptr;
  tp.ck_cidx = nullptr;
  csa2_status st;
  if (cand_path(a->T, E)) {
    // Sampled candidates.  Inside the keys area (written only by the exact path at the
    // end): first the packed sample, then, once the thresholds are known, the candidate
    // counts, keys and indices.  Thresholds and flags sit after the store sink.
    const int G = cand_page_gap(E);
    const int64_t ns = (((E + kPage - 1) / kPage + G - 1) / G) * kPage;
    const int nch = (int)((E + kGemmChunk - 1) / kGemmChunk);
    char* w = static_cast<char*>(ws);
    uint32_t* sample = reinterpret_cast<uint32_t*>(w);
    uint32_t* ccnt = reinterpret_cast<uint32_t*>(w);
    w += round_up((size_t)a->T * nch * sizeof(uint32_t));
    uint32_t* ckey = reinterpret_cast<uint32_t*>(w);
    w += round_up((size_t)a->T * nch * kCandCap * sizeof(uint32_t));
    int32_t* cidx = reinterpret_cast<int32_t*>(w);
    char* w2 = reinterpret_cast<char*>(ck) + round_up(1024);
    uint32_t* thr = reinterpret_cast<uint32_t*>(w2);
    uint32_t* flags = reinterpret_cast<uint32_t*>(w2 + round_up((size_t)a->T * sizeof(uint32_t)));

    // the side branch forks when the candidate scoring ends, so that it runs beside the
    // latency-bound candidate Top-K rather than the scoring (2.239 -> 2.219 ms a prefill
    // step)
    hipEvent_t fork_ev = g_stop_next;
    g_stop_next = nullptr;
    IdxScoreParams s1 = sp;                          // 1: the sample
    s1.gemm_mode = kGemmSample;
    s1.page_gap = G;
    s1.key_stride = ns;
    s1.keys = sample;
    st = timed("idx_sample", s, [&] { return launch_idx_score(s1, s); });
    if (st) return st;
    TopkParams t1 = tp;                              // 2: thresholds
    t1.key_stride = ns;
    t1.keys = sample;
    t1.thr = thr;
    t1.row_flags = flags;
    t1.page_gap = G;
    st = timed("topk_thr", s, [&] { return launch_topk_thr(t1, s); });
    if (st) return st;
    IdxScoreParams s3 = sp;                          // 3: scoring into candidates
    s3.gemm_mode = kGemmCand;
    s3.thr = thr;
    s3.row_flags = flags;
    s3.cand_key = ckey;
    s3.cand_idx = cidx;
    s3.cand_cnt = ccnt;
    s3.n_chunks = nch;
    g_stop_next = fork_ev;
    st = timed("idx_score", s, [&] { return launch_idx_score(s3, s); });
    if (st) return st;
    st = between();
    if (st) return st;
    TopkParams t4 = tp;                              // 4: the exact Top-K of the candidates
    t4.cand_key = ckey;
    t4.cand_idx = cidx;
    t4.cand_cnt = ccnt;
    t4.row_flags = flags;
    t4.n_chunks = nch;
    st = timed("topk", s, [&] { return launch_topk_cand(t4, s); });
    if (st) return st;
    // 5, 6: the exact path for flagged rows only (the other workgroups leave at once)
    IdxScoreParams s5 = sp;
    s5.row_flags = flags;
    st = timed("idx_exact", s, [&] { return launch_idx_score(s5, s); });
    if (st) return st;
    TopkParams t6 = tp;
    t6.row_flags = flags;
    return timed("topk_exact", s, [&] { return launch_topk(t6, s); });
  }
  const int64_t n1 = (g_stop_next && g_fork_early && sp.T < kIdxGemmMinRows)   // per-row kernel
                         ? score_fork_blocks((int64_t)sp.T * sp.chunks, device_cus()) : 0;
  if (fuse_swa && sp.T < kIdxGemmMinRows) {
    st = timed("idx_score", s, [&] { return launch_idx_score_swa(sp, *fuse_swa, swa_blocks, s); });
  } else if (n1 > 0) {
    // the side branch's start latency overlaps the last round of the scoring
    IdxScoreParams a1 = sp, a2 = sp;
    a1.block_end = (int)n1;
    a2.block0 = (int)n1;
    st = timed("idx_score", s, [&] { return launch_idx_score(a1, s); });
    if (!st) st = timed("idx_score", s, [&] { return launch_idx_score(a2, s); });
  } else {
    st = timed("idx_score", s, [&] { return launch_idx_score(sp, s); });
  }
  if (st) return st;
  st = between();
  if (st) return st;
  if (!chunked) return timed("topk", s, [&] { return launch_topk(tp, s); });
  tp.ck_hist = ck;
  char* w = reinterpret_cast<char*>(ck);
  w += round_up((size_t)a->T * kCkHistWords * sizeof(uint32_t));
  tp.ck_counts = reinterpret_cast<uint32_t*>(w);
  w += round_up((size_t)a->T * topk_chunks(E) * sizeof(uint32_t));
  tp.ck_sel = reinterpret_cast<uint32_t*>(w);
  w += round_up((size_t)a->T * 8 * sizeof(uint32_t));
  tp.ck_ckey = reinterpret_cast<uint32_t*>(w);
  w += round_up((size_t)a->T * (size_t)E * sizeof(uint32_t));
  tp.ck_cidx = reinterpret_cast<int32_t*>(w);
  static const char* const names[4] = {"", "topk_ck_hist", "topk_ck_compact", "topk_ck_select"};
  for (int pass = 1; pass < 4; ++pass) {
    st = timed(names[pass], s, [&] { return launch_topk_chunked(tp, pass, s); });
    if (st) return st;
  }
  return CSA2_OK;
}

csa2_status run_index(const csa2_index_args* a, void* ws, hipStream_t s) {
  return run_index_split(a, ws, s, [] { return CSA2_OK; });
}

// ---------------------------------------------------------------- pooled search
// Keys [T, pool_key_stride(K_sel)]: 8 slots per selection.
size_t pool_ws_bytes(int32_t T, int32_t K_sel) {
  return round_up((size_t)T * (size_t)pool_key_stride(K_sel) * sizeof(uint32_t));
}

csa2_status validate_pool(const csa2_pool_args* a) {
  const char* fn = "csa2_index_topk_pool";
  if (!a) return fail(CSA2_ERR_NULL, "%s: args is NULL", fn);
  if (a->K_sel < 1 || a->K_sel > kPoolMaxSel)
    return fail(CSA2_ERR_SHAPE, "%s: K_sel=%d outside [1, %d]", fn, a->K_sel, kPoolMaxSel);
  if (a->ix.K > kPoolMaxK)
    return fail(CSA2_ERR_SHAPE, "%s: K=%d above %d", fn, a->ix.K, kPoolMaxK);
  csa2_status st = validate_index(&a->ix);
  if (st) {
    std::string m = g_err;
    return fail(st, "%s: %s", fn, m.c_str());
  }
  if (a->ix.T > 0) REQ(a->sel, "sel");
  return CSA2_OK;
}

// Scoring of the pool of sel [T, K_sel], then its Top-K; `between` runs after the scoring
// launch.
template <class Between>
csa2_status run_index_pool_split(const csa2_index_args* a, const int32_t* sel, int K_sel,
                                 void* ws, hipStream_t s, Between&& between) {
  if (a->T == 0) return between();
  IdxScoreParams sp;
  sp.T = a->T;
  sp.H_I = a->H_I;
  sp.max_pages = a->max_pages;
  sp.chunks = (K_sel + kPoolSelPerBlock - 1) / kPoolSelPerBlock;
  sp.key_stride = pool_key_stride(K_sel);
  sp.q_idx = static_cast<const uint16_t*>(a->q_idx);
  sp.w_idx = a->w_idx;
  sp.k_idx = static_cast<const uint16_t*>(a->k_idx);
  sp.page_table = a->page_table;
  sp.seq_id = a->seq_id;
  sp.n_vis = a->n_vis;
  sp.keys = static_cast<uint32_t*>(ws);
  sp.clear = nullptr;
  sp.clear_words = 0;
  sp.trash = nullptr;
  sp.pool_sel = sel;
  sp.pool_K = K_sel;
  csa2_status st = timed("idx_pool_score", s, [&] { return launch_idx_score(sp, s); });
  if (st) return st;
  st = between();
  if (st) return st;
  TopkParams tp;
  tp.T = a->T;
  tp.K = a->K;
  tp.key_stride = sp.key_stride;
  tp.keys = sp.keys;
  tp.n_vis = a->n_vis;
  tp.idx_out = a->idx_out;
  tp.ck_hist = tp.ck_counts = tp.ck_sel = tp.ck_ckey = nullptr;
  tp.ck_cidx = nullptr;
  tp.pool_sel = sel;
  tp.pool_K = K_sel;
  return timed("topk_pool", s, [&] { return launch_topk(tp, s); });
}

// ---------------------------------------------------------------- attention
csa2_status validate_attn(const csa2_attn_args* a) {
  const char* fn = "csa2_sparse_attn_fp4";
  if (!a) return fail(CSA2_ERR_NULL, "%s: args is NULL", fn);
  if (a->T < 0) return fail(CSA2_ERR_SHAPE, "%s: T=%d < 0", fn, a->T);
  if (!(a->H == 16 || a->H == 32 || a->H == 64 || a->H == 128))
    return fail(CSA2_ERR_SHAPE, "%s: H=%d must be 16, 32, 64 or 128", fn, a->H);
  if (a->K < 1 || a->K > CSA2_MAX_K)
    return fail(CSA2_ERR_SHAPE, "%s: K=%d outside [1, %d]", fn, a->K, CSA2_MAX_K);
  csa2_status st = check_paging(fn, a->B, a->max_pages, a->n_pages);
  if (st) return st;
  if (!std::isfinite(a->sm_scale)) return fail(CSA2_ERR_SHAPE, "%s: sm_scale not finite", fn);
  if (a->kv_format != CSA2_KV_MXFP4 && a->kv_format != CSA2_KV_FP4_E4M3)
    return fail(CSA2_ERR_UNSUPPORTED, "%s: kv_format=%d is not a known format", fn,
                a->kv_format);
  st = check_row_bytes(fn, a->kv_row_bytes, a->kv_format);
  if (st) return st;
  const bool swa = a->q_swa != nullptr;
  if (swa) {
    if (a->H_kv < 1 || a->H % a->H_kv != 0)
      return fail(CSA2_ERR_SHAPE, "%s: H_kv=%d must divide H=%d", fn, a->H_kv, a->H);
    const int G = a->H / a->H_kv;
    if (!(G == 1 || G == 2 || G == 4 || G == 8))
      return fail(CSA2_ERR_SHAPE, "%s: H/H_kv=%d must be 1, 2, 4 or 8", fn, G);
    if (a->L_swa < 1) return fail(CSA2_ERR_SHAPE, "%s: L_swa=%d < 1", fn, a->L_swa);
    if (!std::isfinite(a->sm_scale_swa))
      return fail(CSA2_ERR_SHAPE, "%s: sm_scale_swa not finite", fn);
  }
  if (a->T == 0) return CSA2_OK;
  REQ(a->q, "q");
  REQ(a->kv_lat, "kv_lat");
  REQ(a->kv_scl, "kv_scl");
  REQ(a->kv_rope, "kv_rope");
  REQ(a->page_table, "page_table");
  REQ(a->seq_id, "seq_id");
  REQ(a->idx, "idx");
  REQ(a->o, "o");
  REQ(a->lse, "lse");
  if (swa) {
    REQ(a->swa_k, "swa_k");
    REQ(a->swa_v, "swa_v");
    REQ(a->swa_start, "swa_start");
    REQ(a->swa_len, "swa_len");
    REQ(a->o_swa, "o_swa");
    REQ(a->lse_swa, "lse_swa");
  } else {
    FORBID(a->swa_k, "swa_k (no q_swa)");
    FORBID(a->swa_v, "swa_v (no q_swa)");
    FORBID(a->swa_start, "swa_start (no q_swa)");
    FORBID(a->swa_len, "swa_len (no q_swa)");
    FORBID(a->o_swa, "o_swa (no q_swa)");
    FORBID(a->lse_swa, "lse_swa (no q_swa)");
  }
  return CSA2_OK;
}

csa2_status run_attn(const csa2_attn_args* a, void* ws, hipStream_t s, bool swa_beside = true) {
  if (a->T == 0) return CSA2_OK;
  // with an SWA branch on persistent workgroups beside it, plan for the CUs they leave
  const int cus = device_cus();
  const int swa_wgs = (a->q_swa && swa_beside) ? swa_persist_wgs(a->T, a->H, a->H_kv, cus) : 0;
  int S, per;
  attn_plan(a->T, a->H, a->K, &S, &per, cus - swa_wgs);
  AttnParams ap;
  ap.T = a->T;
  ap.H = a->H;
  ap.K = a->K;
  ap.max_pages = a->max_pages;
  ap.splits = S;
  ap.per_split = per;
  ap.split_heads = attn_split_heads(a->T, a->H, S, cus - swa_wgs) ? 1 : 0;
  ap.fmt = a->kv_format;
  ap.sm_scale_log2 = a->sm_scale * 1.4426950408889634f;
  ap.q = static_cast<const uint16_t*>(a->q);
  ap.kv_lat = a->kv_lat;
  ap.kv_scl = a->kv_scl;
  ap.kv_rope = static_cast<const uint16_t*>(a->kv_rope);
  const KvStrides ks = kv_strides(a->kv_format, a->kv_row_bytes);
  ap.lat_stride = ks.lat;
  ap.rope_stride = ks.rope;
  ap.scl_stride = ks.scl;
  ap.page_table = a->page_table;
  ap.seq_id = a->seq_id;
  ap.idx = a->idx;
  ap.o = a->o;
  ap.lse = a->lse;
  ap.o_part = nullptr;
  ap.lse_part = nullptr;
  if (S > 1) {
    char* w = static_cast<char*>(ws);
    ap.o_part = reinterpret_cast<float*>(w);
    ap.lse_part = reinterpret_cast<float*>(
        w + round_up((size_t)a->T * S * a->H * CSA2_D_LAT * sizeof(float)));
  }
  csa2_status st = timed("sparse_attn", s, [&] { return launch_sparse_attn(ap, s); });
  if (st) return st;
  if (S > 1) {
    MergeParams mp{a->T, a->H, S, ap.o_part, ap.lse_part, a->o, a->lse};
    st = timed("attn_merge", s, [&] { return launch_attn_merge(mp, s); });
    if (st) return st;
  }
  return CSA2_OK;
}

SwaParams swa_params(const csa2_attn_args* a) {
  SwaParams wp;
  wp.T = a->T;
  wp.H = a->H;
  wp.H_kv = a->H_kv;
  wp.L_swa = a->L_swa;
  wp.sm_scale_log2 = a->sm_scale_swa * 1.4426950408889634f;
  wp.q_swa = static_cast<const uint16_t*>(a->q_swa);
  wp.k = static_cast<const uint16_t*>(a->swa_k);
  wp.v = static_cast<const uint16_t*>(a->swa_v);
  wp.seq_id = a->seq_id;
  wp.start = a->swa_start;
  wp.len = a->swa_len;
  wp.o = a->o_swa;
  wp.lse = a->lse_swa;
  wp.wgs = swa_persist_wgs(a->T, a->H, a->H_kv, device_cus());
  return wp;
}

csa2_status run_swa(const csa2_attn_args* a, hipStream_t s) {
  if (a->T == 0 || !a->q_swa) return CSA2_OK;
  const SwaParams wp = swa_params(a);
  return timed("swa", s, [&] { return launch_swa(wp, s); });
}

// The global branch on `s` and the SWA branches of `a[0..n)` on the side stream (on `s`
// itself while kernel timing is on, or if no side stream could be made).
template <class Global>
csa2_status run_with_swa(const csa2_attn_args* a, int n, hipStream_t s, Global&& global) {
  bool any_swa = false;
  for (int i = 0; i < n; ++i) any_swa |= (a[i].q_swa != nullptr && a[i].T > 0);
  // with per-kernel timing on, the branches run in sequence so that each kernel's
  // events bracket that kernel alone
  Side* sd = (any_swa && !g_timing.on) ? side_for_current_device() : nullptr;
  csa2_status st;
  if (sd) {
    st = fork_to(sd, s);
    if (st) return st;
    for (int i = 0; i < n && !st; ++i) st = run_swa(&a[i], sd->s);
    csa2_status st2 = global();
    csa2_status st3 = join_from(sd, s);
    return st ? st : (st2 ? st2 : st3);
  }
  st = global();
  for (int i = 0; i < n && !st; ++i) st = run_swa(&a[i], s);
  return st;
}

// ---------------------------------------------------------------- layer group
csa2_status validate_group(const csa2_layer_desc* L, int32_t n_layers, const csa2_group_args* g,
                           csa2_index_args* ia, csa2_attn_args* aa) {
  const char* fn = "csa2_layer_group";
  if (!g) return fail(CSA2_ERR_NULL, "%s: group args is NULL", fn);
  if (!L) return fail(CSA2_ERR_NULL, "%s: layer array is NULL", fn);
  if (n_layers < 1) return fail(CSA2_ERR_SHAPE, "%s: n_layers=%d < 1", fn, n_layers);
  if (L[0].mode != CSA2_FULL) return fail(CSA2_ERR_MODE, "%s: layer 0 must be Full", fn);
  for (int i = 0; i < n_layers; ++i) {
    const csa2_layer_desc& d = L[i];
    char what[96];
    if (d.mode != CSA2_FULL && d.mode != CSA2_REINDEX && d.mode != CSA2_REUSE &&
        d.mode != CSA2_REINDEX_POOL)
      return fail(CSA2_ERR_MODE, "%s: layer %d has unknown mode %d", fn, i, d.mode);
    if (d.mode == CSA2_REINDEX_POOL && g->K > kPoolMaxSel)
      return fail(CSA2_ERR_SHAPE, "%s: layer %d searches a pool, which needs K <= %d (K=%d)",
                  fn, i, kPoolMaxSel, g->K);
    const bool own_idx = d.mode != CSA2_REUSE, own_kv = d.mode == CSA2_FULL;
#define LAYER_REQ(field)                                            \
    do {                                                            \
      snprintf(what, sizeof(what), "layer %d " #field, i);          \
      if (g->T > 0) REQ(d.field, what);                             \
    } while (0)
#define LAYER_FORBID(field)                                         \
    do {                                                            \
      snprintf(what, sizeof(what), "layer %d " #field, i);          \
      FORBID(d.field, what);                                        \
    } while (0)
    LAYER_REQ(q);
    LAYER_REQ(o);
    LAYER_REQ(lse);
    if (own_idx) {
      LAYER_REQ(q_idx);
      LAYER_REQ(w_idx);
      LAYER_REQ(k_idx);
      LAYER_REQ(idx_out);
    } else {
      LAYER_FORBID(q_idx);
      LAYER_FORBID(w_idx);
      LAYER_FORBID(k_idx);
      LAYER_FORBID(idx_out);
    }
    if (own_kv) {
      LAYER_REQ(kv_lat);
      LAYER_REQ(kv_scl);
      LAYER_REQ(kv_rope);
    } else {
      LAYER_FORBID(kv_lat);
      LAYER_FORBID(kv_scl);
      LAYER_FORBID(kv_rope);
    }
#undef LAYER_REQ
#undef LAYER_FORBID
  }
  // shapes through the per-op validators (first layer's pointers stand in)
  *ia = csa2_index_args{g->T, g->B, g->H_I, g->K, g->max_pages, g->n_pages, L[0].q_idx,
                        L[0].w_idx, L[0].k_idx, g->page_table, g->seq_id, g->n_vis,
                        L[0].idx_out};
  csa2_status st = validate_index(ia);
  if (st) return st;
  for (int i = 0; i < n_layers; ++i) {
    aa[i] = csa2_attn_args{};
    aa[i].T = g->T;
    aa[i].B = g->B;
    aa[i].H = g->H;
    aa[i].K = g->K;
    aa[i].max_pages = g->max_pages;
    aa[i].n_pages = g->n_pages;
    aa[i].q = L[i].q;
    aa[i].page_table = g->page_table;
    aa[i].seq_id = g->seq_id;
    aa[i].sm_scale = g->sm_scale;
    aa[i].kv_format = g->kv_format;
    aa[i].kv_row_bytes = g->kv_row_bytes;
    aa[i].o = L[i].o;
    aa[i].lse = L[i].lse;
    aa[i].H_kv = g->H_kv;
    aa[i].L_swa = g->L_swa;
    aa[i].q_swa = L[i].q_swa;
    if (L[i].q_swa) {
      aa[i].swa_k = L[i].swa_k;
      aa[i].swa_v = L[i].swa_v;
      aa[i].swa_start = g->swa_start;
      aa[i].swa_len = g->swa_len;
      aa[i].sm_scale_swa = g->sm_scale_swa;
      aa[i].o_swa = L[i].o_swa;
      aa[i].lse_swa = L[i].lse_swa;
    }
    // resolve KV (nearest Full at or before i) and indices (nearest Full/Reindex)
    int kv = i, ix = i;
    while (L[kv].mode != CSA2_FULL) --kv;
    while (L[ix].mode == CSA2_REUSE) --ix;
    aa[i].kv_lat = L[kv].kv_lat;
    aa[i].kv_scl = L[kv].kv_scl;
    aa[i].kv_rope = L[kv].kv_rope;
    aa[i].idx = L[ix].idx_out;
    st = validate_attn(&aa[i]);
    if (st) {
      std::string m = g_err;
      return fail(st, "layer %d: %s", i, m.c_str());
    }
  }
  return CSA2_OK;
}

}  // namespace

extern "C" {

csa2_status csa2_index_topk_pool(const csa2_pool_args* a, void* ws, size_t ws_bytes,
                                 void* stream) {
  csa2_status st = validate_pool(a);
  if (st) return st;
  st = check_ws("csa2_index_topk_pool", ws, ws_bytes,
                a->ix.T ? pool_ws_bytes(a->ix.T, a->K_sel) : 0);
  if (st) return st;
  return run_index_pool_split(&a->ix, a->sel, a->K_sel, ws, static_cast<hipStream_t>(stream),
                              [] { return CSA2_OK; });
}

csa2_status csa2_index_topk(const csa2_index_args* a, void* ws, size_t ws_bytes, void* stream) {
  csa2_status st = validate_index(a);
  if (st) return st;
  st = check_ws("csa2_index_topk", ws, ws_bytes, a->T ? index_ws_bytes(a->T, a->max_pages) : 0);
  if (st) return st;
  return run_index(a, ws, static_cast<hipStream_t>(stream));
}

csa2_status csa2_sparse_attn_fp4(const csa2_attn_args* a, void* ws, size_t ws_bytes,
                                 void* stream) {
  csa2_status st = validate_attn(a);
  if (st) return st;
  st = check_ws("csa2_sparse_attn_fp4", ws, ws_bytes, a->T ? attn_ws_bytes(a->T, a->H, a->K) : 0);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return run_with_swa(a, 1, s, [&] { return run_attn(a, ws, s); });
}

}  // extern "C"

namespace csa2 {
csa2_status layer_group_validate(const csa2_layer_desc* L, int32_t n_layers,
                                 const csa2_group_args* g) {
  if (n_layers > kMaxGroupLayers)
    return fail(CSA2_ERR_SHAPE, "csa2_layer_group: n_layers=%d > %d", n_layers, kMaxGroupLayers);
  csa2_index_args ia;
  csa2_attn_args aa[kMaxGroupLayers];
  return validate_group(L, n_layers, g, &ia, aa);
}

csa2_status layer_group_run(const csa2_layer_desc* L, int32_t n_layers,
                            const csa2_group_args* g, void* ws, size_t ws_bytes,
                            hipStream_t s, Side* side) {
  csa2_index_args ia;
  if (n_layers > kMaxGroupLayers)
    return fail(CSA2_ERR_SHAPE, "csa2_layer_group: n_layers=%d > %d", n_layers, kMaxGroupLayers);
  csa2_attn_args aa[kMaxGroupLayers];
  csa2_status st = validate_group(L, n_layers, g, &ia, aa);
  if (st) return st;
  if (g->T == 0) return CSA2_OK;
  st = check_ws("csa2_layer_group", ws, ws_bytes,
                csa2_workspace_bytes(CSA2_OP_LAYER_GROUP, g));
  if (st) return st;
  // Layer i's SWA branch goes to the side stream once layer i's indexer scoring is queued:
  // both stream from HBM, so SWA overlaps Top-K, attention and the merge instead (forking
  // before the scoring or after Top-K measured slower).
  bool any_swa = false;
  for (int i = 0; i < n_layers; ++i) any_swa |= (aa[i].q_swa != nullptr);
  Side* sd = (any_swa && !g_timing.on) ? side : nullptr;
  csa2_status st_swa = CSA2_OK;
  bool forked = false;
  // The fork event is recorded by the scoring launch itself when there is one (an event
  // record of its own would add a packet, and a gap, between the scoring and Top-K).
  bool armed = false;                                // g_stop_next set for the scoring
  auto swa_now = [&](int i, bool after_launch) -> csa2_status {
    if (!sd) return CSA2_OK;
    if (after_launch && armed && g_stop_next == nullptr) {   // the scoring launch took it
      hipError_t e = hipStreamWaitEvent(sd->s, sd->fork, 0);
      if (e != hipSuccess) return fail(CSA2_ERR_HIP, "side stream fork: %s", hipGetErrorString(e));
    } else {
      g_stop_next = nullptr;
      csa2_status f = fork_to(sd, s);
      if (f) return f;
    }
    forked = true;
    if (!st_swa) st_swa = run_swa(&aa[i], sd->s);
    return CSA2_OK;
  };
  // Under stream capture the fork is an explicit event record (a graph records event
  // nodes, not a kernel's own completion event).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  const bool capturing =
      sd && hipStreamIsCapturing(s, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone;
  bool fused[kMaxGroupLayers] = {};
  for (int i = 0; i < n_layers && !st; ++i) {
    if (L[i].mode != CSA2_REUSE) {
      ia.q_idx = L[i].q_idx;
      ia.w_idx = L[i].w_idx;
      ia.k_idx = L[i].k_idx;
      ia.idx_out = L[i].idx_out;
      // The SWA branch reads its K and V windows (at most L_swa positions, 128 bf16
      // channels per KV head), the scoring 64 bf16 of indexer key per entry.
      const int64_t swa_bytes = (int64_t)aa[i].T * aa[i].L_swa * aa[i].H_kv * 512;
      const int64_t key_bytes = (int64_t)ia.T * ia.max_pages * CSA2_PAGE * 128;
      // A branch of at most a quarter of the scoring's bytes runs inside the per-row
      // scoring's launch: the scoring's own time then covers most of it, and the fork and
      // join events (about 6 us a step) go away (4 x 1M decode 0.0765 -> 0.0723 ms).  Not
      // while kernels are timed one by one.
      fused[i] = !g_timing.on && L[i].mode != CSA2_REINDEX_POOL && aa[i].q_swa != nullptr &&
                 aa[i].T > 0 && aa[i].T < kIdxGemmMinRows && aa[i].H == aa[i].H_kv &&
                 swa_persist_wgs(aa[i].T, aa[i].H, aa[i].H_kv, device_cus()) > 0 &&
                 4 * swa_bytes <= key_bytes;
      armed = sd && !capturing && !fused[i];
      if (armed) g_stop_next = sd->fork;
      // The scoring forks the side branch before its last round when that branch is idle
      // and likely the longer one after the scoring: at least the scoring's bytes.
      // (Measured: the 64 x 128K decode step -3%; a 32 x 256K group, whose side branch
      // reads half the scoring's bytes, +1.5% with the early fork, so there it stays at
      // the scoring's end.)
      g_fork_early = armed && !forked && aa[i].q_swa != nullptr && swa_bytes >= key_bytes;
      if (fused[i]) {
        const SwaParams wp = swa_params(&aa[i]);
        const int blocks = (int)std::min<int64_t>(((int64_t)aa[i].T * aa[i].H_kv + 3) / 4, 1024);
        st = run_index_split(&ia, ws, s, [] { return CSA2_OK; }, &wp, blocks);
      } else if (L[i].mode == CSA2_REINDEX_POOL) {   // the pool of layer 0's (Full) selection
        st = run_index_pool_split(&ia, L[0].idx_out, g->K, ws, s, [&] { return swa_now(i, true); });
      } else {
        st = run_index_split(&ia, ws, s, [&] { return swa_now(i, true); });
      }
      g_stop_next = nullptr;
      g_fork_early = false;
    } else {
      st = swa_now(i, false);
    }
    if (!st) st = run_attn(&aa[i], ws, s, !fused[i]);
  }
  if (forked) {
    csa2_status sj = join_from(sd, s);
    if (!st) st = sj;
  }
  if (!sd)
    for (int i = 0; i < n_layers && !st; ++i)
      if (!fused[i]) st = run_swa(&aa[i], s);
  return st ? st : st_swa;
}

csa2_status set_error(csa2_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace csa2

extern "C" {

csa2_status csa2_layer_group(const csa2_layer_desc* L, int32_t n_layers,
                             const csa2_group_args* g, void* ws, size_t ws_bytes, void* stream) {
  // the side stream is made (once per host thread and device) only when a branch needs it
  csa2_status st = layer_group_validate(L, n_layers, g);
  if (st) return st;
  bool any_swa = false;
  for (int i = 0; i < n_layers; ++i) any_swa |= (L[i].q_swa != nullptr);
  Side* sd = (g->T > 0 && any_swa && !g_timing.on) ? side_for_current_device() : nullptr;
  return layer_group_run(L, n_layers, g, ws, ws_bytes, static_cast<hipStream_t>(stream), sd);
}

csa2_status csa2_mxfp4_quantize(const float* x, int64_t rows, uint8_t* lat, uint8_t* scl,
                                const int64_t* dst_row, int32_t row_bytes, void* stream) {
  const char* fn = "csa2_mxfp4_quantize";
  csa2_status st = check_row_bytes(fn, row_bytes, CSA2_KV_MXFP4);
  if (st) return st;
  if (rows < 0) return fail(CSA2_ERR_SHAPE, "%s: rows=%lld < 0", fn, (long long)rows);
  if (rows > (int64_t)0xffffffff * 4)
    return fail(CSA2_ERR_SHAPE, "%s: rows=%lld too large", fn, (long long)rows);
  if (rows == 0) return CSA2_OK;
  REQ(x, "x");
  REQ(lat, "lat");
  REQ(scl, "scl");
  if (dst_row && misaligned(dst_row))
    return fail(CSA2_ERR_ALIGN, "%s: dst_row is not 16-byte aligned", fn);
  const KvStrides ks = kv_strides(CSA2_KV_MXFP4, row_bytes);
  QuantParams p{rows, x, lat, scl, dst_row, ks.lat, ks.scl};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed("mxfp4_quantize", s, [&] { return launch_quantize(p, s); });
}

csa2_status csa2_kv_append(const csa2_append_args* a, void* stream) {
  const char* fn = "csa2_kv_append";
  if (!a) return fail(CSA2_ERR_NULL, "%s: args is NULL", fn);
  if (a->n < 0) return fail(CSA2_ERR_SHAPE, "%s: n=%lld < 0", fn, (long long)a->n);
  if (a->n > (int64_t)0xffffffff * 4)
    return fail(CSA2_ERR_SHAPE, "%s: n=%lld too large", fn, (long long)a->n);
  if ((a->c_idx != nullptr) != (a->z_idx != nullptr) ||
      (a->c_idx != nullptr) != (a->k_idx != nullptr))
    return fail(CSA2_ERR_MODE, "%s: c_idx, z_idx and k_idx must be all set or all NULL", fn);
  csa2_status st = check_row_bytes(fn, a->kv_row_bytes, CSA2_KV_MXFP4);
  if (st) return st;
  if (a->n == 0) return CSA2_OK;
  REQ(a->c, "c");
  REQ(a->z, "z");
  REQ(a->kv_lat, "kv_lat");
  REQ(a->kv_scl, "kv_scl");
  REQ(a->kv_rope, "kv_rope");
  if (a->c_idx) {
    REQ(a->c_idx, "c_idx");
    REQ(a->z_idx, "z_idx");
    REQ(a->k_idx, "k_idx");
  }
  if (a->dst_row && misaligned(a->dst_row))
    return fail(CSA2_ERR_ALIGN, "%s: dst_row is not 16-byte aligned", fn);
  const KvStrides ks = kv_strides(CSA2_KV_MXFP4, a->kv_row_bytes);
  AppendParams p{a->n, a->c, a->z, a->c_idx, a->z_idx, a->dst_row, a->kv_lat, a->kv_scl,
                 static_cast<uint16_t*>(a->kv_rope), static_cast<uint16_t*>(a->k_idx),
                 ks.lat, ks.scl, ks.rope};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed("kv_append", s, [&] { return launch_kv_append(p, s); });
}

csa2_status csa2_fp4e4m3_quantize(const float* x, int64_t rows, uint8_t* lat, uint8_t* scl,
                                  const int64_t* dst_row, int32_t row_bytes, void* stream) {
  const char* fn = "csa2_fp4e4m3_quantize";
  csa2_status st = check_row_bytes(fn, row_bytes, CSA2_KV_FP4_E4M3);
  if (st) return st;
  if (rows < 0) return fail(CSA2_ERR_SHAPE, "%s: rows=%lld < 0", fn, (long long)rows);
  if (rows > (int64_t)0xffffffff * 4)
    return fail(CSA2_ERR_SHAPE, "%s: rows=%lld too large", fn, (long long)rows);
  if (rows == 0) return CSA2_OK;
  REQ(x, "x");
  REQ(lat, "lat");
  REQ(scl, "scl");
  if (dst_row && misaligned(dst_row))
    return fail(CSA2_ERR_ALIGN, "%s: dst_row is not 16-byte aligned", fn);
  const KvStrides ks = kv_strides(CSA2_KV_FP4_E4M3, row_bytes);
  QuantParams p{rows, x, lat, scl, dst_row, ks.lat, ks.scl};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed("fp4e4m3_quantize", s, [&] { return launch_fp4e4m3_quantize(p, s); });
}

size_t csa2_workspace_bytes(int32_t op, const void* args) {
  if (!args) return 0;
  switch (op) {
    case CSA2_OP_INDEX_TOPK: {
      const csa2_index_args* a = static_cast<const csa2_index_args*>(args);
      if (a->T <= 0 || a->max_pages <= 0) return 0;
      return index_ws_bytes(a->T, a->max_pages);
    }
    case CSA2_OP_SPARSE_ATTN: {
      const csa2_attn_args* a = static_cast<const csa2_attn_args*>(args);
      if (a->T <= 0 || a->K <= 0 || a->H <= 0) return 0;
      return attn_ws_bytes(a->T, a->H, a->K);
    }
    case CSA2_OP_LAYER_GROUP: {
      const csa2_group_args* g = static_cast<const csa2_group_args*>(args);
      if (g->T <= 0 || g->max_pages <= 0 || g->K <= 0 || g->H <= 0) return 0;
      const size_t a = index_ws_bytes(g->T, g->max_pages);
      const size_t b = attn_ws_bytes(g->T, g->H, g->K);
      const size_t c = g->K <= kPoolMaxSel ? pool_ws_bytes(g->T, g->K) : 0;   // pooled layers
      return std::max(a, std::max(b, c));
    }
    case CSA2_OP_INDEX_TOPK_POOL: {
      const csa2_pool_args* a = static_cast<const csa2_pool_args*>(args);
      if (a->ix.T <= 0 || a->K_sel <= 0) return 0;
      return pool_ws_bytes(a->ix.T, a->K_sel);
    }
    default:
      return 0;
  }
}

const char* csa2_last_error(void) { return g_err.c_str(); }

const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_ERR_NULL: return "CSA2_ERR_NULL";
    case CSA2_ERR_SHAPE: return "CSA2_ERR_SHAPE";
    case CSA2_ERR_ALIGN: return "CSA2_ERR_ALIGN";
    case CSA2_ERR_MODE: return "CSA2_ERR_MODE";
    case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE";
    case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED";
    case CSA2_ERR_HIP: return "CSA2_ERR_HIP";
  }
  return "CSA2_ERR_UNKNOWN";
}

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

int32_t csa2_plan_cus(void) { return device_cus(); }

csa2_status csa2_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  return CSA2_OK;
}

int32_t csa2_timing_read(char* names_64, int64_t* launches, double* total_ms, int32_t max) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (const TimedLaunch& tl : g_timing.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(tl.e1) != hipSuccess) continue;
    if (hipEventElapsedTime(&ms, tl.e0, tl.e1) != hipSuccess) continue;
    size_t k = 0;
    while (k < g_timing.names.size() && g_timing.names[k] != tl.name) ++k;
    if (k == g_timing.names.size()) {
      g_timing.names.emplace_back(tl.name);
      g_timing.launches.push_back(0);
      g_timing.ms.push_back(0.0);
    }
    g_timing.launches[k] += 1;
    g_timing.ms[k] += ms;
  }
  g_timing.pending.clear();
  g_timing.used = 0;
  int32_t n = 0;
  for (size_t k = 0; k < g_timing.names.size() && n < max; ++k, ++n) {
    if (names_64) {
      memset(names_64 + 64 * n, 0, 64);
      strncpy(names_64 + 64 * n, g_timing.names[k].c_str(), 63);
    }
    if (launches) launches[n] = g_timing.launches[k];
    if (total_ms) total_ms[n] = g_timing.ms[k];
  }
  g_timing.names.clear();
  g_timing.launches.clear();
  g_timing.ms.clear();
  return n;
}

}  // extern "C"
