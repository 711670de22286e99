// C-ABI layer: argument checks, workspace layout and kernel dispatch.
// Declarations and the contract of every entry point are in include/misa.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "misa.h"
#include "misa_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_err[0] = '\0';
  return MISA_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Checks shared by the entry points that read q, w, k.
int32_t check_common(const char* fn, const void* q, const float* w, const void* k, const int32_t* q_seq,
                     const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax) {
  if (T < 0) return fail(MISA_ERR_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (!(d == 32 || d == 64 || d == 128 || d == 256))
    return fail(MISA_ERR_ARG, "%s: d = %d not in {32, 64, 128, 256}", fn, d);
  if (H < 1 || H > 64) return fail(MISA_ERR_ARG, "%s: H = %d not in [1, 64]", fn, H);
  if (nseq < 1) return fail(MISA_ERR_ARG, "%s: nseq = %lld < 1", fn, (long long)nseq);
  if (Lmax < 1 || Lmax >= (int64_t(1) << 31)) return fail(MISA_ERR_ARG, "%s: Lmax = %lld out of range", fn, (long long)Lmax);
  if (T > 0 && (!q || !w || !k || !q_seq || !q_len)) return fail(MISA_ERR_ARG, "%s: null input pointer", fn);
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(MISA_ERR_ALIGN, "%s: q and k must be 16-byte aligned", fn);
  if (!aligned(w, 4) || !aligned(q_seq, 4) || !aligned(q_len, 4))
    return fail(MISA_ERR_ALIGN, "%s: w, q_seq, q_len must be 4-byte aligned", fn);
  return MISA_OK;
}

int32_t check_ws(const char* fn, void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MISA_OK;
  if (!ws || ws_bytes < need)
    return fail(MISA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
  if (!aligned(ws, kAlign)) return fail(MISA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  return MISA_OK;
}

bool wide_tiles(int64_t T, int64_t nseq) { return T >= 64 && T >= 8 * nseq; }
// several queries per sequence on average, too few for wide tiles: a decode step
// over consecutive positions (multi-token prediction) shares each key pass
bool few_tiles(int64_t T, int64_t nseq) { return !wide_tiles(T, nseq) && T >= 2 * nseq; }

// Workspace of the block filter: the block score rows and the block counts.
size_t block_filter_ws_bytes(int64_t T, int64_t Lmax, int32_t B) {
  return round_up((size_t)T * (size_t)(Lmax / B) * sizeof(float)) + round_up((size_t)T * sizeof(int32_t));
}

// Workspace of the proxy queries (sized for d up to 256), weights, group
// sequences and prefixes, and the groups' candidate rows.
size_t pivot_head_bytes(int64_t ng, int32_t H, int32_t kc) {
  return round_up((size_t)ng * H * 256 * 2) + round_up((size_t)ng * H * 4) + 2 * round_up((size_t)ng * 4) +
         round_up((size_t)ng * (size_t)kc * 4);
}

// Scoring + selection keeps the fp32 score rows of at most this many bytes of
// queries at a time: a larger batch (a long causal prefill) is scored and
// selected in consecutive slabs of queries that reuse one slab of rows, so that
// the workspace grows with the row length, not with the batch times the row length.
#ifndef MISA_SCORE_SLAB_BYTES
#define MISA_SCORE_SLAB_BYTES (1ull << 30)
#endif
constexpr size_t kScoreSlabBytes = MISA_SCORE_SLAB_BYTES;

// Queries per slab for rows of max_len scores (the whole batch when it fits).
int64_t slab_rows(int64_t T, int64_t max_len) {
  const int64_t per = max_len > 0 ? (int64_t)(kScoreSlabBytes / ((size_t)max_len * sizeof(float))) : T;
  const int64_t r = per < 1 ? 1 : per;
  return T < r ? T : r;
}

// Workspace of scoring + selection over rows of at most max_len: the fp32 score
// rows of one slab of queries, then (for few long rows) the split top-k's state.
size_t select_ws_bytes(int64_t T, int64_t max_len) {
  const int64_t S = slab_rows(T, max_len);
  size_t b = round_up((size_t)S * (size_t)max_len * sizeof(float));
  if (misa::use_split_topk(S, max_len, true)) b += round_up(misa::split_topk_ws_bytes(S, max_len));
  return b;
}

// Decode batches of at most this many queries take the fused pipeline below
// (larger ones, and every prefill or multi-token batch, take the separate
// calls, whose score rows are bounded by the query slabs).
constexpr int64_t kFusedMaxRows = 4096;

// Workspace of the fused decode pipeline (misa_indexer / misa_hier_indexer):
// router partials and partial-block dots, the coarse score rows and their split
// top-k state, and for MISA† the candidate list, its dense scores and their
// split top-k state, and the dense scores of the coarse members of the
// one-launch MISA† selection.
struct FusedLayout {
  size_t bytes = 0;
  int nchunk_r = 1, chunk_blocks = 1;
  float* partial = nullptr;
  float* xtail = nullptr;
  float* scores = nullptr;
  misa::SplitTopkWs sw{};
  int32_t* cand = nullptr;
  float* rr_scores = nullptr;
  misa::SplitTopkWs rw{};
  float* mscore = nullptr;
};

FusedLayout fused_layout(int64_t T, int H, int64_t Lmax, int B, int64_t kc, void* base) {
  FusedLayout f;
  (void)misa::route_partial_floats(T, H, Lmax, B, &f.nchunk_r, &f.chunk_blocks);
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* r = p ? p + off : nullptr;
    off += round_up(bytes);
    return r;
  };
  f.partial = reinterpret_cast<float*>(take((size_t)T * f.nchunk_r * H * 4));
  f.xtail = reinterpret_cast<float*>(take((size_t)T * H * 4));
  f.scores = reinterpret_cast<float*>(take((size_t)T * Lmax * 4));
  char* sw = take(misa::split_topk_ws_bytes(T, Lmax));
  if (p) f.sw = misa::split_topk_carve(sw, T, Lmax);
  if (kc > 0) {
    f.cand = reinterpret_cast<int32_t*>(take((size_t)T * kc * 4));
    f.rr_scores = reinterpret_cast<float*>(take((size_t)T * kc * 4));
    char* rw = take(misa::split_topk_ws_bytes(T, kc));
    if (p) f.rw = misa::split_topk_carve(rw, T, kc);
    if (kc <= 8192) f.mscore = reinterpret_cast<float*>(take((size_t)T * Lmax * 4));
  }
  f.bytes = off;
  return f;
}

// ---------------------------------------------------------------- timing
// Event timing for measurement tools, registered per stream: only launches on
// a stream whose timing was begun are bracketed, and the launch hooks of every
// other call return after one atomic load while no stream is being timed.
struct TimingEntry {
  hipStream_t stream = nullptr;
  int kid = 0;
  int cap = 0;
  int n = 0;
  std::vector<hipEvent_t> ev;
};
struct Timing {
  std::mutex mu;
  std::atomic<int> active{0};   // entries registered (guarded writes, lock-free reads)
  std::vector<TimingEntry> entries;
};
Timing g_timing;

// The entry of stream st timing kernel class kid with room left (mu held).
TimingEntry* timing_entry(int kid, hipStream_t st) {
  for (TimingEntry& e : g_timing.entries)
    if (e.stream == st) return (e.kid == kid && e.n < e.cap) ? &e : nullptr;
  return nullptr;
}

void timing_release(TimingEntry& e) {
  for (hipEvent_t ev : e.ev)
    if (ev) (void)hipEventDestroy(ev);
  e.ev.clear();
}

}  // namespace

namespace misa {
void timing_before(int kid, hipStream_t st) {
  if (g_timing.active.load(std::memory_order_acquire) == 0) return;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (TimingEntry* e = timing_entry(kid, st)) (void)hipEventRecord(e->ev[2 * e->n], st);
}
void timing_after(int kid, hipStream_t st) {
  if (g_timing.active.load(std::memory_order_acquire) == 0) return;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (TimingEntry* e = timing_entry(kid, st)) {
    (void)hipEventRecord(e->ev[2 * e->n + 1], st);
    ++e->n;
  }
}
bool timing_take(int kid, hipStream_t st, hipEvent_t& start, hipEvent_t& stop) {
  if (g_timing.active.load(std::memory_order_acquire) == 0) return false;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  TimingEntry* e = timing_entry(kid, st);
  if (!e) return false;
  start = e->ev[2 * e->n];
  stop = e->ev[2 * e->n + 1];
  ++e->n;
  return true;
}
}  // namespace misa

namespace {

// ---------------------------------------------------------------- library-owned scratch
// Device memory of the allocation-free entry point: one array per GPU (each
// device holds its own copy while the library is loaded). Host code never
// passes the array's name to a kernel or a copy (on the host it only stands in
// for the symbol); it uses the device address that hipGetSymbolAddress returns
// for the GPU in question, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[MISA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the scratch array on the device of stream st.
int32_t scratch_of_stream(const char* fn, hipStream_t st, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(MISA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  int dev = cur;
  if (st) {
    e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return fail(MISA_ERR_HIP, "%s: hipStreamGetDevice: %s", fn, hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(MISA_ERR_ARG, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(MISA_ERR_HIP, "%s: hipSetDevice(%d): %s", fn, dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return fail(MISA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MISA_OK;
}

}  // namespace

extern "C" {

int32_t misa_version(void) { return 100; }

const char* misa_status_string(int32_t code) {
  switch (code) {
    case MISA_OK: return "MISA_OK";
    case MISA_ERR_ARG: return "MISA_ERR_ARG";
    case MISA_ERR_ALIGN: return "MISA_ERR_ALIGN";
    case MISA_ERR_WORKSPACE: return "MISA_ERR_WORKSPACE";
    case MISA_ERR_HIP: return "MISA_ERR_HIP";
  }
  return "MISA_ERR_UNKNOWN";
}

const char* misa_last_error(void) { return g_err; }

size_t misa_workspace_bytes(int32_t op, int64_t T, int32_t H, int64_t Lmax, int32_t B, int32_t topk, int32_t kc) {
  (void)topk;
  if (T <= 0) return 0;
  switch (op) {
    case MISA_OP_ROUTE: {
      if (B < 1 || H < 1) return 0;
      int nchunk, cb;
      return round_up(misa::route_partial_floats(T, H, Lmax, B, &nchunk, &cb) * sizeof(float));
    }
    case MISA_OP_SCORE_TOPK:
    case MISA_OP_DSA_DENSE:
      return select_ws_bytes(T, Lmax);
    case MISA_OP_HIER_RERANK:
      return select_ws_bytes(T, kc > 0 ? kc : 0);
    case MISA_OP_BLOCK_FILTER:
      if (B < 1) return 0;
      return block_filter_ws_bytes(T, Lmax, B);
    case MISA_OP_BLOCK_INDEXER: {
      if (B < 1 || H < 1 || kc < 1) return 0;
      const int64_t nc = ((int64_t)kc + 1) * B;
      const size_t fs = block_filter_ws_bytes(T, Lmax, B), ss = select_ws_bytes(T, nc);
      return misa_workspace_bytes(MISA_OP_ROUTE, T, H, Lmax, B, 0, 0) + round_up((size_t)T * H * 4) +
             round_up((size_t)T * (size_t)kc * 4) + round_up((size_t)T * (size_t)nc * 4) + (fs > ss ? fs : ss);
    }
    case MISA_OP_PIVOT_INDEXER: {
      if (B < 1 || H < 1 || kc < 1) return 0;
      const int64_t ng = (T + B - 1) / B;
      const size_t sa = select_ws_bytes(ng, Lmax), sb = select_ws_bytes(T, kc);
      return pivot_head_bytes(ng, H, kc) + round_up((size_t)T * (size_t)kc * 4) + (sa > sb ? sa : sb);
    }
    case MISA_OP_INDEXER:
    case MISA_OP_HIER_INDEXER: {
      if (B < 1 || H < 1) return 0;
      const bool hier = op == MISA_OP_HIER_INDEXER;
      // the fused layout holds score rows for the whole batch: only batches that
      // may take the fused pipeline (at most kFusedMaxRows queries) size it
      const size_t fb = T <= kFusedMaxRows ? fused_layout(T, H, Lmax, B, hier ? kc : 0, nullptr).bytes : 0;
      size_t sep = misa_workspace_bytes(MISA_OP_ROUTE, T, H, Lmax, B, 0, 0) + round_up((size_t)T * H * 4);
      size_t sc = misa_workspace_bytes(MISA_OP_SCORE_TOPK, T, H, Lmax, B, hier ? kc : topk, 0);
      if (hier) sc += round_up((size_t)T * (size_t)kc * 4) + misa_workspace_bytes(MISA_OP_HIER_RERANK, T, H, Lmax, B, topk, kc);
      sep += sc;
      return fb > sep ? fb : sep;
    }
  }
  return 0;
}

int32_t misa_pool_keys(const void* k, int64_t nseq, int64_t Lmax, int32_t d, int32_t B, float* kbar, void* stream) {
  const char* fn = "misa_pool_keys";
  if (!(d == 32 || d == 64 || d == 128 || d == 256)) return fail(MISA_ERR_ARG, "%s: d = %d not in {32, 64, 128, 256}", fn, d);
  if (nseq < 0) return fail(MISA_ERR_ARG, "%s: nseq < 0", fn);
  if (Lmax < 1 || Lmax >= (int64_t(1) << 31)) return fail(MISA_ERR_ARG, "%s: Lmax out of range", fn);
  if (B < 1 || B > Lmax) return fail(MISA_ERR_ARG, "%s: B = %d not in [1, Lmax]", fn, B);
  if (nseq == 0) return ok();
  if (!k || !kbar) return fail(MISA_ERR_ARG, "%s: null pointer", fn);
  if (!aligned(k, 16) || !aligned(kbar, 16)) return fail(MISA_ERR_ALIGN, "%s: k and kbar must be 16-byte aligned", fn);
  hipStream_t st = (hipStream_t)stream;
  misa::timing_before(misa::KID_POOL, st);
  hipError_t e = misa::launch_pool(static_cast<const uint16_t*>(k), nseq, Lmax, d, B, kbar, st);
  misa::timing_after(misa::KID_POOL, st);
  return hip_status(e, fn);
}

int32_t misa_pool_update(const void* k, int64_t nseq, int64_t Lmax, int32_t d, int32_t B, const int32_t* prev_len,
                         const int32_t* new_len, int32_t max_new, float* kbar, void* stream) {
  const char* fn = "misa_pool_update";
  if (!(d == 32 || d == 64 || d == 128 || d == 256)) return fail(MISA_ERR_ARG, "%s: d = %d not in {32, 64, 128, 256}", fn, d);
  if (nseq < 0) return fail(MISA_ERR_ARG, "%s: nseq < 0", fn);
  if (Lmax < 1 || Lmax >= (int64_t(1) << 31)) return fail(MISA_ERR_ARG, "%s: Lmax out of range", fn);
  if (B < 1 || B > Lmax) return fail(MISA_ERR_ARG, "%s: B = %d not in [1, Lmax]", fn, B);
  if (max_new < 0 || max_new > Lmax) return fail(MISA_ERR_ARG, "%s: max_new = %d not in [0, Lmax]", fn, max_new);
  if (nseq == 0) return ok();
  if (!k || !kbar || !prev_len || !new_len) return fail(MISA_ERR_ARG, "%s: null pointer", fn);
  if (!aligned(k, 16) || !aligned(kbar, 16)) return fail(MISA_ERR_ALIGN, "%s: k and kbar must be 16-byte aligned", fn);
  if (!aligned(prev_len, 4) || !aligned(new_len, 4))
    return fail(MISA_ERR_ALIGN, "%s: prev_len/new_len must be 4-byte aligned", fn);
  if (nseq * (int64_t)(max_new / B + 1) >= (int64_t(1) << 33)) return fail(MISA_ERR_ARG, "%s: grid too large", fn);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = misa::launch_pool_update(static_cast<const uint16_t*>(k), nseq, Lmax, d, B, prev_len, new_len,
                                          max_new, kbar, st);
  return hip_status(e, fn);
}

int32_t misa_route(const void* q, const float* w, const void* k, const float* kbar, const int32_t* q_seq,
                   const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax, int32_t B,
                   int32_t h, int32_t* heads, float* router_key, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "misa_route";
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  if (B < 1 || B > Lmax) return fail(MISA_ERR_ARG, "%s: B = %d not in [1, Lmax]", fn, B);
  if (h < 1 || h > H) return fail(MISA_ERR_ARG, "%s: h = %d not in [1, H = %d]", fn, h, H);
  if (T == 0) return ok();
  if (!kbar || !heads) return fail(MISA_ERR_ARG, "%s: null kbar or heads", fn);
  if (!aligned(kbar, 16) || !aligned(heads, 4) || !aligned(router_key, 4))
    return fail(MISA_ERR_ALIGN, "%s: kbar must be 16-byte aligned, heads/router_key 4-byte", fn);
  misa::RouteArgs a{};
  const size_t nfl = misa::route_partial_floats(T, H, Lmax, B, &a.nchunk, &a.chunk_blocks);
  rc = check_ws(fn, ws, ws_bytes, round_up(nfl * sizeof(float)));
  if (rc) return rc;
  a.q = static_cast<const uint16_t*>(q);
  a.w = w;
  a.k = static_cast<const uint16_t*>(k);
  a.kbar = kbar;
  a.q_seq = q_seq;
  a.q_len = q_len;
  a.T = T;
  a.H = H;
  a.nseq = nseq;
  a.Lmax = Lmax;
  a.B = B;
  a.h = h;
  a.heads = heads;
  a.router_key = router_key;
  a.partial = static_cast<float*>(ws);
  a.counter = nullptr;
  hipStream_t st = (hipStream_t)stream;
  misa::timing_before(misa::KID_ROUTE, st);
  hipError_t e = misa::launch_route(a, d, st);
  misa::timing_after(misa::KID_ROUTE, st);
  return hip_status(e, fn);
}

namespace {

// Scoring (routed / dense / gathered) into `scores`, then top-k.
int32_t score_and_select(const char* fn, const void* q, const float* w, const void* k, const int32_t* heads,
                         int32_t hh, const int32_t* cand, int32_t kc, const int32_t* q_seq, const int32_t* q_len,
                         int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax, int32_t topk, int32_t* idx,
                         float* score, float* scores, int64_t stride, hipStream_t st) {
  const int64_t S = slab_rows(T, stride);
  if (idx && S < T) {   // (without a selection the rows themselves are the output: no slabs)
    // consecutive slabs of queries, each scored into the same rows and selected
    // before the next one overwrites them (stream order); every pointer that is
    // indexed by the query moves with the slab
    for (int64_t t0 = 0; t0 < T; t0 += S) {
      const int64_t n = T - t0 < S ? T - t0 : S;
      const int32_t rc = score_and_select(
          fn, static_cast<const uint16_t*>(q) + t0 * H * d, w + t0 * H, k, heads ? heads + t0 * hh : nullptr, hh,
          cand ? cand + t0 * kc : nullptr, kc, q_seq + t0, q_len + t0, n, H, d, nseq, Lmax, topk,
          idx ? idx + t0 * topk : nullptr, score ? score + t0 * topk : nullptr, scores, stride, st);
      if (rc) return rc;
    }
    return ok();
  }
  misa::ScoreArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.w = w;
  a.k = static_cast<const uint16_t*>(k);
  a.heads = heads;
  a.hh = hh;
  a.q_seq = q_seq;
  a.q_len = q_len;
  a.cand = cand;
  a.kc = kc;
  a.T = T;
  a.H = H;
  a.nseq = nseq;
  a.Lmax = Lmax;
  a.out = scores;
  a.out_stride = stride;
  a.chunk = 0;
  a.hist = nullptr;
  const bool gather = cand != nullptr;
  const int64_t max_len = gather ? kc : Lmax;
  const bool wide = !gather && wide_tiles(T, nseq);
  const bool few = !gather && few_tiles(T, nseq);
  const bool split = idx && misa::use_split_topk(T, max_len, !gather && !wide && !few);
  misa::SplitTopkWs sw{};
  hipError_t e = hipSuccess;
  if (split) {
    void* base = reinterpret_cast<char*>(scores) + round_up((size_t)T * (size_t)stride * sizeof(float));
    sw = misa::split_topk_carve(base, T, max_len);
    e = misa::launch_zero(sw.hist, misa::split_topk_zero_words(T), st);
    if (e != hipSuccess) return hip_status(e, fn);
    if (!wide && !few) a.hist = sw.hist;   // the decode scoring kernel builds the level-1 histogram
  }
  e = misa::launch_score(a, d, gather, wide, max_len, st, few);   // timed by the launch itself
  if (e != hipSuccess) return hip_status(e, fn);
  if (!idx) return ok();
  misa::TopkArgs b{};
  b.scores = scores;
  b.stride = stride;
  b.q_seq = q_seq;
  b.q_len = q_len;
  b.nseq = nseq;
  b.Lmax = Lmax;
  b.imap = cand;
  b.kc = kc;
  b.T = T;
  b.k = topk;
  b.idx = idx;
  b.score = score;
  misa::timing_before(misa::KID_TOPK, st);
  e = split ? misa::launch_topk_split(b, sw, a.hist != nullptr, st) : misa::launch_topk(b, st);
  misa::timing_after(misa::KID_TOPK, st);
  return hip_status(e, fn);
}

int32_t check_outputs(const char* fn, int32_t topk, const int32_t* idx, const float* score) {
  if (topk < 1) return fail(MISA_ERR_ARG, "%s: topk = %d < 1", fn, topk);
  if (!idx) return fail(MISA_ERR_ARG, "%s: null idx", fn);
  if (!aligned(idx, 4) || !aligned(score, 4)) return fail(MISA_ERR_ALIGN, "%s: idx/score must be 4-byte aligned", fn);
  return MISA_OK;
}

}  // namespace

int32_t misa_score_topk(const void* q, const float* w, const void* k, const int32_t* heads, int32_t h,
                        const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq,
                        int64_t Lmax, int32_t topk, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                        void* stream) {
  const char* fn = "misa_score_topk";
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  if (h < 1 || h > H) return fail(MISA_ERR_ARG, "%s: h = %d not in [1, H = %d]", fn, h, H);
  if (topk < 1) return fail(MISA_ERR_ARG, "%s: topk = %d < 1", fn, topk);
  if (T == 0) return ok();
  if (!heads) return fail(MISA_ERR_ARG, "%s: null heads", fn);
  if (!aligned(heads, 4)) return fail(MISA_ERR_ALIGN, "%s: heads must be 4-byte aligned", fn);
  rc = check_outputs(fn, topk, idx, score);
  if (rc) return rc;
  rc = check_ws(fn, ws, ws_bytes, misa_workspace_bytes(MISA_OP_SCORE_TOPK, T, H, Lmax, 0, topk, 0));
  if (rc) return rc;
  return score_and_select(fn, q, w, k, heads, h, nullptr, 0, q_seq, q_len, T, H, d, nseq, Lmax, topk, idx, score,
                          static_cast<float*>(ws), Lmax, (hipStream_t)stream);
}

int32_t dsa_index_dense(const void* q, const float* w, const void* k, const int32_t* q_seq, const int32_t* q_len,
                        int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax, int32_t topk, int32_t* idx,
                        float* score, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsa_index_dense";
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  if (topk < 1) return fail(MISA_ERR_ARG, "%s: topk = %d < 1", fn, topk);
  if (T == 0) return ok();
  rc = check_outputs(fn, topk, idx, score);
  if (rc) return rc;
  rc = check_ws(fn, ws, ws_bytes, misa_workspace_bytes(MISA_OP_DSA_DENSE, T, H, Lmax, 0, topk, 0));
  if (rc) return rc;
  return score_and_select(fn, q, w, k, nullptr, H, nullptr, 0, q_seq, q_len, T, H, d, nseq, Lmax, topk, idx, score,
                          static_cast<float*>(ws), Lmax, (hipStream_t)stream);
}

int32_t misa_hier_rerank(const void* q, const float* w, const void* k, const int32_t* cand, int32_t kc,
                         const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq,
                         int64_t Lmax, int32_t topk, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                         void* stream) {
  const char* fn = "misa_hier_rerank";
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  if (topk < 1) return fail(MISA_ERR_ARG, "%s: topk = %d < 1", fn, topk);
  if (kc < topk) return fail(MISA_ERR_ARG, "%s: kc = %d < topk = %d", fn, kc, topk);
  if (T == 0) return ok();
  if (!cand) return fail(MISA_ERR_ARG, "%s: null cand", fn);
  if (!aligned(cand, 4)) return fail(MISA_ERR_ALIGN, "%s: cand must be 4-byte aligned", fn);
  rc = check_outputs(fn, topk, idx, score);
  if (rc) return rc;
  rc = check_ws(fn, ws, ws_bytes, misa_workspace_bytes(MISA_OP_HIER_RERANK, T, H, Lmax, 0, topk, kc));
  if (rc) return rc;
  return score_and_select(fn, q, w, k, nullptr, H, cand, kc, q_seq, q_len, T, H, d, nseq, Lmax, topk, idx, score,
                          static_cast<float*>(ws), kc, (hipStream_t)stream);
}

namespace {

// The fused decode pipeline (decode shapes) or the separate calls (prefill shapes).
int32_t run_indexer(const char* fn, bool hier, const void* q, const float* w, const void* k, const float* kbar,
                    const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq,
                    int64_t Lmax, int32_t B, int32_t h, int32_t kc, int32_t topk, int32_t* heads, int32_t* cand,
                    int32_t* idx, float* score, void* ws, size_t ws_bytes, hipStream_t st) {
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  if (B < 1 || B > Lmax) return fail(MISA_ERR_ARG, "%s: B = %d not in [1, Lmax]", fn, B);
  if (h < 1 || h > H) return fail(MISA_ERR_ARG, "%s: h = %d not in [1, H = %d]", fn, h, H);
  if (topk < 1) return fail(MISA_ERR_ARG, "%s: topk = %d < 1", fn, topk);
  if (hier && kc < topk) return fail(MISA_ERR_ARG, "%s: kc = %d < topk = %d", fn, kc, topk);
  if (T == 0) return ok();
  if (!kbar || !aligned(kbar, 16)) return fail(MISA_ERR_ARG, "%s: kbar must be a 16-byte aligned pointer", fn);
  rc = check_outputs(fn, topk, idx, score);
  if (rc) return rc;
  if (!aligned(heads, 4) || !aligned(cand, 4)) return fail(MISA_ERR_ALIGN, "%s: heads/cand must be 4-byte aligned", fn);
  const int32_t op = hier ? MISA_OP_HIER_INDEXER : MISA_OP_INDEXER;
  rc = check_ws(fn, ws, ws_bytes, misa_workspace_bytes(op, T, H, Lmax, B, topk, hier ? kc : 0));
  if (rc) return rc;

  const bool fused = T <= kFusedMaxRows && !wide_tiles(T, nseq) && !few_tiles(T, nseq) &&
                     misa::split_topk_always_ok(Lmax) && (!hier || misa::split_topk_always_ok(kc));
  if (!fused) {
    char* p = static_cast<char*>(ws);
    const size_t rws = misa_workspace_bytes(MISA_OP_ROUTE, T, H, Lmax, B, 0, 0);
    int32_t* hd = heads ? heads : reinterpret_cast<int32_t*>(p + rws);
    char* rest = p + rws + round_up((size_t)T * H * 4);
    rc = misa_route(q, w, k, kbar, q_seq, q_len, T, H, d, nseq, Lmax, B, h, hd, nullptr, p, rws, st);
    if (rc) return rc;
    if (!hier)
      return misa_score_topk(q, w, k, hd, h, q_seq, q_len, T, H, d, nseq, Lmax, topk, idx, score, rest,
                             select_ws_bytes(T, Lmax), st);
    int32_t* cd = cand ? cand : reinterpret_cast<int32_t*>(rest);
    char* rest2 = rest + round_up((size_t)T * (size_t)kc * 4);
    rc = misa_score_topk(q, w, k, hd, h, q_seq, q_len, T, H, d, nseq, Lmax, kc, cd, nullptr, rest2,
                         select_ws_bytes(T, Lmax), st);
    if (rc) return rc;
    return misa_hier_rerank(q, w, k, cd, kc, q_seq, q_len, T, H, d, nseq, Lmax, topk, idx, score, rest2,
                            select_ws_bytes(T, kc), st);
  }

  FusedLayout f = fused_layout(T, H, Lmax, B, hier ? kc : 0, ws);
  // coarse selection: split over chunks for long rows (MISA† always: its
  // compaction also re-scores the kept tokens); one workgroup per row otherwise
  const bool coarse_split = hier || misa::use_split_topk(T, Lmax, true);
  const bool fine_split = hier && kc > misa::topk_row_reg_max();
  // 1. router partials (+ partial-block dots), clearing the top-k state of the later launches
  misa::RouteArgs ra{};
  ra.q = static_cast<const uint16_t*>(q);
  ra.w = w;
  ra.k = static_cast<const uint16_t*>(k);
  ra.kbar = kbar;
  ra.q_seq = q_seq;
  ra.q_len = q_len;
  ra.T = T;
  ra.H = H;
  ra.nseq = nseq;
  ra.Lmax = Lmax;
  ra.B = B;
  ra.h = h;
  ra.partial = f.partial;
  ra.nchunk = f.nchunk_r;
  ra.chunk_blocks = f.chunk_blocks;
  ra.fused = true;
  ra.xtail = f.xtail;
  ra.zero[0] = coarse_split ? f.sw.hist : nullptr;
  ra.zero_words[0] = coarse_split ? misa::split_topk_zero_words(T) : 0;
  ra.zero[1] = fine_split ? f.rw.hist : nullptr;
  ra.zero_words[1] = fine_split ? misa::split_topk_zero_words(T) : 0;
  misa::timing_before(misa::KID_ROUTE, st);
  hipError_t e = misa::launch_route(ra, d, st);
  misa::timing_after(misa::KID_ROUTE, st);
  if (e != hipSuccess) return hip_status(e, fn);
  // 2. head selection + routed scoring + level-1 histogram
  misa::ScoreArgs sa{};
  sa.q = ra.q;
  sa.w = w;
  sa.k = ra.k;
  sa.heads = nullptr;
  sa.hh = h;
  sa.q_seq = q_seq;
  sa.q_len = q_len;
  sa.T = T;
  sa.H = H;
  sa.nseq = nseq;
  sa.Lmax = Lmax;
  sa.out = f.scores;
  sa.out_stride = Lmax;
  sa.hist = coarse_split ? f.sw.hist : nullptr;
  sa.partial = f.partial;
  sa.xtail = f.xtail;
  sa.nchunk_r = f.nchunk_r;
  sa.B = B;
  sa.heads_out = heads;
  e = misa::launch_score(sa, d, false, false, Lmax, st);
  if (e != hipSuccess) return hip_status(e, fn);
  // 3. top-k of the routed scores
  misa::TopkArgs b{};
  b.scores = f.scores;
  b.stride = Lmax;
  b.q_seq = q_seq;
  b.q_len = q_len;
  b.nseq = nseq;
  b.Lmax = Lmax;
  b.T = T;
  misa::timing_before(misa::KID_TOPK, st);
  if (!hier) {
    b.k = topk;
    b.idx = idx;
    b.score = score;
    e = coarse_split ? misa::launch_topk_split(b, f.sw, true, st) : misa::launch_topk(b, st);
  } else {
    int32_t* cd = cand ? cand : f.cand;
    b.k = kc;
    b.idx = cd;
    b.score = nullptr;
    misa::RescoreArgs r{};
    r.q = ra.q;
    r.w = w;
    r.k = ra.k;
    r.H = H;
    r.d = d;
    r.scores = f.rr_scores;
    r.hist = fine_split ? f.rw.hist : nullptr;   // level-1 histogram of the split fine stage
    r.fidx = idx;
    r.fscore = score;
    r.ftopk = topk;
    // rows of at most 8192 candidates: coarse selection, re-scoring and fine
    // selection in one launch
    const bool one = kc <= 8192;
    e = one ? misa::launch_hier_select(b, f.sw, r, f.mscore, st) : misa::launch_topk_split_rescore(b, f.sw, r, st);
    if (e == hipSuccess && !one) {
      // 4. MISA† fine stage: top-k of the candidates' dense scores
      misa::TopkArgs b2{};
      b2.scores = f.rr_scores;
      b2.stride = kc;
      b2.q_seq = q_seq;
      b2.q_len = q_len;
      b2.nseq = nseq;
      b2.Lmax = Lmax;
      b2.imap = cd;
      b2.kc = kc;
      b2.T = T;
      b2.k = topk;
      b2.idx = idx;
      b2.score = score;
      e = fine_split ? misa::launch_topk_split(b2, f.rw, true, st) : misa::launch_topk(b2, st);
    }
  }
  misa::timing_after(misa::KID_TOPK, st);
  return hip_status(e, fn);
}

}  // namespace

int32_t misa_indexer(const void* q, const float* w, const void* k, const float* kbar, const int32_t* q_seq,
                     const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax, int32_t B,
                     int32_t h, int32_t topk, int32_t* heads, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                     void* stream) {
  return run_indexer("misa_indexer", false, q, w, k, kbar, q_seq, q_len, T, H, d, nseq, Lmax, B, h, 0, topk, heads,
                     nullptr, idx, score, ws, ws_bytes, (hipStream_t)stream);
}

int32_t misa_hier_indexer(const void* q, const float* w, const void* k, const float* kbar, const int32_t* q_seq,
                          const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax,
                          int32_t B, int32_t h, int32_t kc, int32_t topk, int32_t* heads, int32_t* cand, int32_t* idx,
                          float* score, void* ws, size_t ws_bytes, void* stream) {
  return run_indexer("misa_hier_indexer", true, q, w, k, kbar, q_seq, q_len, T, H, d, nseq, Lmax, B, h, kc, topk,
                     heads, cand, idx, score, ws, ws_bytes, (hipStream_t)stream);
}

int32_t misa_hier_indexer_noalloc(const void* q, const float* w, const void* k, const float* kbar,
                                  const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d,
                                  int64_t nseq, int64_t Lmax, int32_t B, int32_t h, int32_t kc, int32_t topk,
                                  int32_t* heads, int32_t* cand, int32_t* idx, float* score, void* stream) {
  const char* fn = "misa_hier_indexer_noalloc";
  const size_t need = misa_workspace_bytes(MISA_OP_HIER_INDEXER, T, H, Lmax, B, topk, kc);
  if (need > (size_t)MISA_SCRATCH_BYTES)
    return fail(MISA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch; the library holds %zu per GPU", fn,
                need, (size_t)MISA_SCRATCH_BYTES);
  void* ws = nullptr;
  if (T > 0) {
    const int32_t rc = scratch_of_stream(fn, (hipStream_t)stream, &ws);
    if (rc) return rc;
  }
  return run_indexer(fn, true, q, w, k, kbar, q_seq, q_len, T, H, d, nseq, Lmax, B, h, kc, topk, heads, cand, idx,
                     score, ws, (size_t)MISA_SCRATCH_BYTES, (hipStream_t)stream);
}

namespace {

// Checks of the block filter's own arguments (q, w, kbar, q_seq, q_len checked before).
int32_t check_block(const char* fn, int64_t T, int32_t H, int64_t Lmax, int32_t B, int32_t h, int32_t m) {
  if (B < 1 || B > Lmax) return fail(MISA_ERR_ARG, "%s: B = %d not in [1, Lmax]", fn, B);
  if (h < 1 || h > H) return fail(MISA_ERR_ARG, "%s: h = %d not in [1, H = %d]", fn, h, H);
  if (m < 1 || m > Lmax / B) return fail(MISA_ERR_ARG, "%s: m = %d not in [1, Lmax / B = %lld]", fn, m, (long long)(Lmax / B));
  const int64_t kc = ((int64_t)m + 1) * B;
  if (kc >= (int64_t(1) << 30)) return fail(MISA_ERR_ARG, "%s: (m + 1) * B too large", fn);
  const int64_t nchunk = (Lmax / B + 63) / 64;
  if (T * nchunk >= (int64_t(1) << 32) || T * ((kc + 255) / 256) >= (int64_t(1) << 32))
    return fail(MISA_ERR_ARG, "%s: grid too large", fn);
  return MISA_OK;
}

// Block scores, the top-m complete blocks (ordinary top-k over the score rows)
// and, if cand is given, the candidate token list.
int32_t block_filter_run(const char* fn, const void* q, const float* w, const float* kbar, const int32_t* heads,
                         int32_t h, const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d,
                         int64_t nseq, int64_t Lmax, int32_t B, int32_t m, int32_t* blocks, int32_t* cand, void* ws,
                         hipStream_t st) {
  misa::BlockArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.w = w;
  a.kbar = kbar;
  a.heads = heads;
  a.h = h;
  a.q_seq = q_seq;
  a.q_len = q_len;
  a.T = T;
  a.H = H;
  a.nseq = nseq;
  a.Lmax = Lmax;
  a.B = B;
  a.nblk = Lmax / B;
  a.bscore = static_cast<float*>(ws);
  a.blen = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + round_up((size_t)T * (size_t)a.nblk * sizeof(float)));
  hipError_t e = misa::launch_block_score(a, d, st);
  if (e != hipSuccess) return hip_status(e, fn);
  if (cand && misa::block_select_fused(a))   // selection and candidate list in one launch
    return hip_status(misa::launch_block_select(a, m, blocks, cand, (m + 1) * B, st), fn);
  misa::TopkArgs b{};
  b.scores = a.bscore;
  b.stride = a.nblk;
  b.q_seq = q_seq;
  b.q_len = a.blen;
  b.nseq = nseq;
  b.Lmax = a.nblk;
  b.imap = nullptr;
  b.kc = 0;
  b.T = T;
  b.k = m;
  b.idx = blocks;
  b.score = nullptr;
  e = misa::launch_topk(b, st);
  if (e != hipSuccess) return hip_status(e, fn);
  if (cand) e = misa::launch_block_expand(a, blocks, m, cand, (m + 1) * B, st);
  return hip_status(e, fn);
}

}  // namespace

int32_t misa_block_filter(const void* q, const float* w, const float* kbar, const int32_t* heads, int32_t h,
                          const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq,
                          int64_t Lmax, int32_t B, int32_t m, int32_t* blocks, int32_t* cand, void* ws,
                          size_t ws_bytes, void* stream) {
  const char* fn = "misa_block_filter";
  int32_t rc = check_common(fn, q, w, kbar, q_seq, q_len, T, H, d, nseq, Lmax);   // kbar in the place of k
  if (rc) return rc;
  rc = check_block(fn, T, H, Lmax, B, h, m);
  if (rc) return rc;
  if (T == 0) return ok();
  if (!heads || !blocks) return fail(MISA_ERR_ARG, "%s: null heads/blocks", fn);
  if (!aligned(heads, 4) || !aligned(blocks, 4) || !aligned(cand, 4))
    return fail(MISA_ERR_ALIGN, "%s: heads/blocks/cand must be 4-byte aligned", fn);
  rc = check_ws(fn, ws, ws_bytes, misa_workspace_bytes(MISA_OP_BLOCK_FILTER, T, H, Lmax, B, 0, m));
  if (rc) return rc;
  return block_filter_run(fn, q, w, kbar, heads, h, q_seq, q_len, T, H, d, nseq, Lmax, B, m, blocks, cand, ws,
                          (hipStream_t)stream);
}

int32_t misa_block_indexer(const void* q, const float* w, const void* k, const float* kbar, const int32_t* q_seq,
                           const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax,
                           int32_t B, int32_t h, int32_t m, int32_t topk, int32_t* heads, int32_t* blocks,
                           int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "misa_block_indexer";
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  rc = check_block(fn, T, H, Lmax, B, h, m);
  if (rc) return rc;
  if (topk < 1) return fail(MISA_ERR_ARG, "%s: topk = %d < 1", fn, topk);
  if (T == 0) return ok();
  if (!kbar || !aligned(kbar, 16)) return fail(MISA_ERR_ARG, "%s: kbar must be a 16-byte aligned pointer", fn);
  rc = check_outputs(fn, topk, idx, score);
  if (rc) return rc;
  if (!aligned(heads, 4) || !aligned(blocks, 4)) return fail(MISA_ERR_ALIGN, "%s: heads/blocks must be 4-byte aligned", fn);
  rc = check_ws(fn, ws, ws_bytes, misa_workspace_bytes(MISA_OP_BLOCK_INDEXER, T, H, Lmax, B, topk, m));
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int32_t kc = (m + 1) * B;
  char* p = static_cast<char*>(ws);
  const size_t rws = misa_workspace_bytes(MISA_OP_ROUTE, T, H, Lmax, B, 0, 0);
  int32_t* hd = heads ? heads : reinterpret_cast<int32_t*>(p + rws);
  p += rws + round_up((size_t)T * H * 4);
  int32_t* bl = blocks ? blocks : reinterpret_cast<int32_t*>(p);
  p += round_up((size_t)T * (size_t)m * 4);
  int32_t* cd = reinterpret_cast<int32_t*>(p);
  p += round_up((size_t)T * (size_t)kc * 4);
  rc = misa_route(q, w, k, kbar, q_seq, q_len, T, H, d, nseq, Lmax, B, h, hd, nullptr, ws, rws, st);
  if (rc) return rc;
  rc = block_filter_run(fn, q, w, kbar, hd, h, q_seq, q_len, T, H, d, nseq, Lmax, B, m, bl, cd, p, st);
  if (rc) return rc;
  return score_and_select(fn, q, w, k, hd, h, cd, kc, q_seq, q_len, T, H, d, nseq, Lmax, topk, idx, score,
                          reinterpret_cast<float*>(p), kc, st);
}

int32_t misa_pivot_indexer(const void* q, const float* w, const void* k, const int32_t* q_seq, const int32_t* q_len,
                           int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax, int32_t G, int32_t kc,
                           int32_t topk, int32_t* cand, int32_t* idx, float* score, void* ws, size_t ws_bytes,
                           void* stream) {
  const char* fn = "misa_pivot_indexer";
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  if (G < 1) return fail(MISA_ERR_ARG, "%s: G = %d < 1", fn, G);
  if (topk < 1) return fail(MISA_ERR_ARG, "%s: topk = %d < 1", fn, topk);
  if (kc < topk || kc > Lmax) return fail(MISA_ERR_ARG, "%s: kc = %d not in [topk, Lmax]", fn, kc);
  if (T == 0) return ok();
  rc = check_outputs(fn, topk, idx, score);
  if (rc) return rc;
  if (!aligned(cand, 4)) return fail(MISA_ERR_ALIGN, "%s: cand must be 4-byte aligned", fn);
  const int64_t ng = (T + G - 1) / G;
  if (ng * (int64_t)H * (d / 8) >= (int64_t(1) << 38) || T * (int64_t)kc >= (int64_t(1) << 38))
    return fail(MISA_ERR_ARG, "%s: grid too large", fn);
  rc = check_ws(fn, ws, ws_bytes, misa_workspace_bytes(MISA_OP_PIVOT_INDEXER, T, H, Lmax, G, topk, kc));
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* p = static_cast<char*>(ws);
  misa::PivotArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.w = w;
  a.q_seq = q_seq;
  a.q_len = q_len;
  a.T = T;
  a.H = H;
  a.d = d;
  a.G = G;
  a.ng = ng;
  a.qp = reinterpret_cast<uint16_t*>(p);
  p += round_up((size_t)ng * H * 256 * 2);
  a.wp = reinterpret_cast<float*>(p);
  p += round_up((size_t)ng * H * 4);
  a.gseq = reinterpret_cast<int32_t*>(p);
  p += round_up((size_t)ng * 4);
  a.glen = reinterpret_cast<int32_t*>(p);
  p += round_up((size_t)ng * 4);
  int32_t* gcand = reinterpret_cast<int32_t*>(p);
  p += round_up((size_t)ng * (size_t)kc * 4);
  int32_t* cd = cand ? cand : reinterpret_cast<int32_t*>(p);
  p += round_up((size_t)T * (size_t)kc * 4);
  hipError_t e = misa::launch_pivot_proxy(a, st);
  if (e != hipSuccess) return hip_status(e, fn);
  // the proxies' dense scan of their groups' longest prefixes keeps kc candidates
  rc = score_and_select(fn, a.qp, a.wp, k, nullptr, H, nullptr, 0, a.gseq, a.glen, ng, H, d, nseq, Lmax, kc, gcand,
                        nullptr, reinterpret_cast<float*>(p), Lmax, st);
  if (rc) return rc;
  e = misa::launch_pivot_broadcast(gcand, cd, T, G, kc, st);
  if (e != hipSuccess) return hip_status(e, fn);
  // each query re-ranks its group's candidates with its own dense indexer
  return score_and_select(fn, q, w, k, nullptr, H, cd, kc, q_seq, q_len, T, H, d, nseq, Lmax, topk, idx, score,
                          reinterpret_cast<float*>(p), kc, st);
}

int32_t misa_debug_scores(const void* q, const float* w, const void* k, const int32_t* heads, int32_t h,
                          const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq,
                          int64_t Lmax, float* scores, void* stream) {
  const char* fn = "misa_debug_scores";
  int32_t rc = check_common(fn, q, w, k, q_seq, q_len, T, H, d, nseq, Lmax);
  if (rc) return rc;
  if (h < 1 || h > H) return fail(MISA_ERR_ARG, "%s: h = %d not in [1, H = %d]", fn, h, H);
  if (!heads && h != H) return fail(MISA_ERR_ARG, "%s: heads = NULL needs h == H", fn);
  if (T == 0) return ok();
  if (!scores || !aligned(scores, 4)) return fail(MISA_ERR_ARG, "%s: null or misaligned scores", fn);
  return score_and_select(fn, q, w, k, heads, h, nullptr, 0, q_seq, q_len, T, H, d, nseq, Lmax, 0, nullptr, nullptr,
                          scores, Lmax, (hipStream_t)stream);
}

int32_t misa_timing_begin(int32_t kernel, int32_t capacity, void* stream) {
  if (kernel < 1 || kernel > 5 || capacity < 1) return fail(MISA_ERR_ARG, "misa_timing_begin: bad kernel or capacity");
  hipStream_t st = (hipStream_t)stream;
  TimingEntry fresh;
  fresh.stream = st;
  fresh.kid = kernel;
  fresh.cap = capacity;
  fresh.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& ev : fresh.ev) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      timing_release(fresh);
      return hip_status(e, "misa_timing_begin");
    }
  }
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto it = g_timing.entries.begin(); it != g_timing.entries.end(); ++it)
    if (it->stream == st) {   // a second begin on the stream replaces the first
      timing_release(*it);
      g_timing.entries.erase(it);
      break;
    }
  g_timing.entries.push_back(std::move(fresh));
  g_timing.active.store((int)g_timing.entries.size(), std::memory_order_release);
  return ok();
}

int32_t misa_timing_end(void* stream, float* total_ms, int32_t* launches) {
  hipStream_t st = (hipStream_t)stream;
  TimingEntry e;
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    auto it = g_timing.entries.begin();
    while (it != g_timing.entries.end() && it->stream != st) ++it;
    if (it == g_timing.entries.end()) return fail(MISA_ERR_ARG, "misa_timing_end: no timing begun on this stream");
    e = std::move(*it);
    g_timing.entries.erase(it);
    g_timing.active.store((int)g_timing.entries.size(), std::memory_order_release);
  }
  float tot = 0.f;
  for (int i = 0; i < e.n; ++i) {
    hipError_t r = hipEventSynchronize(e.ev[2 * i + 1]);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, e.ev[2 * i], e.ev[2 * i + 1]);
    if (r != hipSuccess) {
      timing_release(e);
      return hip_status(r, "misa_timing_end");
    }
    tot += ms;
  }
  timing_release(e);
  if (total_ms) *total_ms = tot;
  if (launches) *launches = e.n;
  return ok();
}

}  // extern "C"
