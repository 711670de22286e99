// C-ABI layer: argument checks, workspace layout and kernel dispatch.
// Declarations and the contract of every entry point are in include/misa.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/misa.h"
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

// Workspace of scoring + selection over rows of at most max_len: the fp32 score
// rows, then (for few long rows) the split top-k's state.
size_t select_ws_bytes(int64_t T, int64_t max_len) {
  size_t b = round_up((size_t)T * (size_t)max_len * sizeof(float));
  if (misa::use_split_topk(T, max_len)) b += round_up(misa::split_topk_ws_bytes(T, max_len));
  return b;
}

// ---------------------------------------------------------------- timing
struct Timing {
  std::mutex mu;
  int kid = 0;
  int cap = 0;
  int n = 0;
  std::vector<hipEvent_t> ev;
};
Timing g_timing;

}  // namespace

namespace misa {
void timing_before(int kid, hipStream_t st) {
  if (g_timing.kid != kid || g_timing.n >= g_timing.cap) return;
  (void)hipEventRecord(g_timing.ev[2 * g_timing.n], st);
}
void timing_after(int kid, hipStream_t st) {
  if (g_timing.kid != kid || g_timing.n >= g_timing.cap) return;
  (void)hipEventRecord(g_timing.ev[2 * g_timing.n + 1], st);
  ++g_timing.n;
}
}  // namespace misa

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
  const bool split = idx && misa::use_split_topk(T, max_len);
  misa::SplitTopkWs sw{};
  hipError_t e = hipSuccess;
  if (split) {
    void* base = reinterpret_cast<char*>(scores) + round_up((size_t)T * (size_t)stride * sizeof(float));
    sw = misa::split_topk_carve(base, T, max_len);
    e = misa::launch_zero(sw.hist, misa::split_topk_zero_words(T), st);
    if (e != hipSuccess) return hip_status(e, fn);
    if (!wide) a.hist = sw.hist;   // the decode scoring kernel builds the level-1 histogram
  }
  const int kid = gather ? misa::KID_GATHER_SCORE : misa::KID_SCORE;
  misa::timing_before(kid, st);
  e = misa::launch_score(a, d, gather, wide, max_len, st);
  misa::timing_after(kid, st);
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

int32_t misa_timing_begin(int32_t kernel, int32_t capacity) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (kernel < 1 || kernel > 5 || capacity < 1) return fail(MISA_ERR_ARG, "misa_timing_begin: bad kernel or capacity");
  for (hipEvent_t ev : g_timing.ev) (void)hipEventDestroy(ev);
  g_timing.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& ev : g_timing.ev) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      g_timing.kid = 0;
      return hip_status(e, "misa_timing_begin");
    }
  }
  g_timing.cap = capacity;
  g_timing.n = 0;
  g_timing.kid = kernel;
  return ok();
}

int32_t misa_timing_end(float* total_ms, int32_t* launches) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  const int n = g_timing.n;
  g_timing.kid = 0;
  float tot = 0.f;
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(g_timing.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_status(e, "misa_timing_end");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_status(e, "misa_timing_end");
    tot += ms;
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = n;
  g_timing.n = 0;
  return ok();
}

}  // extern "C"
