// Internal launcher interface between the C-ABI layer (abi.hip) and the kernel
// translation units. Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

// Arguments of the token-scoring kernel (one fp32 score per (query, key)).
struct ScoreArgs {
  const uint16_t* q;        // bf16 [T][H][d]
  const float* w;           // fp32 [T][H]
  const uint16_t* k;        // bf16 [nseq][Lmax][d]
  const int32_t* heads;     // [T][hh] head ids, or null: heads 0..hh-1
  int hh;                   // heads per query
  const int32_t* q_seq;     // [T]
  const int32_t* q_len;     // [T]
  const int32_t* cand;      // [T][kc] key indices (gather mode) or null; ids outside [0, q_len) are skipped
  int kc;
  int64_t T;
  int H;
  int64_t nseq;
  int64_t Lmax;
  float* out;               // [T][out_stride]
  int64_t out_stride;
  int chunk;                // keys per workgroup chunk
  uint32_t* hist;           // optional [T][4096]: level-1 histogram of the written scores (decode
                            // kernel; bin b at word hist_word(b))
  // fused decode pipeline: heads selected in the kernel from the router's partials
  const float* partial;     // [T][nchunk_r][H] or null (then heads come from `heads`)
  const float* xtail;       // [T][H]
  int nchunk_r;
  int B;
  int32_t* heads_out;       // optional [T][hh], written by chunk 0
  float* router_key;        // optional [T][H], written by chunk 0
};

int score_rows_per_query(int hh);
// gather: keys come from cand; wide: many queries of one sequence per tile (prefill);
// few: several queries per sequence over long prefixes (small tiles, short key chunks)
hipError_t launch_score(const ScoreArgs& a, int d, bool gather, bool wide, int64_t max_len, hipStream_t st,
                        bool few = false);

hipError_t launch_pool(const uint16_t* k, int64_t nseq, int64_t Lmax, int d, int B, float* kbar,
                       hipStream_t st);
hipError_t launch_pool_update(const uint16_t* k, int64_t nseq, int64_t Lmax, int d, int B, const int32_t* prev_len,
                              const int32_t* new_len, int max_new, float* kbar, hipStream_t st);

struct RouteArgs {
  const uint16_t* q;        // bf16 [T][H][d]
  const float* w;           // fp32 [T][H]
  const uint16_t* k;        // bf16 [nseq][Lmax][d]
  const float* kbar;        // fp32 [nseq][Lmax / B][d]
  const int32_t* q_seq;
  const int32_t* q_len;
  int64_t T;
  int H;
  int64_t nseq;
  int64_t Lmax;
  int B;
  int h;
  int32_t* heads;           // [T][h]
  float* router_key;        // [T][H] or null
  float* partial;           // workspace [T][nchunk][H]
  int32_t* counter;         // unused
  int nchunk;
  int chunk_blocks;
  // fused decode pipeline: always emit partials, the partial-block dot into
  // xtail [T][H], select nothing, and zero the two regions below
  bool fused;
  float* xtail;
  uint32_t* zero[2];
  int64_t zero_words[2];
};
// Decode chunking of the pooled blocks (partials workspace in floats); prefill
// shapes (many queries per sequence) route one query per wave and need none.
size_t route_partial_floats(int64_t T, int H, int64_t Lmax, int B, int* nchunk, int* chunk_blocks);
bool route_is_prefill(int64_t T, int64_t nseq);
hipError_t launch_route(const RouteArgs& a, int d, hipStream_t st);

// Per-row top-k of fp32 score rows.
struct TopkArgs {
  const float* scores;      // [T][stride]
  int64_t stride;
  const int32_t* q_seq;     // rows: q_len clamped to [0, Lmax] tokens, or kc slots in gather mode

  const int32_t* q_len;
  int64_t nseq;
  int64_t Lmax;
  const int32_t* imap;      // [T][kc] output index map (gather mode) or null; ids outside [0, q_len) -> -1
  int kc;
  int64_t T;
  int k;
  int32_t* idx;             // [T][k]
  float* score;             // [T][k] or null
  // rows of length n with len_lo < n <= len_hi only (the register select; a
  // batch split over two launches by row length)
  int64_t len_lo = -1;
  int64_t len_hi = INT64_MAX;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// Longest row the register-resident single-workgroup top-k handles.
int64_t topk_row_reg_max();

// Split top-k for few long rows: several workgroups per row cooperate through
// global memory (level-1 histogram, candidate list, per-chunk offsets).
struct SplitTopkWs {
  uint32_t* hist;      // [T][4096] level-1 histogram (zero on entry; bin b at word hist_word(b))
  uint32_t* hist2;     // [T][4096] key bits 8..19 of the level-1 threshold bin's keys (zero on entry)
  uint32_t* state;     // [T][8] level-1 threshold bin, how many of its keys are kept, how many it holds
  uint32_t* counter;   // [T][4] candidate-list cursor, arrivals of the one-launch selection (zero on entry)
  uint32_t* ndef;      // [T][nchunk] keys above the level-1 threshold bin in each chunk; then
                       // [T][nchunk][3] the MISA† selection's member count and dense-key range
  uint32_t* cand;      // [T][cap][2] (key, index) of the level-1 threshold bin
  int64_t cap;
  int chunk;
  int nchunk;
};
// Workspace layout of the split path for T rows of at most max_len scores.
size_t split_topk_ws_bytes(int64_t T, int64_t max_len);
SplitTopkWs split_topk_carve(void* base, int64_t T, int64_t max_len);
// Words at the start of the carved region that must be zero before the launch.
int64_t split_topk_zero_words(int64_t T);
hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t st);
// hist_in_scoring: the scoring kernel builds the rows' level-1 histogram.
bool use_split_topk(int64_t T, int64_t max_len, bool hist_in_scoring);
// hist_done: the level-1 histogram was already accumulated by the scoring kernel.
hipError_t launch_topk_split(const TopkArgs& a, const SplitTopkWs& w, bool hist_done, hipStream_t st);
// rows of this length can always take the split path (whatever T)
bool split_topk_always_ok(int64_t max_len);

// Dense re-scoring of the kept candidates, fused into the coarse pass of MISA†.
struct RescoreArgs {
  const uint16_t* q;
  const float* w;
  const uint16_t* k;
  int H;
  int d;
  float* scores;            // [T][kc] dense score of each candidate slot (compaction only)
  uint32_t* hist;           // [T][4096] level-1 histogram of those scores (zero on entry; compaction only)
  // the final top-k, selected in the same launch (launch_hier_select only)
  int32_t* fidx;            // [T][ftopk]
  float* fscore;            // [T][ftopk] or null
  int ftopk;
};
// filter + compact of the coarse pass (level-1 histogram already built), the
// compact writing the candidate list (a.idx, k = kc) and its dense scores.
hipError_t launch_topk_split_rescore(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, hipStream_t st);
// The whole MISA† selection of rows of at most 8192 candidates in one launch
// (level-1 histogram of the routed scores already built; counters zero on
// entry): coarse top-k' (a.idx, k = k'), dense scores of the candidates
// (r.scores) and the final top-k (r.fidx, r.fscore). mscore: [T][w.cap] dense
// scores of the coarse members (workspace).
hipError_t launch_hier_select(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, float* mscore,
                              hipStream_t st);


// Coarse stage of the block filter: the routed indexer formula on the pooled
// keys of each query's complete blocks.
struct BlockArgs {
  const uint16_t* q;        // bf16 [T][H][d]
  const float* w;           // fp32 [T][H]
  const float* kbar;        // fp32 [nseq][nblk][d]
  const int32_t* heads;     // [T][h] (an id outside [0, H) contributes nothing)
  int h;
  const int32_t* q_seq;
  const int32_t* q_len;
  int64_t T;
  int H;
  int64_t nseq;
  int64_t Lmax;
  int B;
  int64_t nblk;             // Lmax / B pooled blocks per sequence
  float* bscore;            // [T][nblk] block scores (complete visible blocks)
  int32_t* blen;            // [T] complete visible blocks of each query
};
hipError_t launch_block_score(const BlockArgs& a, int d, hipStream_t st);
// cand [T][kc]: the tokens of the m retained blocks (blocks [T][m], ascending,
// -1 padded), then the partial block's tokens, then -1
hipError_t launch_block_expand(const BlockArgs& a, const int32_t* blocks, int m, int32_t* cand, int kc,
                               hipStream_t st);
// Both in one launch (rows of up to 4096 complete blocks: block_select_fused).
bool block_select_fused(const BlockArgs& a);
hipError_t launch_block_select(const BlockArgs& a, int m, int32_t* blocks, int32_t* cand, int kc, hipStream_t st);

// Proxy queries of groups of G consecutive queries (sum of the group's queries,
// rounded to bf16; sum of their weights; the first query's sequence; the longest prefix).
struct PivotArgs {
  const uint16_t* q;        // bf16 [T][H][d]
  const float* w;           // fp32 [T][H]
  const int32_t* q_seq;
  const int32_t* q_len;
  int64_t T;
  int H;
  int d;
  int G;
  int64_t ng;               // ceil(T / G)
  uint16_t* qp;             // bf16 [ng][H][d]
  float* wp;                // fp32 [ng][H]
  int32_t* gseq;            // [ng]
  int32_t* glen;            // [ng]
};
hipError_t launch_pivot_proxy(const PivotArgs& a, hipStream_t st);
// cand[t][:] = gcand[t / G][:] for t < T
hipError_t launch_pivot_broadcast(const int32_t* gcand, int32_t* cand, int64_t T, int G, int kc, hipStream_t st);

// Event timing of one internal kernel class (measurement aid).
enum KernelId { KID_NONE = 0, KID_SCORE = 1, KID_TOPK = 2, KID_ROUTE = 3, KID_POOL = 4, KID_GATHER_SCORE = 5 };
void timing_before(int kid, hipStream_t st);
void timing_after(int kid, hipStream_t st);
// Events for one launch of kernel class kid on stream st, stamped by the
// kernel's own start and end (hipExtLaunchKernelGGL); false when that class is
// not being timed on st.
bool timing_take(int kid, hipStream_t st, hipEvent_t& start, hipEvent_t& stop);

}  // namespace misa
