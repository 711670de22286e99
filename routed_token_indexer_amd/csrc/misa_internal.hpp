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
  const int32_t* cand;      // [T][kc] key indices (gather mode) or null
  const int32_t* row_len;   // [T] valid candidates per row (gather mode) or null
  int kc;
  int64_t T;
  int H;
  int64_t nseq;
  int64_t Lmax;
  float* out;               // [T][out_stride]
  int64_t out_stride;
  int chunk;                // keys per workgroup chunk
};

int score_rows_per_query(int hh);
// gather: keys come from cand; wide: many queries of one sequence per tile (prefill)
hipError_t launch_score(const ScoreArgs& a, int d, bool gather, bool wide, int64_t max_len, hipStream_t st);

hipError_t launch_pool(const uint16_t* k, int64_t nseq, int64_t Lmax, int d, int B, float* kbar,
                       hipStream_t st);

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
  int32_t* counter;         // workspace [T]
  int nchunk;
  int chunk_blocks;
};
size_t route_partial_floats(int64_t T, int H, int64_t Lmax, int B, int* nchunk, int* chunk_blocks);
hipError_t launch_route(const RouteArgs& a, int d, hipStream_t st);

// Per-row top-k of fp32 score rows.
struct TopkArgs {
  const float* scores;      // [T][stride]
  int64_t stride;
  const int32_t* row_len;   // [T] or null (then q_len clamped to [0, Lmax], q_seq checked)
  const int32_t* q_seq;
  const int32_t* q_len;
  int64_t nseq;
  int64_t Lmax;
  const int32_t* imap;      // [T][kc] output index map (gather mode) or null
  int kc;
  int64_t T;
  int k;
  int32_t* idx;             // [T][k]
  float* score;             // [T][k] or null
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

// Number of leading valid entries of each candidate row.
hipError_t launch_cand_count(const int32_t* cand, int kc, const int32_t* q_seq, const int32_t* q_len,
                             int64_t T, int64_t nseq, int64_t Lmax, int32_t* row_len, hipStream_t st);

// Event timing of one internal kernel class (measurement aid).
enum KernelId { KID_NONE = 0, KID_SCORE = 1, KID_TOPK = 2, KID_ROUTE = 3, KID_POOL = 4 };
void timing_before(int kid, hipStream_t st);
void timing_after(int kid, hipStream_t st);

}  // namespace misa
