// Token scoring of the MISA / DSA indexer on the gfx950 matrix cores.
//
// MISA pages (MISA abstract; gist.science "Methodologie: MISA", sparse token
// scoring): only the routed heads score every prefix token. The score of token s
// for query t with head set R is
//     S[t][s] = sum_{g in R} w[t][g] * max(q[t][g] . k[s], 0).
// The dense DSA indexer ("Probleemstelling") is the same with R = all H heads,
// and the MISA† fine stage ("Hiërarchische Variant") applies it to a candidate
// list instead of the whole prefix.
//
// The query's gathered head rows are MFMA A-fragments held in registers; keys
// stream from HBM as B-fragments, 16 keys per 16x16x32 MFMA column tile; ReLU,
// the head weight and the head sum are applied to the accumulators in
// registers and one fp32 score per (query, key) is stored. Lane i of a wave
// supplies A row / B column (i % 16) and k-slots 8 * (i / 16) .. + 8 of each
// 32-dim step, so one load instruction reads 64 contiguous bytes of each of 16
// keys.
//   decode kernel  one query per workgroup and a chunk of its keys (decode
//                  batches and candidate lists); can also build the level-1
//                  histogram of the split top-k for the scores it writes.
//   wide kernel    a tile of consecutive queries of one sequence per workgroup
//                  (causal prefill), so each key tile loaded serves the whole
//                  query tile.
#include <hip/hip_ext.h>

#include "misa_common.hpp"
#include "misa_internal.hpp"
#include "misa_score_dev.hpp"

namespace misa {

namespace {

// Row length of query t (tokens it can see, or valid candidates) and its key
// sequence; seq = -1 marks an absent or invalid query (it produces nothing).
__device__ __forceinline__ void query_info(const ScoreArgs& a, int64_t t, int& seq, int& n) {
  seq = -1;
  n = 0;
  if (t >= a.T) return;
  const int sq = a.q_seq[t];
  if (sq < 0 || sq >= a.nseq) return;
  seq = sq;
  const int p = a.q_len[t];
  n = p < 0 ? 0 : (p > a.Lmax ? (int)a.Lmax : p);
}

// Head id of row slot hs of query t (-1: padding row or invalid id).
__device__ __forceinline__ int row_head(const ScoreArgs& a, int64_t t, int hs) {
  if (hs >= a.hh) return -1;
  const int g = a.heads ? a.heads[t * a.hh + hs] : hs;
  return (g >= 0 && g < a.H) ? g : -1;
}

template <int D, int NHP, int RT, int KT, bool GATHER>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  constexpr int QT = (16 * RT) / NHP;       // query slots of the tile
  constexpr int KS = D / 32;                // 32-wide k-steps
  // per-lane output slots: how many different slots one lane writes
  constexpr int NOUT = NHP == 4 ? RT : (NHP == 8 ? RT : QT);
  static_assert(QT >= 1 && (16 * RT) % NHP == 0, "row tiling");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;                // MFMA column (key) / A row within a tile
  const int grp = lane >> 4;                // lane group
  const int64_t tile = (int64_t)gridDim.y - 1 - blockIdx.y;   // longest prefixes first
  const int64_t t0 = tile * QT;

  // ---- tile-wide slot info (indexed with compile-time indices only)
  int slot_seq[QT], slot_n[QT];
  int nmax = 0;
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    query_info(a, t0 + s, slot_seq[s], slot_n[s]);
    nmax = max(nmax, slot_n[s]);
  }
  const int c_begin = blockIdx.x * a.chunk;
  if (c_begin >= nmax) return;
  const int c_end = min(c_begin + a.chunk, nmax);

  // ---- A fragments (gathered query rows) and row weights, loaded once
  u32x4 afrag[RT][KS];
  float wrow[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = 16 * r + col;
    const int64_t t = t0 + row / NHP;
    int seq, n;
    query_info(a, t, seq, n);
    const int head = seq < 0 ? -1 : row_head(a, t, row % NHP);
    const uint16_t* qp = a.q + ((t * a.H + (head < 0 ? 0 : head)) * D) + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head >= 0) v = *reinterpret_cast<const u32x4*>(qp + ks * 32);
      afrag[r][ks] = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row2 = 16 * r + 4 * grp + j;
      const int64_t t2 = t0 + row2 / NHP;
      int seq2, n2;
      query_info(a, t2, seq2, n2);
      const int hd = seq2 < 0 ? -1 : row_head(a, t2, row2 % NHP);
      wrow[r][j] = hd < 0 ? 0.f : a.w[t2 * a.H + hd];
    }
  }

  // ---- the slots this lane stores (slot index, its sequence and row length)
  int out_slot[NOUT], out_seq[NOUT], out_n[NOUT];
#pragma unroll
  for (int i = 0; i < NOUT; ++i) {
    out_slot[i] = NHP == 4 ? 4 * i + grp : (NHP == 8 ? 2 * i + (grp >> 1) : i);
    query_info(a, t0 + out_slot[i], out_seq[i], out_n[i]);
  }
  const bool writer = NHP == 4 ? true : (NHP == 8 ? (grp & 1) == 0 : grp == 0);

  // ---- one pass per distinct key source among the slots
#pragma unroll
  for (int lead = 0; lead < QT; ++lead) {
    if (slot_seq[lead] < 0) continue;
    bool first = true;
#pragma unroll
    for (int s = 0; s < lead; ++s)
      if (!GATHER && slot_seq[s] == slot_seq[lead]) first = false;
    if (!first) continue;
    int pass_n = 0;
#pragma unroll
    for (int s = 0; s < QT; ++s)
      if (s == lead || (!GATHER && slot_seq[s] == slot_seq[lead])) pass_n = max(pass_n, slot_n[s]);
    const int p_end = min(c_end, pass_n);
    const uint16_t* kseq = a.k + (int64_t)slot_seq[lead] * a.Lmax * D + grp * 8;
    const int32_t* crow = GATHER ? a.cand + (t0 + lead) * a.kc : nullptr;
    // which of this lane's output slots belong to this pass
    bool in_pass[NOUT];
#pragma unroll
    for (int i = 0; i < NOUT; ++i)
      in_pass[i] = writer && out_seq[i] >= 0 &&
                   (GATHER ? out_slot[i] == lead : out_seq[i] == slot_seq[lead]);

    for (int base = c_begin + wave * (16 * KT); base < p_end; base += 4 * 16 * KT) {
      u32x4 bfrag[KT][KS];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int s = base + kt * 16 + col;
        int64_t key = -1;
        if (s < p_end) key = GATHER ? (int64_t)crow[s] : (int64_t)s;
        const uint16_t* kp = kseq + (key < 0 ? 0 : key) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (key >= 0) v = *reinterpret_cast<const u32x4*>(kp + ks * 32);
          bfrag[kt][ks] = v;
        }
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        floatx4 acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          acc[r] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc[r] = mfma_16x16x32(afrag[r][ks], bfrag[kt][ks], acc[r]);
        }
        // epilogue: ReLU, head weight, per-query head sum (rows 4*grp..4*grp+3 of each tile)
        float part[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          part[r] = wrow[r][0] * fmaxf(acc[r][0], 0.f) + wrow[r][1] * fmaxf(acc[r][1], 0.f) +
                    wrow[r][2] * fmaxf(acc[r][2], 0.f) + wrow[r][3] * fmaxf(acc[r][3], 0.f);
        }
        float val[NOUT];
        if constexpr (NHP == 4) {
#pragma unroll
          for (int r = 0; r < RT; ++r) val[r] = part[r];
        } else if constexpr (NHP == 8) {
#pragma unroll
          for (int r = 0; r < RT; ++r) val[r] = part[r] + __shfl_xor(part[r], 16, kWave);
        } else {
          constexpr int m = NHP / 16;
#pragma unroll
          for (int s = 0; s < QT; ++s) {
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < m; ++i) v += part[s * m + i];
            v += __shfl_xor(v, 16, kWave);
            v += __shfl_xor(v, 32, kWave);
            val[s] = v;
          }
        }
        const int s_out = base + kt * 16 + col;
#pragma unroll
        for (int i = 0; i < NOUT; ++i) {
          if (in_pass[i] && s_out < p_end && s_out < out_n[i])
            a.out[(t0 + out_slot[i]) * a.out_stride + s_out] = val[i] + 0.f;
        }
      }
    }
  }
}

// decode: grid (key chunks, T); one query per workgroup, its rows padded to RT tiles.
// Startup is ordered for a memory system that the key stream is about to
// saturate: everything that does not depend on the query's sequence (its H
// query rows, which are staged in LDS, its weights, the routed head ids or the
// router's chunk partials) is requested first, then the first key tiles, and
// only then are the routed heads selected and the A fragments read from LDS.
// Every iteration prefetches the next iteration's keys before computing the
// current one. With a.partial set, the workgroup selects the query's routed
// heads itself from the router's chunk partials (the fused decode pipeline).
template <int D, int RT, bool GATHER, bool HIST>
__global__ __launch_bounds__(256) void score_decode_kernel(ScoreArgs a) {
  constexpr int KT = 4;           // 16-key tiles per wave iteration: 64 keys, one per lane at the end
  constexpr int LDQ = D + 8;      // LDS row stride of the staged query rows (bf16)
  constexpr int QV = D / 8;       // 16-byte pieces per query row
  constexpr int QPT = (64 * QV + 255) / 256;   // staging pieces per thread (H <= 64)
  __shared__ uint32_t lh[HIST ? 4096 : 1];
  __shared__ __align__(16) uint16_t s_q[64 * LDQ];
  __shared__ float s_w[64];
  __shared__ int s_heads[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t t = blockIdx.y;
  const bool fused_route = a.partial != nullptr;

  // 1. requests that do not depend on the sequence
  u32x4 qv[QPT];
  const int nqv = a.H * QV;
  const uint16_t* qsrc = a.q + t * a.H * D;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = threadIdx.x + 256 * j;
    qv[j] = *reinterpret_cast<const u32x4*>(qsrc + (int64_t)(i < nqv ? i : 0) * 8);
  }
  // Issued by every lane from clamped, in-bounds addresses (a conditional load
  // would make the compiler wait for it before the key requests go out); the
  // pointer selects only depend on kernel arguments.
  const int gl = lane < a.H ? lane : a.H - 1;
  const float wg = a.w[t * a.H + gl];
  const float x = (fused_route ? a.xtail : a.w)[t * a.H + gl];
  PartialBatch pb;
  load_partials(fused_route ? a.partial : a.w, t, fused_route ? a.nchunk_r : 1, a.H, lane, pb);
  const int32_t* hp = a.heads ? a.heads + t * a.hh + (lane < a.hh ? lane : a.hh - 1) : a.q_seq + t;
  const int hv = *hp;
  const int head_in = a.heads ? hv : lane;

  int seq = a.q_seq[t];
  int p = a.q_len[t];
  if (seq < 0 || seq >= a.nseq) {
    seq = -1;
    p = 0;
  }
  p = p < 0 ? 0 : (p > a.Lmax ? (int)a.Lmax : p);
  const int n = GATHER ? (seq < 0 ? 0 : a.kc) : p;
  const int c_begin = blockIdx.x * a.chunk;
  if (c_begin >= n && !(fused_route && blockIdx.x == 0)) return;
  const int c_end = min(c_begin + a.chunk, n);
  const uint16_t* kseq = a.k + (int64_t)(seq < 0 ? 0 : seq) * a.Lmax * D + grp * 8;
  const int32_t* crow = GATHER ? a.cand + t * a.kc : nullptr;
  auto key_of = [&](int s) -> int {
    if constexpr (GATHER) {
      const int id = crow[s];
      return (id >= 0 && id < p) ? id : -1;
    } else {
      return s;
    }
  };
  // c_begin < max_len <= Lmax, so row c_begin of the (clamped) sequence exists
  const int fallback = GATHER ? 0 : c_begin;

  // 2. consume the small loads before any key request of this wave goes out
  // (workgroups dispatched a little later would otherwise find their small
  // loads queued behind tens of MiB of key requests): stage the query rows and
  // weights, and (wave 0) sum the router's partials.
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < nqv) *reinterpret_cast<u32x4*>(s_q + (i / QV) * LDQ + (i % QV) * 8) = qv[j];
  }
  float A = 0.f;
  if (wave == 0) {
    if (lane < a.H) s_w[lane] = wg;
    if (fused_route) A = finish_partials(a.partial, t, a.nchunk_r, a.H, lane, pb);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. the first two iterations' key tiles (two in flight per wave)
  constexpr int kStep = 4 * 16 * KT;   // keys per workgroup iteration
  const int base0 = c_begin + wave * 16 * KT;
  KeyTiles<D, KT> ta, tb;
  load_key_tiles<D, KT>(kseq, base0, c_end, col, key_of, fallback, ta);
  load_key_tiles<D, KT>(kseq, base0 + kStep, c_end, col, key_of, fallback, tb);
  __builtin_amdgcn_sched_barrier(0);

  // 4. select the heads while the keys stream in
  if (wave == 0) {
    if (fused_route) {
      const int n_tail = p - (p / a.B) * a.B;
      int pos;
      float r;
      const bool sel = route_rank(a.H, a.hh, lane, wg, A, x, n_tail, pos, r);
      if (sel) s_heads[pos] = lane;
      if (blockIdx.x == 0) {
        if (sel && a.heads_out) a.heads_out[t * a.hh + pos] = lane;
        if (lane < a.H && a.router_key) a.router_key[t * a.H + lane] = r;
      }
    } else if (lane < a.hh) {
      s_heads[lane] = (head_in >= 0 && head_in < a.H) ? head_in : -1;
    }
  }
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < 4096; i += 256) lh[i] = 0;
  }
  __syncthreads();
  if (c_begin >= n) return;

  u32x4 afrag[RT][D / 32];
  float wrow[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = 16 * r + col;
    const int head = row < a.hh ? s_heads[row] : -1;
    const uint16_t* qa = s_q + (head < 0 ? 0 : head) * LDQ + grp * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qa + ks * 32);
      afrag[r][ks] = head < 0 ? u32x4{0u, 0u, 0u, 0u} : v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row2 = 16 * r + 4 * grp + j;
      const int hd = row2 < a.hh ? s_heads[row2] : -1;
      wrow[r][j] = hd < 0 ? 0.f : s_w[hd];
    }
  }

  // Scores of this chunk go through a buffer view of [c_begin, c_end), so the
  // stores of lanes past c_end are dropped by the range check instead of being
  // branched around: the loop body stays straight-line and the compiler can
  // count the loads in flight exactly.
  const auto ov = buffer_view(a.out + t * a.out_stride + c_begin, (uint32_t)(c_end - c_begin) * 4u);
  auto emit = [&](const KeyTiles<D, KT>& tiles, int b) {
    const float v = score_four_tiles<D, RT>(afrag, wrow, tiles, grp);
    const int s = b + lane;
    buffer_store_f32(v, ov, (uint32_t)(s - c_begin) * 4u);
    if constexpr (HIST) atomicAdd(&lh[score_key(v) >> 20], s < c_end ? 1u : 0u);
  };
  // Two register sets alternate, so no in-flight tile is ever copied (a copy
  // would wait for its load). The iteration count is uniform over the
  // workgroup; each wave masks its own tail through c_end. Inside the loop the
  // loads are unconditional (an odd count prefetches one spare iteration of
  // in-bounds rows).
  const int nit = (c_end - c_begin + kStep - 1) / kStep;
  int it = 0;
  for (; it + 2 < nit; it += 2) {
    const int b = base0 + it * kStep;
    emit(ta, b);
    load_key_tiles<D, KT>(kseq, b + 2 * kStep, c_end, col, key_of, fallback, ta);
    emit(tb, b + kStep);
    load_key_tiles<D, KT>(kseq, b + 3 * kStep, c_end, col, key_of, fallback, tb);
  }
  if (it < nit) emit(ta, base0 + it * kStep);
  if (it + 1 < nit) emit(tb, base0 + (it + 1) * kStep);
  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + t * 4096;
    for (int i = threadIdx.x; i < 4096; i += 256)
      if (lh[i]) atomicAdd(&gh[i], lh[i]);
  }
}

// Launch, stamping the timing events at the kernel's own start and end when
// the scoring kernels are being timed.
template <typename K, typename... Args>
hipError_t launch_timed(int kid, K kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  hipEvent_t e0, e1;
  if (timing_take(kid, e0, e1))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  return hipGetLastError();
}

template <int D, int RT, bool GATHER>
hipError_t launch_decode(ScoreArgs a, int64_t max_len, hipStream_t st) {
  if (a.chunk <= 0) {
    // about 512 workgroups (two per CU), at least 256 keys each
    int64_t c = 256;
    while (c < 16384 && c * 512 < max_len * a.T) c *= 2;
    a.chunk = (int)c;
  }
  dim3 grid((unsigned)((max_len + a.chunk - 1) / a.chunk), (unsigned)a.T);
  const int kid = GATHER ? KID_GATHER_SCORE : KID_SCORE;
  if (a.hist) return launch_timed(kid, score_decode_kernel<D, RT, GATHER, true>, grid, dim3(256), st, a);
  return launch_timed(kid, score_decode_kernel<D, RT, GATHER, false>, grid, dim3(256), st, a);
}

template <int D>
hipError_t launch_decode_d(const ScoreArgs& a, bool gather, int64_t max_len, hipStream_t st) {
  const int rt = (a.hh + 15) / 16;
  if (gather) {
    switch (rt) {
      case 1: return launch_decode<D, 1, true>(a, max_len, st);
      case 2: return launch_decode<D, 2, true>(a, max_len, st);
      case 3: return launch_decode<D, 3, true>(a, max_len, st);
      default: return launch_decode<D, 4, true>(a, max_len, st);
    }
  }
  switch (rt) {
    case 1: return launch_decode<D, 1, false>(a, max_len, st);
    case 2: return launch_decode<D, 2, false>(a, max_len, st);
    case 3: return launch_decode<D, 3, false>(a, max_len, st);
    default: return launch_decode<D, 4, false>(a, max_len, st);
  }
}

template <int D, int NHP, int RT, int KT, bool GATHER>
hipError_t launch_cfg(const ScoreArgs& a, int64_t ntile, int nchunk, hipStream_t st) {
  dim3 grid(nchunk, (unsigned)ntile);
  return launch_timed(GATHER ? KID_GATHER_SCORE : KID_SCORE, score_kernel<D, NHP, RT, KT, GATHER>, grid, dim3(256),
                      st, a);
}

// Keys per workgroup: wide tiles (prefill) take 2048-key chunks; otherwise the
// chunk shrinks until the grid has about 2048 workgroups (at least 256 keys).
inline int pick_chunk(int64_t ntile, int64_t max_len, bool wide) {
  if (wide) return 2048;
  int64_t c = 256;
  while (c < 8192 && c * 2048 < max_len * ntile) c *= 2;
  return (int)c;
}

template <int D, bool GATHER>
hipError_t launch_d(ScoreArgs a, int nhp, bool wide, int64_t max_len, hipStream_t st) {
  // rows per query nhp in {4, 8, 16, 32, 48, 64}; wide = many queries per key chunk (prefill)
#define MISA_SCORE_CASE(NHP_, RT_, KT_)                                      \
  {                                                                          \
    constexpr int QT_ = (16 * RT_) / NHP_;                                   \
    const int64_t ntile = (a.T + QT_ - 1) / QT_;                             \
    if (a.chunk <= 0) a.chunk = pick_chunk(ntile, max_len, wide);            \
    const int nchunk = (int)((max_len + a.chunk - 1) / a.chunk);             \
    return launch_cfg<D, NHP_, RT_, KT_, GATHER>(a, ntile, nchunk, st);      \
  }
  (void)wide;
  switch (nhp) {
    case 4: MISA_SCORE_CASE(4, 4, 2)
    case 8: MISA_SCORE_CASE(8, 8, 2)
    case 16: MISA_SCORE_CASE(16, 8, 2)
    case 32: MISA_SCORE_CASE(32, 8, 2)
    case 48: MISA_SCORE_CASE(48, 6, 2)
    case 64: MISA_SCORE_CASE(64, 8, 2)
    default: return hipErrorInvalidValue;
  }
#undef MISA_SCORE_CASE
}

}  // namespace

int score_rows_per_query(int hh) {
  if (hh <= 4) return 4;
  if (hh <= 8) return 8;
  return 16 * ((hh + 15) / 16);
}

hipError_t launch_score(const ScoreArgs& a, int d, bool gather, bool wide, int64_t max_len, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (gather || !wide) {
    switch (d) {
      case 32: return launch_decode_d<32>(a, gather, max_len, st);
      case 64: return launch_decode_d<64>(a, gather, max_len, st);
      case 128: return launch_decode_d<128>(a, gather, max_len, st);
      case 256: return launch_decode_d<256>(a, gather, max_len, st);
    }
    return hipErrorInvalidValue;
  }
  const int nhp = score_rows_per_query(a.hh);
  switch (d) {
    case 32: return launch_d<32, false>(a, nhp, true, max_len, st);
    case 64: return launch_d<64, false>(a, nhp, true, max_len, st);
    case 128: return launch_d<128, false>(a, nhp, true, max_len, st);
    case 256: return launch_d<256, false>(a, nhp, true, max_len, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace misa
