// Split per-query top-k for few, long score rows (decode: a handful of queries
// over 10^4..10^6 tokens), where one workgroup per row would leave the chip idle.
//
// Same selection rule as the per-row kernel (MISA pages: the indexer keeps the
// top-k tokens of each query; order by score descending, token index
// ascending; output in ascending token index, -1 padded), computed by three
// launches over (row, chunk) grids:
//   1. hist     each chunk adds its LDS histogram of the key's top 12 bits into
//               the row's global histogram (atomics).
//   2. filter   each chunk reads the finished histogram, finds the threshold
//               bin b1 (and how many of it are kept), counts its keys above b1
//               and appends the keys of bin b1 (key, index) to the row's list.
//   3. compact  each chunk resolves the exact k-th key u* on the candidate list
//               (12 + 8 more bits), derives its output offset from the counts of
//               the chunks before it, and writes its selected indices in index
//               order (ballots inside waves, counts across waves).
// No workgroup waits for or signals another inside a launch: on gfx950 the L2
// of each XCD is not coherent with the others within a kernel, so everything a
// chunk needs from other chunks comes from an earlier launch (global atomics
// for the histogram and the list cursor).
#include "misa_common.hpp"
#include "misa_internal.hpp"
#include "misa_score_dev.hpp"

namespace misa {
namespace {

constexpr int kThreads = 1024;               // 16 waves: four per SIMD hide LDS and barrier latency
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;
constexpr int kMaxChunks = 1024;
constexpr int kSpec = 4;                     // candidate entries each thread requests before knowing m
constexpr int kCandCap = kSpec * kThreads;   // candidates held in LDS

// state[t][*]: written by chunk 0 of the filter launch
enum { ST_B1 = 0, ST_KREM1 = 1, ST_M = 2 };
// counter[t][*]
enum { CT_CAND = 0 };

__device__ __forceinline__ int64_t row_len_of(const TopkArgs& a, int64_t t, int& p) {
  p = query_prefix_len(a.q_seq, a.q_len, a.nseq, a.Lmax, t);
  if (p < 0) {
    p = 0;
    return 0;
  }
  return a.imap ? a.kc : p;
}

// Output token id of score slot e (-1 for a skipped candidate) and its score.
__device__ __forceinline__ void out_entry(const int32_t* imap, int p, int64_t e, uint32_t u, int32_t& id,
                                          float& sc) {
  if (imap) {
    const int32_t v = imap[e];
    const bool ok = v >= 0 && v < p;
    id = ok ? v : -1;
    sc = ok ? key_score(u) : 0.f;
  } else {
    id = (int32_t)e;
    sc = key_score(u);
  }
}

// Sum over the workgroup (every thread gets it).
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* wsum) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wsum[wave] = v;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += wsum[w];
  __syncthreads();
  return tot;
}

// Exclusive prefix sum over the workgroup's threads (ascending thread id).
__device__ __forceinline__ uint32_t excl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t pre = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pre += w < wave ? wsum[w] : 0u;
  __syncthreads();
  return pre + inc - v;
}

// Digit d of an NB-bin histogram (scanned from the top) at which the running
// count reaches krem: count(bins > d) < krem <= count(bins >= d). Every thread
// returns the same (digit, krem - count(bins > d)).
template <int NB>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t krem, uint32_t* wsum, uint32_t* sh,
                                           uint32_t& digit, uint32_t& krem_out) {
  constexpr int PER = NB >= kThreads ? NB / kThreads : 1;
  const int tid = threadIdx.x;
  uint32_t c[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int b = PER * tid + j;
    c[j] = b < NB ? hist[NB - 1 - b] : 0u;
    mine += c[j];
  }
  uint32_t above = excl_scan(mine, wsum);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (above < krem && above + c[j] >= krem) {
      sh[0] = (uint32_t)(NB - 1 - (PER * tid + j));
      sh[1] = krem - above;
    }
    above += c[j];
  }
  __syncthreads();
  digit = sh[0];
  krem_out = sh[1];
  __syncthreads();
}

// The chunk of a workgroup is kThreads * EPT consecutive scores; wave w owns the
// contiguous run [64 * EPT * w, 64 * EPT * (w + 1)) of it, lane l holds
// elements 64 * j + l of that run (j < EPT): every load is a coalesced 256-byte
// row, and index order is (wave, j, lane).
template <int EPT>
__device__ __forceinline__ void load_chunk(const float* row, int64_t e0, int64_t n, uint32_t (&u)[EPT],
                                           bool (&in)[EPT]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = e0 + (int64_t)wave * 64 * EPT + lane;
  float v[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int64_t e = base + 64 * j;
    in[j] = e < n;
    v[j] = in[j] ? row[e] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) u[j] = score_key(v[j]);
}

template <int EPT>
__global__ __launch_bounds__(kThreads) void split_hist_kernel(TopkArgs a, SplitTopkWs w) {
  __shared__ uint32_t lh[kBins];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x;
  int p;
  const int64_t n = row_len_of(a, t, p);
  const int64_t e0 = (int64_t)c * kThreads * EPT;
  if (n <= a.k || e0 >= n) return;
  uint32_t u[EPT];
  bool in[EPT];
  load_chunk<EPT>(a.scores + t * a.stride, e0, n, u, in);
  for (int i = tid; i < kBins; i += kThreads) lh[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if (in[j]) atomicAdd(&lh[u[j] >> 20], 1u);
  __syncthreads();
  uint32_t* gh = w.hist + t * kBins;
  for (int i = tid; i < kBins; i += kThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Every chunk finds the row's threshold bin b1 from the finished histogram,
// counts its keys above b1 and appends the keys of bin b1 (key, index) to the
// row's candidate list (one cursor reservation per workgroup).
template <int EPT>
__global__ __launch_bounds__(kThreads) void split_filter_kernel(TopkArgs a, SplitTopkWs w) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wcnt[kWaves], wdef[kWaves], wbase[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x;
  int p;
  const int64_t n = row_len_of(a, t, p);
  const int64_t e0 = (int64_t)c * kThreads * EPT;
  if (n <= a.k || e0 >= n) return;
  uint32_t u[EPT];
  bool in[EPT];
  load_chunk<EPT>(a.scores + t * a.stride, e0, n, u, in);
  const uint32_t* gh = w.hist + t * kBins;
  for (int i = tid; i < kBins; i += kThreads) lh[i] = gh[i];
  __syncthreads();
  uint32_t b1, krem1;
  find_digit<kBins>(lh, (uint32_t)a.k, wsum, sh, b1, krem1);
  if (c == 0 && tid == 0) {
    uint32_t* st = w.state + t * 8;
    st[ST_B1] = b1;
    st[ST_KREM1] = krem1;
    st[ST_M] = lh[b1];
  }
  uint32_t ndef = 0, ncand = 0;
  uint64_t mk[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const uint32_t bin = u[j] >> 20;
    ndef += (in[j] && bin > b1) ? 1u : 0u;
    mk[j] = __ballot(in[j] && bin == b1);
    ncand += (uint32_t)__popcll(mk[j]);
  }
  ndef = wave_sum(ndef);
  if (lane == 0) {
    wdef[wave] = ndef;
    wcnt[wave] = ncand;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t tot = 0, nd = 0;
    for (int ww = 0; ww < kWaves; ++ww) {
      tot += wcnt[ww];
      nd += wdef[ww];
    }
    uint32_t b = tot ? atomicAdd(w.counter + t * 4 + CT_CAND, tot) : 0u;
    for (int ww = 0; ww < kWaves; ++ww) {
      wbase[ww] = b;
      b += wcnt[ww];
    }
    w.ndef[t * w.nchunk + c] = nd;
  }
  __syncthreads();
  uint2* cand = reinterpret_cast<uint2*>(w.cand) + t * w.cap;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t run = wbase[wave];
  const int64_t base = e0 + (int64_t)wave * 64 * EPT + lane;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const uint32_t pos = run + (uint32_t)__popcll(mk[j] & lt);
    if (((mk[j] >> lane) & 1ull) && pos < (uint32_t)w.cap) cand[pos] = uint2{u[j], (uint32_t)(base + 64 * j)};
    run += (uint32_t)__popcll(mk[j]);
  }
}

// Visit the m candidates of a row (cached in LDS, or read from global memory
// 8 per thread per round with all loads issued first).
template <typename F>
__device__ __forceinline__ void for_candidates(const uint2* gl, const uint2* lds, uint32_t m, F&& f) {
  if (lds) {
    for (uint32_t i = threadIdx.x; i < m; i += kThreads) {
      const uint2 v = lds[i];
      f(v.x, v.y);
    }
    return;
  }
  for (uint32_t b = 0; b < m; b += 8 * kThreads) {
    uint2 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t i = b + q * kThreads + threadIdx.x;
      v[q] = i < m ? gl[i] : uint2{0u, 0xffffffffu};
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (v[q].y != 0xffffffffu) f(v[q].x, v[q].y);
  }
}

// Every chunk resolves the row's exact k-th key u* from the candidate list
// (three more digits: bits 19..12, 11..4, 3..0), counts the selected keys in
// front of it (keys above b1 from the filter's per-chunk counts, plus the
// candidates above / equal to u* with a lower index), then writes its selected
// indices in index order.
// RESCORE (the coarse pass of the fused MISA† pipeline): the kept tokens of the
// chunk are then scored with all H heads (D-dim keys, RT row tiles) into the
// candidate-slot score row r.scores, and the re-rank's level-1 histogram of
// those scores is accumulated into r.hist; slots beyond a short prefix are
// marked -1 / -inf.
template <int EPT, int D, int RT, bool RESCORE>
__global__ __launch_bounds__(kThreads) void split_compact_kernel(TopkArgs a, SplitTopkWs w, RescoreArgs r) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wgt[kWaves], weq[kWaves], wend[kWaves];
  __shared__ uint2 ccache[kCandCap];
  __shared__ int s_tok[RESCORE ? kThreads * EPT : 1];
  constexpr int LDQ = D + 8;   // padded row stride of the staged query rows (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t s_q[RESCORE ? 16 * RT * LDQ : 8];
  __shared__ float s_w[RESCORE ? 16 * RT : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x;
  int p;
  const int64_t n = row_len_of(a, t, p);
  const float* row = a.scores + t * a.stride;
  int32_t* oi = a.idx + t * (int64_t)a.k;
  float* os = a.score ? a.score + t * (int64_t)a.k : nullptr;
  const int32_t* imap = a.imap ? a.imap + t * (int64_t)a.kc : nullptr;
  constexpr int CH = kThreads * EPT;
  const int64_t e0 = (int64_t)c * CH;

  // dense query rows (all heads) staged in LDS for the re-scoring; requested
  // first so that the loads overlap the selection
  const uint16_t* kseq = nullptr;
  if constexpr (RESCORE) {
    const int seq = a.q_seq[t];
    kseq = r.k + (int64_t)((seq >= 0 && seq < a.nseq) ? seq : 0) * a.Lmax * D + grp * 8;
    constexpr int PIECES = 16 * RT * D / 8;   // 16-byte pieces of the padded row block
    for (int i = tid; i < PIECES; i += kThreads) {
      const int rr = i / (D / 8), cc = (i % (D / 8)) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rr < r.H) v = *reinterpret_cast<const u32x4*>(r.q + (t * r.H + rr) * D + cc);
      *reinterpret_cast<u32x4*>(s_q + rr * LDQ + cc) = v;
    }
    if (tid < 16 * RT) s_w[tid] = tid < r.H ? r.w[t * r.H + tid] : 0.f;
  }
  uint32_t off = 0, nsel = 0;

  if (n <= a.k) {
    const int64_t e1 = min(e0 + CH, n);
    if constexpr (RESCORE) {
      for (int i = tid; i < kBins; i += kThreads) lh[i] = 0;
    }
    for (int64_t e = e0 + tid; e < e1; e += kThreads) {
      int32_t id;
      float sc;
      out_entry(imap, p, e, score_key(row[e]), id, sc);
      oi[e] = id;
      if (os) os[e] = sc;
      if constexpr (RESCORE) s_tok[e - e0] = (int)e;
    }
    if constexpr (RESCORE) {
      off = (uint32_t)e0;
      nsel = e1 > e0 ? (uint32_t)(e1 - e0) : 0u;
      __syncthreads();
    }
    // padding [n, k), spread over the row's chunks
    for (int64_t j = n + (int64_t)c * kThreads + tid; j < a.k; j += (int64_t)w.nchunk * kThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.f;
      if constexpr (RESCORE) {
        r.scores[t * (int64_t)a.k + j] = -INFINITY;
        atomicAdd(&lh[score_key(-INFINITY) >> 20], 1u);
      }
    }
    if constexpr (!RESCORE) return;
  } else {
    if (e0 >= n) return;
    // ---- everything independent is requested at once
    const uint32_t* st = w.state + t * 8;
    const uint32_t b1 = st[ST_B1], m_all = st[ST_M];
    uint32_t krem = st[ST_KREM1];
    const uint32_t nd_mine = tid < c ? w.ndef[t * w.nchunk + tid] : 0u;
    const uint2* gcand = reinterpret_cast<const uint2*>(w.cand) + t * w.cap;
    uint2 spec[kSpec];
#pragma unroll
    for (int q = 0; q < kSpec; ++q) spec[q] = gcand[q * kThreads + tid];   // within the list's capacity
    uint32_t u[EPT];
    bool in[EPT];
    load_chunk<EPT>(row, e0, n, u, in);
    const uint32_t m = min(m_all, (uint32_t)w.cap);
    const uint2* lds = nullptr;
    if (m <= (uint32_t)kCandCap) {
#pragma unroll
      for (int q = 0; q < kSpec; ++q)
        if ((uint32_t)(q * kThreads + tid) < m) ccache[q * kThreads + tid] = spec[q];
      lds = ccache;
    }
    for (int i = tid; i < 256; i += kThreads) lh[i] = 0;
    __syncthreads();
    // ---- exact k-th key: digits 19..12, 11..4, 3..0 on the candidates (all share b1)
    uint32_t prefix = b1 << 20, pmask = 0xfff00000u;
    const int shifts[3] = {12, 4, 0};
    const uint32_t masks[3] = {0xffu, 0xffu, 0xfu};
#pragma unroll
    for (int lv = 0; lv < 3; ++lv) {
      const int shift = shifts[lv];
      const uint32_t dm = masks[lv];
      for_candidates(gcand, lds, m, [&](uint32_t uu, uint32_t) {
        if ((uu & pmask) == prefix) atomicAdd(&lh[(uu >> shift) & dm], 1u);
      });
      __syncthreads();
      uint32_t dg, kr;
      if (lv < 2) find_digit<256>(lh, krem, wsum, sh, dg, kr);
      else find_digit<16>(lh, krem, wsum, sh, dg, kr);
      prefix |= dg << shift;
      pmask |= dm << shift;
      krem = kr;
      for (int i = tid; i < 256; i += kThreads) lh[i] = 0;
      __syncthreads();
    }
    const uint32_t ustar = prefix;   // the k-th key; krem keys equal to it are kept (lowest indices)
    // ---- selected keys in front of this chunk
    uint32_t gtb = 0, eqb = 0;
    for_candidates(gcand, lds, m, [&](uint32_t uu, uint32_t e) {
      if ((int64_t)e < e0) {
        gtb += uu > ustar ? 1u : 0u;
        eqb += uu == ustar ? 1u : 0u;
      }
    });
    const uint32_t gt_before = block_sum(gtb, wsum);
    const uint32_t eq_before = block_sum(eqb, wsum);
    const uint32_t nd_before = block_sum(nd_mine, wsum);
    const uint32_t sel_before = nd_before + gt_before + (eq_before < krem ? eq_before : krem);
    if constexpr (RESCORE) {
      for (int i = tid; i < kBins; i += kThreads) lh[i] = 0;   // the re-rank histogram from here on
    }
    // ---- compaction of this chunk (from registers)
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      cgt += (in[j] && u[j] > ustar) ? 1u : 0u;
      ceq += (in[j] && u[j] == ustar) ? 1u : 0u;
    }
    cgt = wave_sum(cgt);
    ceq = wave_sum(ceq);
    if (lane == 0) {
      wgt[wave] = cgt;
      weq[wave] = ceq;
    }
    __syncthreads();
    uint32_t eq_run = eq_before, sel_run = sel_before;
    for (int ww = 0; ww < wave; ++ww) {
      const uint32_t take = eq_run >= krem ? 0u : min(weq[ww], krem - eq_run);
      sel_run += wgt[ww] + take;
      eq_run += weq[ww];
    }
    const uint64_t lt = (1ull << lane) - 1ull;
    const int64_t base = e0 + (int64_t)wave * 64 * EPT + lane;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const bool gt = in[j] && u[j] > ustar;
      const bool eq = in[j] && u[j] == ustar;
      const uint64_t meq = __ballot(eq);
      const uint32_t eq_rank = eq_run + (uint32_t)__popcll(meq & lt);
      const bool sel = gt || (eq && eq_rank < krem);
      const uint64_t msel = __ballot(sel);
      const uint32_t pos = sel_run + (uint32_t)__popcll(msel & lt);
      if (sel && pos < (uint32_t)a.k) {
        int32_t id;
        float sc;
        out_entry(imap, p, base + 64 * j, u[j], id, sc);
        oi[pos] = id;
        if (os) os[pos] = sc;
        if constexpr (RESCORE) s_tok[pos - sel_before] = (int)(base + 64 * j);
      }
      eq_run += (uint32_t)__popcll(meq);
      sel_run += (uint32_t)__popcll(msel);
    }
    if constexpr (!RESCORE) return;
    if (lane == 0) wend[wave] = sel_run;
    __syncthreads();
    off = sel_before;
    const uint32_t last = wend[kWaves - 1] < (uint32_t)a.k ? wend[kWaves - 1] : (uint32_t)a.k;
    nsel = last > off ? last - off : 0u;
  }

  if constexpr (RESCORE) {
    // ---- dense scores of the chunk's kept tokens (slots off .. off + nsel), one 16-key tile per wave
    float* rrow = r.scores + t * (int64_t)a.k;
    for (int b = wave * 16; b < (int)nsel; b += kWaves * 16) {
      KeyTiles<D, 1> tile;
      load_key_tiles<D, 1>(kseq, b, (int)nsel, col, [&](int s) { return s_tok[s]; }, tile);
      const float v = score_one_tile_lds<D, RT>(s_q, LDQ, s_w, tile, grp, col);
      if (grp == 0 && b + col < (int)nsel) {
        rrow[off + b + col] = v;
        atomicAdd(&lh[score_key(v) >> 20], 1u);
      }
    }
    __syncthreads();
    uint32_t* gh = r.hist + t * kBins;
    for (int i = tid; i < kBins; i += kThreads)
      if (lh[i]) atomicAdd(&gh[i], lh[i]);
  }
}

// Scores per chunk: 4096 (4 per thread) for long rows, 1024 for shorter ones
// so that a row still spreads over several workgroups.
inline int split_ept(int64_t max_len) { return max_len >= 65536 ? 4 : 1; }
inline int split_chunk(int64_t max_len) { return kThreads * split_ept(max_len); }

inline size_t al(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool use_split_topk(int64_t T, int64_t max_len) {
  // rows of up to 12288 scores are selected from LDS by one workgroup each
  return T <= 4096 && max_len > 12288 && max_len <= (int64_t)kMaxChunks * kThreads * 4;
}

int64_t split_topk_zero_words(int64_t T) { return (int64_t)(al((size_t)T * (kBins + 4) * 4) / 4); }

inline int64_t cand_cap(int64_t max_len) { return max_len > kCandCap ? max_len : kCandCap; }

size_t split_topk_ws_bytes(int64_t T, int64_t max_len) {
  const int chunk = split_chunk(max_len);
  const int64_t nchunk = (max_len + chunk - 1) / chunk;
  return al((size_t)T * (kBins + 4) * 4) + al((size_t)T * 8 * 4) + 3 * al((size_t)T * nchunk * 4) +
         al((size_t)T * cand_cap(max_len) * 8);
}

SplitTopkWs split_topk_carve(void* base, int64_t T, int64_t max_len) {
  SplitTopkWs w{};
  w.chunk = split_chunk(max_len);
  w.nchunk = (int)((max_len + w.chunk - 1) / w.chunk);
  w.cap = cand_cap(max_len);
  char* p = static_cast<char*>(base);
  // zeroed region first: histogram and counters
  w.hist = reinterpret_cast<uint32_t*>(p);
  w.counter = w.hist + T * kBins;
  p += al((size_t)T * (kBins + 4) * 4);
  w.state = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * 8 * 4);
  w.ndef = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.ccnt = reinterpret_cast<uint32_t*>(p);   // unused
  p += al((size_t)T * w.nchunk * 4);
  w.eqb = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.cand = reinterpret_cast<uint32_t*>(p);
  return w;
}

hipError_t launch_topk_split(const TopkArgs& a, const SplitTopkWs& w, bool hist_done, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  dim3 grid(w.nchunk, (unsigned)a.T);
  RescoreArgs none{};
  if (w.chunk == kThreads * 4) {
    if (!hist_done) hipLaunchKernelGGL(split_hist_kernel<4>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL(split_filter_kernel<4>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL((split_compact_kernel<4, 32, 1, false>), grid, dim3(kThreads), 0, st, a, w, none);
  } else {
    if (!hist_done) hipLaunchKernelGGL(split_hist_kernel<1>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL(split_filter_kernel<1>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL((split_compact_kernel<1, 32, 1, false>), grid, dim3(kThreads), 0, st, a, w, none);
  }
  return hipGetLastError();
}

namespace {
template <int EPT, int D>
hipError_t launch_rescore_d(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, hipStream_t st) {
  dim3 grid(w.nchunk, (unsigned)a.T);
  hipLaunchKernelGGL(split_filter_kernel<EPT>, grid, dim3(kThreads), 0, st, a, w);
  switch ((r.H + 15) / 16) {
    case 1: hipLaunchKernelGGL((split_compact_kernel<EPT, D, 1, true>), grid, dim3(kThreads), 0, st, a, w, r); break;
    case 2: hipLaunchKernelGGL((split_compact_kernel<EPT, D, 2, true>), grid, dim3(kThreads), 0, st, a, w, r); break;
    case 3: hipLaunchKernelGGL((split_compact_kernel<EPT, D, 3, true>), grid, dim3(kThreads), 0, st, a, w, r); break;
    default: hipLaunchKernelGGL((split_compact_kernel<EPT, D, 4, true>), grid, dim3(kThreads), 0, st, a, w, r); break;
  }
  return hipGetLastError();
}
template <int EPT>
hipError_t launch_rescore_e(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, hipStream_t st) {
  switch (r.d) {
    case 32: return launch_rescore_d<EPT, 32>(a, w, r, st);
    case 64: return launch_rescore_d<EPT, 64>(a, w, r, st);
    case 128: return launch_rescore_d<EPT, 128>(a, w, r, st);
    case 256: return launch_rescore_d<EPT, 256>(a, w, r, st);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_topk_split_rescore(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  return w.chunk == kThreads * 4 ? launch_rescore_e<4>(a, w, r, st) : launch_rescore_e<1>(a, w, r, st);
}

bool split_topk_always_ok(int64_t max_len) { return max_len <= (int64_t)kMaxChunks * kThreads * 4; }

}  // namespace misa
