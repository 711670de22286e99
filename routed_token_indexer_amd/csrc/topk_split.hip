// Split per-query top-k for few, long score rows (decode: a handful of queries
// over 10^4..10^6 tokens), where one workgroup per row would leave the chip idle.
//
// Same selection rule as the per-row kernels (MISA pages: the indexer keeps the
// top-k tokens of each query; order by score descending, token index
// ascending; output in ascending token index, -1 padded), computed over
// (row, chunk) grids after a level-1 histogram of each row (the key's top 12
// bits; the decode scoring kernel usually builds it, else `hist` below):
//   - up to 256 rows of scores (decode batches): one launch, split_select_kernel.
//     Each chunk lists its members, the keys in the threshold bin b1 or above it
//     (a superset of its share of the top-k), and adds their next 12 key bits
//     to the row's level-2 histogram; the chunk that arrives last on a row
//     resolves the exact threshold key and writes the row's selection. With RR
//     (the fused MISA† step, k' <= 8192) every chunk first scores its members
//     with all heads, and the last chunk also selects the final top-k by those
//     dense scores.
//   - more rows, or rows of candidate slots (an index map): two launches.
//       filter   each chunk finds b1, counts its keys above b1, appends the
//                keys of b1 (key, index) to the row's candidate list and counts
//                their next 12 key bits into the row's level-2 histogram;
//       compact  each chunk resolves the exact threshold key from the level-2
//                histogram (and, when its threshold sub-bin is not kept whole,
//                the low 8 bits of that sub-bin's few candidates) and its own
//                output offset from the candidates' per-chunk counts, then
//                writes its kept indices in index order from that offset; with
//                RESCORE (MISA† with k' > 8192) it scores them with all heads.
//     Every chunk of the compaction works the threshold out for itself, so no
//     chunk waits for another within a launch.
// The one-launch form hands the members on to the last chunk through
// device-coherent stores (sc1: written through to memory, which every XCD's
// loads with sc1 see) completed before an atomic arrival count; the L2
// write-back fence that a release would add costs more than the whole
// selection on gfx950.
#include "misa_common.hpp"
#include "misa_internal.hpp"
#include "misa_score_dev.hpp"
#include "misa_select.hpp"

namespace misa {
namespace {

constexpr int kThreads = kSelThreads;       // 16 waves: four per SIMD hide LDS and barrier latency
constexpr int kWaves = kThreads / 64;
constexpr int kBins = kSelBins;
constexpr int kMaxChunks = 1024;
constexpr int kCandReg = 8 * kThreads;       // candidates a compaction chunk holds in registers
constexpr int kOneLaunchRows = 256;          // rows of the one-launch split selection at most
constexpr int kSplitShortRows = 64;          // rows at most for the split selection of rows <= 32K

// state[t][*]: the row's level-1 threshold bin, how many of its keys are kept,
// and how many keys it holds (written by the filter launch's first chunk)
enum { ST_B1 = 0, ST_KREM1 = 1, ST_M = 2 };
// counter[t][*] (zero on entry): candidate-list cursor (two-launch form),
// arrivals of the one-launch selection
enum { CT_CAND = 0, CT_ARRIVE = 2 };

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
    if (lh[i]) atomicAdd(&gh[hist_word(i)], lh[i]);
}

// Every chunk finds the row's threshold bin b1 from the finished histogram,
// counts its keys above b1 and appends the keys of bin b1 (key, index) to the
// row's candidate list (one cursor reservation per workgroup), and counts key
// bits 8..19 of those keys into the row's level-2 histogram. The first chunk
// records b1, how many of its keys are kept and how many it holds; the
// compaction launch resolves the rest (resolve_threshold below).
template <int EPT>
__global__ __launch_bounds__(kThreads) void split_filter_kernel(TopkArgs a, SplitTopkWs w) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wsum[kWaves];
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
  // the row's histogram: all words requested before the first wait (a strided
  // copy loop would wait for each load in turn)
  const uint32_t* gh = w.hist + t * kBins;
  uint32_t hv[kBins / kThreads];
#pragma unroll
  for (int k = 0; k < kBins / kThreads; ++k) hv[k] = gh[tid + k * kThreads];
#pragma unroll
  for (int k = 0; k < kBins / kThreads; ++k) lh[hist_bin(tid + k * kThreads)] = hv[k];
  __syncthreads();
  find_threshold(lh, kBins, (uint32_t)a.k, wsum, sh);
  const uint32_t b1 = sh[0], krem1 = sh[1], m_all = lh[b1];
  uint32_t ndef = 0, ncand = 0;
  uint64_t mk[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const uint32_t bin = u[j] >> 20;
    ndef += (in[j] && bin > b1) ? 1u : 0u;
    mk[j] = __ballot(in[j] && bin == b1);
    ncand += (uint32_t)__popcll(mk[j]);
  }
  // level 2: bits 8..19 of the keys of bin b1
  uint32_t* h2 = w.hist2 + t * kBins;
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if ((mk[j] >> lane) & 1ull) atomicAdd(&h2[(u[j] >> 8) & 0xfffu], 1u);
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
    if (c == 0) {   // the row's threshold bin, found alike by every chunk
      w.state[t * 8 + ST_B1] = b1;
      w.state[t * 8 + ST_KREM1] = krem1;
      w.state[t * 8 + ST_M] = m_all;
    }
  }
  __syncthreads();
  uint64_t* cand = reinterpret_cast<uint64_t*>(w.cand) + t * w.cap;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t run = wbase[wave];
  const int64_t base = e0 + (int64_t)wave * 64 * EPT + lane;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const uint32_t pos = run + (uint32_t)__popcll(mk[j] & lt);
    if (((mk[j] >> lane) & 1ull) && pos < (uint32_t)w.cap)
      cand[pos] = ((uint64_t)(uint32_t)(base + 64 * j) << 32) | u[j];
    run += (uint32_t)__popcll(mk[j]);
  }
}

// The exact threshold of row t and the output offset of chunk c, worked out by
// every chunk of the compaction launch from what the filter launch left: the
// threshold bin b1 and how many of its keys are kept (krem1), the candidate list
// (key, index) of bin b1, the level-2 histogram of those keys' bits 8..19 and each
// chunk's count of keys above b1.
//   - level 2: the threshold sub-bin b2 of the candidates; when it is not kept
//     whole, a 256-bin histogram of the low 8 bits of its keys (usually one or
//     two) gives the rest of the threshold key thr, and how many keys equal to
//     thr are kept (krem; all of them when b2 is kept whole);
//   - this chunk's output offset: the keys the chunks before it keep (their keys
//     above b1, and their candidates above thr), plus as many of their
//     candidates equal to thr as are kept, which is also the number of keys
//     equal to thr in front of it.
// Every load (the list requested speculatively up to kCandReg entries) goes out
// with the chunk's own scores, so the resolution costs one memory round trip
// and a few barriers, and no chunk waits for another.
template <int EPT>
__device__ __forceinline__ void resolve_threshold(const TopkArgs& a, const SplitTopkWs& w, int64_t t, int c,
                                                  int64_t n, const float* row, int64_t e0, uint32_t (&u)[EPT],
                                                  bool (&in)[EPT], uint32_t& thr, uint32_t& krem_eq,
                                                  uint32_t& sel_before, uint32_t& eq_before) {
  __shared__ uint32_t s_h[kBins];
  __shared__ uint32_t s_h3[256];
  __shared__ uint32_t s_ws[3][2 * kWaves];
  __shared__ uint32_t s_o[3][4];
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int CH = kThreads * EPT;
  const int nact = (int)((n + CH - 1) / CH);
  // ---- every request at once
  const uint32_t* st = w.state + t * 8;
  const uint32_t b1 = st[ST_B1], krem1 = st[ST_KREM1], m_all = st[ST_M];
  const uint64_t* cand = reinterpret_cast<const uint64_t*>(w.cand) + t * w.cap;
  uint64_t cv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {   // list slots past the list's length are masked below
    const int64_t i = 8 * tid + j;
    cv[j] = cand[i < w.cap ? i : w.cap - 1];
  }
  constexpr int H2PT = kBins / kThreads;
  uint32_t h2v[H2PT];
#pragma unroll
  for (int k = 0; k < H2PT; ++k) h2v[k] = w.hist2[t * kBins + tid + k * kThreads];
  const uint32_t nd_l = w.ndef[t * w.nchunk + (tid < nact ? tid : 0)];
  load_chunk<EPT>(row, e0, n, u, in);
  const uint32_t m = m_all < (uint32_t)w.cap ? m_all : (uint32_t)w.cap;
  const bool inreg = m <= (uint32_t)kCandReg;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (!inreg || (uint32_t)(8 * tid + j) >= m) cv[j] = 0ull;
  // visit(f): f(key, index) for each candidate of this thread
  auto visit = [&](auto&& f) {
    if (inreg) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((uint32_t)(8 * tid + j) < m) f((uint32_t)cv[j], (uint32_t)(cv[j] >> 32));
    } else {
      for (uint32_t i = tid; i < m; i += kThreads) {
        const uint64_t x = cand[i];
        f((uint32_t)x, (uint32_t)(x >> 32));
      }
    }
  };
#pragma unroll
  for (int k = 0; k < H2PT; ++k) s_h[tid + k * kThreads] = h2v[k];
  if (tid < 256) s_h3[tid] = 0u;
  __syncthreads();
  // ---- level 2 (and 3): the threshold key
  find_threshold(s_h, kBins, krem1, s_ws[0], s_o[0]);
  const uint32_t b2 = s_o[0][0], krem2 = s_o[0][1];
  if (s_o[0][2]) {
    // the sub-bin is kept whole: every key from its lowest value up
    thr = (b1 << 20) | (b2 << 8);
    krem_eq = 0xffffffffu;
  } else {
    visit([&](uint32_t key, uint32_t) {
      if (((key >> 8) & 0xfffu) == b2) atomicAdd(&s_h3[key & 0xffu], 1u);
    });
    __syncthreads();
    find_threshold(s_h3, 256, krem2, s_ws[1], s_o[1]);
    thr = (b1 << 20) | (b2 << 8) | s_o[1][0];
    krem_eq = s_o[1][1];   // all 32 bits resolved: the first krem_eq keys equal to thr
  }
  // ---- what the chunks before this one keep: their keys above b1 and their
  // candidates above thr, and their candidates equal to thr (a candidate lies
  // in an earlier chunk when its index is below this chunk's first one)
  const int64_t e0c = e0;
  uint32_t g = tid < c ? nd_l : 0u, q = 0u;
  visit([&](uint32_t key, uint32_t idx) {
    if ((int64_t)idx < e0c) {
      g += key > thr ? 1u : 0u;
      q += key == thr ? 1u : 0u;
    }
  });
  g = wave_sum(g);
  q = wave_sum(q);
  if (lane == 0) {
    s_ws[2][tid >> 6] = g;
    s_ws[2][kWaves + (tid >> 6)] = q;
  }
  __syncthreads();
  uint32_t gtb = 0, eqb = 0;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) {
    gtb += s_ws[2][ww];
    eqb += s_ws[2][kWaves + ww];
  }
  sel_before = gtb + (eqb < krem_eq ? eqb : krem_eq);
  eq_before = eqb;
}

// Every chunk writes its kept indices in index order: the keys above the row's
// threshold key thr, and of the keys equal to thr those ranked (in index
// order) below krem. thr, krem, its output offset and the number of keys equal
// to thr in front of it come from resolve_threshold.
// RESCORE (the coarse pass of the fused MISA† pipeline): the kept tokens of the
// chunk are then scored with all H heads (D-dim keys, RT row tiles) into the
// candidate-slot score row r.scores (and, with r.hist, the re-rank's level-1
// histogram of those scores); slots beyond a short prefix are marked -1 / -inf.
template <int EPT, int D, int RT, bool RESCORE>
__global__ __launch_bounds__(kThreads) void split_compact_kernel(TopkArgs a, SplitTopkWs w, RescoreArgs r) {
  __shared__ uint32_t lh[RESCORE ? kBins : 1];
  __shared__ uint32_t wgt[kWaves], weq[kWaves], wend[kWaves];
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

  // dense query rows (all heads) for the re-scoring: requested first, held in
  // registers while the selection runs, and staged in LDS (stage_q) only before
  // the barrier that precedes the re-scoring, so that no wait for them comes
  // earlier
  const uint16_t* kseq = nullptr;
  constexpr int PIECES = 16 * RT * D / 8;   // 16-byte pieces of the padded row block
  constexpr int QPT = RESCORE ? (PIECES + kThreads - 1) / kThreads : 1;
  // (loads from clamped addresses; rows past H are zeroed only when staged)
  u32x4 qv[QPT];
  float wq = 0.f;
  if constexpr (RESCORE) {
    const int seq = a.q_seq[t];
    kseq = r.k + (int64_t)((seq >= 0 && seq < a.nseq) ? seq : 0) * a.Lmax * D + grp * 8;
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = tid + k * kThreads;
      const int rr = i / (D / 8), cc = (i % (D / 8)) * 8;
      const bool ok = i < PIECES && rr < r.H;
      qv[k] = *reinterpret_cast<const u32x4*>(r.q + (t * r.H + (ok ? rr : 0)) * D + (ok ? cc : 0));
    }
    wq = r.w[t * r.H + (tid < r.H ? tid : 0)];
    if (r.hist)
      for (int i = tid; i < kBins; i += kThreads) lh[i] = 0;
  }
  auto stage_q = [&]() {
    if constexpr (RESCORE) {
#pragma unroll
      for (int k = 0; k < QPT; ++k) {
        const int i = tid + k * kThreads;
        const int rr = i / (D / 8), cc = (i % (D / 8)) * 8;
        if (i < PIECES) *reinterpret_cast<u32x4*>(s_q + rr * LDQ + cc) = rr < r.H ? qv[k] : u32x4{0u, 0u, 0u, 0u};
      }
      if (tid < 16 * RT) s_w[tid] = tid < r.H ? wq : 0.f;
    }
  };
  uint32_t off = 0, nsel = 0;

  if (n <= a.k) {
    const int64_t e1 = min(e0 + CH, n);
    for (int64_t e = e0 + tid; e < e1; e += kThreads) {
      int32_t id;
      float sc;
      out_entry(imap, p, e, score_key(row[e]), id, sc);
      oi[e] = id;
      if constexpr (RESCORE) s_tok[e - e0] = (int)e;
      if (os) os[e] = sc;
    }
    if constexpr (RESCORE) {
      off = (uint32_t)e0;
      nsel = e1 > e0 ? (uint32_t)(e1 - e0) : 0u;
      stage_q();
      __syncthreads();
    }
    // padding [n, k), spread over the row's chunks
    for (int64_t j = n + (int64_t)c * kThreads + tid; j < a.k; j += (int64_t)w.nchunk * kThreads) {
      if (os) os[j] = 0.f;
      oi[j] = -1;
      if constexpr (RESCORE) {
        r.scores[t * (int64_t)a.k + j] = -INFINITY;
        if (r.hist) atomicAdd(&lh[score_key(-INFINITY) >> 20], 1u);
      }
    }
    if constexpr (!RESCORE) return;
  } else {
    if (e0 >= n) return;
    uint32_t ustar, krem, sel_before, eq_before;
    uint32_t u[EPT];
    bool in[EPT];
    resolve_threshold<EPT>(a, w, t, c, n, row, e0, u, in, ustar, krem, sel_before, eq_before);
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
        if constexpr (RESCORE) s_tok[pos - sel_before] = (int)(base + 64 * j);
        if (os) os[pos] = sc;
      }
      eq_run += (uint32_t)__popcll(meq);
      sel_run += (uint32_t)__popcll(msel);
    }
    if constexpr (!RESCORE) return;
    stage_q();
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
      load_key_tiles<D, 1>(kseq, b, (int)nsel, col, [&](int s) { return s_tok[s]; }, 0, tile);
      const float v = score_one_tile_lds<D, RT>(s_q, LDQ, s_w, tile, grp, col);
      if (grp == 0 && b + col < (int)nsel) {
        rrow[off + b + col] = v;
        if (r.hist) atomicAdd(&lh[score_key(v) >> 20], 1u);
      }
    }
    if (r.hist) {
      __syncthreads();
      uint32_t* gh = r.hist + t * kBins;
      for (int i = tid; i < kBins; i += kThreads)
        if (lh[i]) atomicAdd(&gh[hist_word(i)], lh[i]);
    }
  }
}

// The split selection in one launch (one workgroup per (chunk, row), the
// rows' level-1 histogram already built). Without RR it selects the top-k of
// the rows (k = a.k) and writes it with its scores. With RR it is the MISA†
// step: coarse top-k' (k' = a.k <= 8192), dense re-scoring and fine top-k:
//   - Members of a chunk: for a row of more than k' visible tokens, its keys in
//     the level-1 threshold bin b1 or above it. That is a superset of the
//     chunk's share of the exact top-k': all the keys above b1 are in it, and of
//     the keys of b1 only krem1 are. For a row of at most k' tokens, every
//     visible token is a member and is kept.
//   - Each chunk (RR: scores its members with all H heads and) stores them in
//     index order as (index, routed key) (RR: and dense score) in its own region
//     of the row's member lists; it adds key bits 8..19 of its members in b1 to
//     the row's level-2 histogram, stores its member count (RR: and dense-key
//     range) and counts its arrival (everything written through before the
//     count).
//   - The chunk that arrives last resolves the exact top-k' among the members
//     (level 2 from the histogram, level 3 over the members of the threshold
//     sub-bin): the kept ones are above the threshold key, or equal to it and
//     among the first krem in index order. Without RR it writes them, with their
//     scores, as the row's selection. With RR it writes their indices as the
//     candidate list (ascending, -1 padded to k') and selects the final top-k
//     among them by dense score out of registers: a histogram of the dense keys
//     over their range, then the few keys of the threshold bin ranked in LDS.
// Compared with the filter and compaction launches (and for RR a fine-stage
// select), this saves a launch, (RR: the exact threshold's round before the
// re-scoring and the candidate list's round trip through memory). The price is
// the single workgroup per row that finishes, and with RR re-scoring the members
// of b1 that are not kept, usually a few thousand keys of a 128K row.
template <int EPT, int D, int RT, bool RR>
__global__ __launch_bounds__(kThreads) void split_select_kernel(TopkArgs a, SplitTopkWs w, RescoreArgs r,
                                                                float* mscore) {
  constexpr int CH = kThreads * EPT;
  constexpr int LDQ = D + 8;    // padded row stride of the staged query rows (bf16)
  constexpr int G = 8, NS = 2;  // last chunk: members per lane and chunk in registers, chunks per wave
  constexpr int kCand = 512;    // keys of the fine threshold bin ranked in LDS
  // histograms: the routed keys' level 1, then the last chunk's coarse level 2
  // and the fine selection's fallback
  __shared__ __attribute__((aligned(16))) RadixScratch<kThreads, 1> rs;
  uint32_t* const lh = rs.hist[0];
  __shared__ uint32_t lf[RR ? kBins : 1];   // the fine level 1
  __shared__ uint32_t s_h3[256];
  __shared__ uint32_t sh[3][4];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[4][kWaves];
  __shared__ uint32_t wcnt[kWaves];
  __shared__ int s_tok[RR ? CH : 1];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[RR ? 16 * RT * LDQ : 8];
  __shared__ float s_w[RR ? 16 * RT : 1];
  __shared__ uint32_t s_last, s_mm[2];
  // the last chunk, per chunk: members; coarse and fine counts and offsets
  __shared__ uint32_t s_cnt[kMaxChunks], s_gt[kMaxChunks], s_eq[kMaxChunks];
  __shared__ uint32_t s_fgt[RR ? kMaxChunks : 1], s_feq[RR ? kMaxChunks : 1];
  __shared__ uint32_t s_tot, s_nc, s_nc2, s_fthr, s_fkrem;
  // keys of the coarse threshold sub-bin, then of the fine threshold bin, with their chunks
  __shared__ uint32_t c_key[kCand], c_ch[kCand];
  __shared__ uint64_t c_kw[RR ? kCand : 1];   // the fine bin's keys: key | weight << 32
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x;
  int p;
  const int64_t n = row_len_of(a, t, p);
  const int nact = n > 0 ? (int)((n + CH - 1) / CH) : 1;   // chunk 0 always takes part
  if (c >= nact) return;
  const int64_t e0 = (int64_t)c * CH;
  const bool all = n <= a.k;   // every visible token is a candidate

  // ---- every request at once: query rows and weights (RR), the chunk's
  // routed scores, the row's level-1 histogram
  const uint16_t* kseq = nullptr;
  constexpr int PIECES = 16 * RT * D / 8;   // 16-byte pieces of the padded row block
  constexpr int QPT = (PIECES + kThreads - 1) / kThreads;
  u32x4 qv[QPT];
  float wq = 0.f;
  if constexpr (RR) {
    const int seq = a.q_seq[t];
    kseq = r.k + (int64_t)((seq >= 0 && seq < a.nseq) ? seq : 0) * a.Lmax * D + grp * 8;
#pragma unroll
    for (int k = 0; k < QPT; ++k) {   // (clamped addresses; rows past H are zeroed when staged)
      const int i = tid + k * kThreads;
      const int rr = i / (D / 8), cc = (i % (D / 8)) * 8;
      const bool ok = i < PIECES && rr < r.H;
      qv[k] = *reinterpret_cast<const u32x4*>(r.q + (t * r.H + (ok ? rr : 0)) * D + (ok ? cc : 0));
    }
    wq = r.w[t * r.H + (tid < r.H ? tid : 0)];
  }
  uint32_t u[EPT];
  bool in[EPT];
  load_chunk<EPT>(a.scores + t * a.stride, e0, n, u, in);
  constexpr int HPT = kBins / kThreads;
  uint32_t b1 = 0u, krem1 = 0u;
  if (!all) {
    uint32_t hv[HPT];
#pragma unroll
    for (int k = 0; k < HPT; ++k) hv[k] = w.hist[t * kBins + tid + k * kThreads];
#pragma unroll
    for (int k = 0; k < HPT; ++k) lh[hist_bin(tid + k * kThreads)] = hv[k];
    __syncthreads();
    find_threshold(lh, kBins, (uint32_t)a.k, wsum[0], sh[0]);
    b1 = sh[0][0];
    krem1 = sh[0][1];
  }

  // ---- the chunk's members, in index order; the level-2 histogram of those in b1
  bool mem[EPT];
  uint32_t cm = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    mem[j] = in[j] && (all || (u[j] >> 20) >= b1);
    cm += (uint32_t)__popcll(__ballot(mem[j]));
  }
  if (lane == 0) wcnt[wave] = cm;
  if (tid == 0) {
    s_mm[0] = 0xffffffffu;
    s_mm[1] = 0u;
  }
  __syncthreads();
  uint32_t run = 0, nsel = 0;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) {
    run += ww < wave ? wcnt[ww] : 0u;
    nsel += wcnt[ww];
  }
  const int64_t cap = w.cap;
  uint64_t* const mlist = reinterpret_cast<uint64_t*>(w.cand) + t * cap;
  float* const mrow = RR ? mscore + t * cap : nullptr;
  uint32_t* const h2 = w.hist2 + t * kBins;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int64_t base = e0 + (int64_t)wave * 64 * EPT + lane;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const uint64_t mk = __ballot(mem[j]);
    const uint32_t pos = run + (uint32_t)__popcll(mk & lt);
    if (mem[j]) {
      if constexpr (RR) s_tok[pos] = (int)(base + 64 * j);
      store_coherent(mlist + e0 + pos, ((uint64_t)(uint32_t)(base + 64 * j) << 32) | u[j]);
      if (!all && (u[j] >> 20) == b1) (void)atomic_add_coherent(h2 + ((u[j] >> 8) & 0xfffu), 1u);
    }
    run += (uint32_t)__popcll(mk);
  }
  if constexpr (RR) {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int i = tid + k * kThreads;
      const int rr = i / (D / 8), cc = (i % (D / 8)) * 8;
      if (i < PIECES) *reinterpret_cast<u32x4*>(s_q + rr * LDQ + cc) = rr < r.H ? qv[k] : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 16 * RT) s_w[tid] = tid < r.H ? wq : 0.f;
    __syncthreads();

    // ---- dense scores of the members, one 16-key tile per wave, and their key range
    uint32_t mlo = 0xffffffffu, mhi = 0u;
    for (int b = wave * 16; b < (int)nsel; b += kWaves * 16) {
      KeyTiles<D, 1> tile;
      load_key_tiles<D, 1>(kseq, b, (int)nsel, col, [&](int s) { return s_tok[s]; }, 0, tile);
      const float v = score_one_tile_lds<D, RT>(s_q, LDQ, s_w, tile, grp, col);
      if (grp == 0 && b + col < (int)nsel) {
        store_coherent(mrow + e0 + b + col, v);
        mlo = min(mlo, score_key(v));
        mhi = max(mhi, score_key(v));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mlo = min(mlo, (uint32_t)__shfl_xor((int)mlo, off, kWave));
      mhi = max(mhi, (uint32_t)__shfl_xor((int)mhi, off, kWave));
    }
    if (lane == 0) {
      atomicMin(&s_mm[0], mlo);
      atomicMax(&s_mm[1], mhi);
    }
  }
  // per chunk: member count (RR: and the smallest and largest dense key)
  uint32_t* const cinfo = w.ndef + (int64_t)a.T * w.nchunk + (t * w.nchunk) * 3;
  if constexpr (RR) __syncthreads();
  if (tid == 0) {
    store_coherent(cinfo + 3 * c, nsel);
    if constexpr (RR) {
      store_coherent(cinfo + 3 * c + 1, s_mm[0]);
      store_coherent(cinfo + 3 * c + 2, s_mm[1]);
    }
  }
  // ---- arrival: this chunk's members, count and range are in memory before it counts
  wait_stores();
  __syncthreads();
  if (tid == 0) s_last = atomic_add_coherent(w.counter + t * 4 + CT_ARRIVE, 1u) == (uint32_t)nact - 1 ? 1u : 0u;
  if (tid == 0) {   // for the last chunk's reduction of the ranges
    s_mm[0] = 0xffffffffu;
    s_mm[1] = 0u;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the last chunk. The members of chunk c2 are the first cnt(c2) entries
  // of its region, in index order; wave w takes the chunks w, w + kWaves, ...
  // and lane l the entries l, l + 64, ... of each, G at a time. When every chunk
  // fits (at most NS per wave, 64 * G members each), all of them stay in
  // registers (loaded with the counts, before the counts are known); otherwise
  // every pass loads them again.
  const uint32_t cnt_l = tid < nact ? load_coherent(cinfo + 3 * tid) : 0u;
  uint32_t klo = RR && tid < nact ? load_coherent(cinfo + 3 * tid + 1) : 0xffffffffu;
  uint32_t khi = RR && tid < nact ? load_coherent(cinfo + 3 * tid + 2) : 0u;
  uint32_t h2v[HPT];
#pragma unroll
  for (int k = 0; k < HPT; ++k) h2v[k] = all ? 0u : load_coherent(h2 + tid + k * kThreads);
  uint64_t rx[NS][G];
  float rd[NS][G];
  const int64_t slot_max = n > 0 ? n - 1 : 0;
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) {
    const int c2 = wave + s2 * kWaves;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int64_t slot = (int64_t)c2 * CH + g * 64 + lane;
      slot = slot < slot_max ? slot : slot_max;
      if (c2 < nact) {
        rx[s2][g] = load_coherent(mlist + slot);
        if constexpr (RR) rd[s2][g] = load_coherent(mrow + slot);
      }
    }
  }
  if (tid < nact) {
    s_cnt[tid] = cnt_l;
    s_gt[tid] = 0u;
    s_eq[tid] = 0u;
    if constexpr (RR) {
      s_fgt[tid] = 0u;
      s_feq[tid] = 0u;
    }
  }
#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    lh[tid + k * kThreads] = h2v[k];
    if constexpr (RR) lf[tid + k * kThreads] = 0u;
  }
  if (tid < 256) s_h3[tid] = 0u;
  if (tid == 0) {
    s_nc = 0u;
    s_nc2 = 0u;
  }
  if constexpr (RR) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      klo = min(klo, (uint32_t)__shfl_xor((int)klo, off, kWave));
      khi = max(khi, (uint32_t)__shfl_xor((int)khi, off, kWave));
    }
    if (lane == 0 && khi >= klo) {
      atomicMin(&s_mm[0], klo);
      atomicMax(&s_mm[1], khi);
    }
  }
  uint32_t nbig;
  (void)block_excl_scan(cnt_l > 64u * G ? 1u : 0u, wsum[1], nbig);   // (its barrier publishes the above)
  const bool fast = nact <= NS * kWaves && nbig == 0;
  klo = s_mm[0];   // the members' dense-key range
  khi = s_mm[1];
  uint32_t rn[NS];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) rn[s2] = wave + s2 * kWaves < nact ? s_cnt[wave + s2 * kWaves] : 0u;
  // body(x, d, nb, c2, j0) for each block of G * 64 members: entry g of the lane
  // is member j0 + 64 * g + lane of chunk c2, valid when 64 * g + lane < nb;
  // a chunk's blocks come in order, from j0 = 0
  auto each_block = [&](auto&& body) {
    if (fast) {
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
        if (wave + s2 * kWaves < nact) body(rx[s2], rd[s2], rn[s2], wave + s2 * kWaves, 0u);
    } else {
      for (int c2 = wave; c2 < nact; c2 += kWaves) {
        const uint32_t cn = s_cnt[c2];
        for (uint32_t j0 = 0; j0 < cn; j0 += 64u * G) {
          uint64_t x[G];
          float d[G];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const uint32_t j = j0 + (uint32_t)(g * 64 + lane);
            const int64_t slot = j < cn ? (int64_t)c2 * CH + j : 0;
            x[g] = load_coherent(mlist + slot);
            if constexpr (RR) d[g] = load_coherent(mrow + slot);
          }
          body(x, d, cn - j0, c2, j0);
        }
      }
    }
  };
  // ---- coarse threshold: the k'-th largest routed key thr, and how many of
  // the members equal to it are kept (the first krem_eq in index order); per
  // chunk, its members above thr (s_gt) and equal to it (s_eq)
  // (predicates below are combined with & and |, not && and ||: no branch per entry)
  uint32_t thr = 0u, krem_eq = 0xffffffffu;
  if (all) {
    if (tid < nact) s_gt[tid] = s_cnt[tid];   // every member is kept
  } else {
    // level 2: bits 8..19 of the keys of b1 (every one of them is a member)
    find_threshold(lh, kBins, krem1, wsum[0], sh[1]);
    const uint32_t b2 = sh[1][0], krem2 = sh[1][1];
    const bool whole = sh[1][2] != 0u;   // the threshold sub-bin is kept whole
    for (int i = tid; i < kBins; i += kThreads) lh[i] = 0u;   // for the fine selection's fallback
    const uint32_t hi24 = (b1 << 12) | b2;
    if (whole) thr = hi24 << 8;
    // one pass: per chunk, the members above sub-bin b2, and when it is kept
    // whole those in it too; otherwise the level-3 histogram of the low 8 bits
    // of its members, which are listed with their chunk
    each_block([&](auto& x, auto&, uint32_t nb, int c2, uint32_t) {
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g * 64 >= (int)nb) break;   // (the rest of the block lies past its members)
        const uint32_t key = (uint32_t)x[g];
        const bool v = (uint32_t)(g * 64 + lane) < nb;
        const bool mid = v & ((key >> 8) == hi24);
        gt += (uint32_t)__popcll(__ballot(v & ((key >> 8) > hi24)));
        if (whole) {
          gt += (uint32_t)__popcll(__ballot(mid & (key > thr)));
          eq += (uint32_t)__popcll(__ballot(mid & (key == thr)));
        } else if (mid) {
          atomicAdd(&s_h3[key & 0xffu], 1u);
          const uint32_t s = atomicAdd(&s_nc2, 1u);
          if (s < (uint32_t)kCand) {
            c_key[s] = key & 0xffu;
            c_ch[s] = (uint32_t)c2;
          }
        }
      }
      if (lane == 0) {
        s_gt[c2] += gt;
        s_eq[c2] += eq;
      }
    });
    __syncthreads();
    if (!whole) {
      // level 3, then each listed member above thr or at it counts in its chunk
      if (wave == 0) find_threshold_wave(s_h3, 256, krem2, sh[2]);
      __syncthreads();
      const uint32_t lo8 = sh[2][0];
      thr = (hi24 << 8) | lo8;
      krem_eq = sh[2][1];
      const uint32_t nc2 = s_nc2;
      if (nc2 <= (uint32_t)kCand) {
        if (tid < (int)nc2) {
          if (c_key[tid] > lo8) atomicAdd(&s_gt[c_ch[tid]], 1u);
          if (c_key[tid] == lo8) atomicAdd(&s_eq[c_ch[tid]], 1u);
        }
      } else {
        // more members in the sub-bin than the list holds (heavy ties): count them again
        each_block([&](auto& x, auto&, uint32_t nb, int c2, uint32_t) {
          uint32_t gt = 0, eq = 0;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (g * 64 >= (int)nb) break;
            const uint32_t key = (uint32_t)x[g];
            const bool mid = ((uint32_t)(g * 64 + lane) < nb) & ((key >> 8) == hi24);
            gt += (uint32_t)__popcll(__ballot(mid & (key > thr)));
            eq += (uint32_t)__popcll(__ballot(mid & (key == thr)));
          }
          if (lane == 0) {
            s_gt[c2] += gt;
            s_eq[c2] += eq;
          }
        });
      }
      __syncthreads();
    }
  }
  // over the chunks in order: selected members and members at the threshold
  // before each chunk (sg, se), and in the whole row (s_tot)
  // (up to 64 chunks: wave 0 alone, one chunk per lane)
  auto chunk_offsets = [&](uint32_t* sg, uint32_t* se, uint32_t kr) {
    uint32_t gt = 0, eq = 0, gt_before = 0, eq_before = 0;
    if (nact <= 64) {
      if (wave == 0) {
        gt = lane < nact ? sg[lane] : 0u;
        eq = lane < nact ? se[lane] : 0u;
        gt_before = wave_incl_scan(gt) - gt;
        eq_before = wave_incl_scan(eq) - eq;
      }
    } else {
      gt = tid < nact ? sg[tid] : 0u;
      eq = tid < nact ? se[tid] : 0u;
      gt_before = block_excl_scan2(gt, eq, &wsum[2][0], eq_before);
    }
    if (tid < nact) {
      sg[tid] = gt_before + (eq_before < kr ? eq_before : kr);
      se[tid] = eq_before;
    }
    if (tid == nact - 1) s_tot = gt_before + gt + (eq_before + eq < kr ? eq_before + eq : kr);
    __syncthreads();
  };
  chunk_offsets(s_gt, s_eq, krem_eq);
  // coarse selection of a block's entries (bit g of the mask): above thr, or
  // equal to it and among the first krem_eq such in index order; eq_run counts
  // the members equal to thr before the block
  auto coarse_kept = [&](auto& x, uint32_t nb, uint32_t& eq_run) {
    uint32_t m = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g * 64 >= (int)nb) break;
      const uint32_t key = (uint32_t)x[g];
      const bool v = (uint32_t)(g * 64 + lane) < nb;
      const bool eq = v & (key == thr);
      const uint64_t meq = __ballot(eq);
      const bool sel = (v & (key > thr)) | (eq & (eq_run + lanes_below(meq) < krem_eq));
      m |= sel ? 1u << g : 0u;
      eq_run += (uint32_t)__popcll(meq);
    }
    return m;
  };
  if constexpr (!RR) {
    // ---- the selection: kept members at their output slots (index order) with
    // their scores, then -1 and 0
    int32_t* const oi = a.idx + t * (int64_t)a.k;
    float* const os = a.score ? a.score + t * (int64_t)a.k : nullptr;
    auto emit = [&](auto& x, uint32_t m, uint32_t nb, uint32_t& sel_run) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g * 64 >= (int)nb) break;
        const bool sel = (m >> g) & 1u;
        const uint64_t msel = __ballot(sel);
        const uint32_t pos = sel_run + lanes_below(msel);
        if (sel & (pos < (uint32_t)a.k)) {   // (every kept member's slot is below k)
          oi[pos] = (int32_t)(x[g] >> 32);
          if (os) os[pos] = key_score((uint32_t)x[g]);
        }
        sel_run += (uint32_t)__popcll(msel);
      }
    };
    if (fast) {
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const int c2 = wave + s2 * kWaves;
        if (c2 < nact) {
          uint32_t eq_run = s_eq[c2], sel_run = s_gt[c2];
          emit(rx[s2], coarse_kept(rx[s2], rn[s2], eq_run), rn[s2], sel_run);
        }
      }
    } else {
      uint32_t eq_run = 0, sel_run = 0;
      each_block([&](auto& x, auto&, uint32_t nb, int c2, uint32_t j0) {
        if (j0 == 0) {
          eq_run = s_eq[c2];
          sel_run = s_gt[c2];
        }
        emit(x, coarse_kept(x, nb, eq_run), nb, sel_run);
      });
    }
    for (int64_t j = (all ? n : (int64_t)a.k) + tid; j < a.k; j += kThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.f;
    }
    return;
  }
  // ---- the candidate list: kept members at their slots (index order), -1 after
  // them. The fine selection ranks their dense-score keys less the smallest of
  // the members' (flo); level 1 takes the top 12 of the range's bits. When the
  // row has fewer than k' visible tokens, its k' - n empty candidate slots take
  // part with the key of -inf, after every member in slot order.
  const uint32_t kpad = score_key(-INFINITY);
  const uint32_t npad = all ? (uint32_t)(a.k - n) : 0u;
  const uint32_t flo = npad ? min(klo, kpad) : klo, fhi = npad ? max(khi, kpad) : khi;
  const int nbits = fhi > flo ? 32 - __clz((int)(fhi - flo)) : 0;
  const int fsh = nbits > 12 ? nbits - 12 : 0;
  int32_t* const oi = a.idx + t * (int64_t)a.k;
  uint32_t km[NS];       // (fast) coarse selection of the lane's entries
  uint32_t fkr[NS][G];   // (fast) their dense-score keys
  {
    auto emit = [&](auto& x, auto& fk, uint32_t m, uint32_t nb, uint32_t& sel_run) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g * 64 >= (int)nb) break;
        const bool sel = (m >> g) & 1u;
        const uint64_t msel = __ballot(sel);
        const uint32_t pos = sel_run + lanes_below(msel);
        if (sel & (pos < (uint32_t)a.k)) {   // (every kept member's slot is below k')
          oi[pos] = (int32_t)(x[g] >> 32);
          atomicAdd(&lf[(fk[g] - flo) >> fsh], 1u);
        }
        sel_run += (uint32_t)__popcll(msel);
      }
    };
    if (fast) {
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const int c2 = wave + s2 * kWaves;
        km[s2] = 0u;
        if (c2 < nact) {
          uint32_t eq_run = s_eq[c2], sel_run = s_gt[c2];
          km[s2] = coarse_kept(rx[s2], rn[s2], eq_run);
#pragma unroll
          for (int g = 0; g < G; ++g) fkr[s2][g] = score_key(rd[s2][g]);
          emit(rx[s2], fkr[s2], km[s2], rn[s2], sel_run);
        }
      }
    } else {
      uint32_t eq_run = 0, sel_run = 0;
      each_block([&](auto& x, auto& d, uint32_t nb, int c2, uint32_t j0) {
        if (j0 == 0) {
          eq_run = s_eq[c2];
          sel_run = s_gt[c2];
        }
        const uint32_t m = coarse_kept(x, nb, eq_run);
        uint32_t fk[G];
#pragma unroll
        for (int g = 0; g < G; ++g) fk[g] = score_key(d[g]);
        emit(x, fk, m, nb, sel_run);
      });
    }
  }
  for (int64_t j = (all ? n : (int64_t)a.k) + tid; j < a.k; j += kThreads) oi[j] = -1;
  if (tid == 0 && npad) atomicAdd(&lf[(kpad - flo) >> fsh], npad);
  // body(fk, m, x, nb, c2, j0) for each block: dense keys, coarse selection, members
  auto each_kept = [&](auto&& body) {
    if (fast) {
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
        if (wave + s2 * kWaves < nact) body(fkr[s2], km[s2], rx[s2], rn[s2], wave + s2 * kWaves, 0u);
    } else {
      uint32_t eq_run = 0;
      each_block([&](auto& x, auto& d, uint32_t nb, int c2, uint32_t j0) {
        if (j0 == 0) eq_run = s_eq[c2];
        const uint32_t m = coarse_kept(x, nb, eq_run);
        uint32_t fk[G];
#pragma unroll
        for (int g = 0; g < G; ++g) fk[g] = score_key(d[g]);
        body(fk, m, x, nb, c2, j0);
      });
    }
  };
  __syncthreads();
  // ---- fine threshold: the rule keeps the kept members whose key less flo,
  // masked by fmask, is above fpre, and of those equal to fpre the first fkrem
  find_threshold(lf, kBins, (uint32_t)r.ftopk, wsum[0], sh[0]);
  const uint32_t d0 = sh[0][0];
  uint32_t fpre = d0 << fsh, fmask = 0xfffu << fsh, fkrem = sh[0][1];
  // the bin decides when it holds whole keys or is kept whole; otherwise its
  // keys are ranked among themselves in LDS
  const bool by_bin = fsh == 0 || sh[0][2];
  // per chunk: kept members above bin d0 (and, when the bin decides, in it);
  // the keys of bin d0 listed with their chunk
  each_kept([&](auto& fk, uint32_t m, auto&, uint32_t nb, int c2, uint32_t) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g * 64 >= (int)nb) break;
      const uint32_t bin = (fk[g] - flo) >> fsh;
      const bool kept = (m >> g) & 1u;
      const bool inb = kept & (bin == d0);
      gt += (uint32_t)__popcll(__ballot(kept & (bin > d0)));
      eq += (uint32_t)__popcll(__ballot(inb));
      if (inb & !by_bin) {
        const uint32_t s = atomicAdd(&s_nc, 1u);
        if (s < (uint32_t)kCand) {
          c_kw[s] = (1ull << 32) | fk[g];
          c_ch[s] = (uint32_t)c2;
        }
      }
    }
    if (lane == 0) {
      s_fgt[c2] += gt;
      s_feq[c2] += by_bin ? eq : 0u;
    }
  });
  if (!by_bin && tid == 0 && npad && ((kpad - flo) >> fsh) == d0) {
    const uint32_t s = atomicAdd(&s_nc, 1u);
    if (s < (uint32_t)kCand) {
      c_kw[s] = ((uint64_t)npad << 32) | kpad;
      c_ch[s] = 0xffffffffu;   // the empty slots: after every chunk
    }
  }
  __syncthreads();
  if (!by_bin) {
    const uint32_t nc = s_nc;
    if (nc <= (uint32_t)kCand) {
      // the key K with fewer than krem keys of the bin above it and at least
      // krem at or above it; krem - (keys above K) of those equal to K are kept
      // (a key with fewer than krem keys at or above it lies above K; each listed
      // key above K or at it counts in its chunk)
      const uint32_t kr = fkrem;
      if (tid < (int)nc) {
        const uint32_t ki = (uint32_t)c_kw[tid];
        uint32_t gt = 0, eq = 0;
        for (uint32_t j = 0; j < nc; j += 4) {   // four list reads in flight (weight 0 past the list)
          uint64_t e[4];
#pragma unroll
          for (int u2 = 0; u2 < 4; ++u2) e[u2] = j + u2 < nc ? c_kw[j + u2] : 0ull;
#pragma unroll
          for (int u2 = 0; u2 < 4; ++u2) {
            const uint32_t kj = (uint32_t)e[u2], wj = (uint32_t)(e[u2] >> 32);
            gt += kj > ki ? wj : 0u;
            eq += kj == ki ? wj : 0u;
          }
        }
        const bool at = (gt < kr) & (kr <= gt + eq);
        if (at) {
          s_fthr = ki;
          s_fkrem = kr - gt;
        }
        if (c_ch[tid] != 0xffffffffu) {
          if (gt + eq < kr) atomicAdd(&s_fgt[c_ch[tid]], 1u);
          if (at) atomicAdd(&s_feq[c_ch[tid]], 1u);
        }
      }
      __syncthreads();
      fpre = s_fthr - flo;
      fmask = 0xffffffffu;
      fkrem = s_fkrem;
    } else {
      // more keys in the bin than the list holds (heavy ties): radix select over
      // all of the kept members, then their counts per chunk again
      fkrem = (uint32_t)r.ftopk;
      bool full;
      radix_select<kThreads, 1>(
          [&](auto&& f) {
            each_kept([&](auto& fk, uint32_t m, auto&, uint32_t, int, uint32_t) {
#pragma unroll
              for (int g = 0; g < G; ++g)
                if ((m >> g) & 1u) f(fk[g] - flo);
            });
          },
          nbits, fpre, fmask, fkrem, full, rs, kpad - flo, npad);
      if (tid < nact) s_fgt[tid] = 0u;
      __syncthreads();
      each_kept([&](auto& fk, uint32_t m, auto&, uint32_t nb, int c2, uint32_t) {
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (g * 64 >= (int)nb) break;
          const uint32_t v = (fk[g] - flo) & fmask;
          const bool kept = (m >> g) & 1u;
          gt += (uint32_t)__popcll(__ballot(kept & (v > fpre)));
          eq += (uint32_t)__popcll(__ballot(kept & (v == fpre)));
        }
        if (lane == 0) {
          s_fgt[c2] += gt;
          s_feq[c2] += eq;
        }
      });
      __syncthreads();
    }
  }
  chunk_offsets(s_fgt, s_feq, fkrem);
  // ---- the final top-k in index order: token ids and dense scores, then -1 / 0
  int32_t* const fi = r.fidx + t * (int64_t)r.ftopk;
  float* const fs = r.fscore ? r.fscore + t * (int64_t)r.ftopk : nullptr;
  {
    uint32_t feq_run = 0, fsel_run = 0;
    each_kept([&](auto& fk, uint32_t m, auto& x, uint32_t nb, int c2, uint32_t j0) {
      if (j0 == 0) {
        feq_run = s_feq[c2];
        fsel_run = s_fgt[c2];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g * 64 >= (int)nb) break;
        const uint32_t v = (fk[g] - flo) & fmask;
        const bool kept = (m >> g) & 1u;
        const bool eq = kept & (v == fpre);
        const uint64_t meq = __ballot(eq);
        const bool sel = (kept & (v > fpre)) | (eq & (feq_run + lanes_below(meq) < fkrem));
        const uint64_t msel = __ballot(sel);
        const uint32_t pos = fsel_run + lanes_below(msel);
        if (sel & (pos < (uint32_t)r.ftopk)) {
          fi[pos] = (int32_t)(x[g] >> 32);
          if (fs) fs[pos] = key_score(fk[g]);
        }
        feq_run += (uint32_t)__popcll(meq);
        fsel_run += (uint32_t)__popcll(msel);
      }
    });
  }
  // after the selected members (ftopk of them, or fewer when empty candidate
  // slots were selected)
  for (int j = (int)s_tot + tid; j < r.ftopk; j += kThreads) {
    fi[j] = -1;
    if (fs) fs[j] = 0.f;
  }
}

// Scores per chunk: 4096 (4 per thread) for long rows, 1024 for shorter ones
// so that a row still spreads over several workgroups.
inline int split_ept(int64_t max_len) { return max_len >= 65536 ? 4 : 1; }
inline int split_chunk(int64_t max_len) { return kThreads * split_ept(max_len); }

inline size_t al(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool use_split_topk(int64_t T, int64_t max_len, bool hist_in_scoring) {
  if (T > 4096 || max_len > (int64_t)kMaxChunks * kThreads * 4) return false;
  // rows too long for the register select: split over chunks for a few rows,
  // or when the scoring kernel has built their histograms; a larger batch
  // without them (a slab of a long prefill) keeps the chip busy with one
  // workgroup per row, whose streaming select reads each row a few times
  // instead of building histograms with device-wide atomics
  if (max_len > topk_row_reg_max()) return T <= 256 || hist_in_scoring;
  // rows of 16K..32K scores in a small batch whose histogram the scoring kernel
  // builds: the one-launch selection over chunks beats a workgroup per row;
  // shorter rows, or rows needing a histogram launch, take one workgroup each
  return hist_in_scoring && T <= kSplitShortRows && max_len > 16384;
}

int64_t split_topk_zero_words(int64_t T) { return (int64_t)(al((size_t)T * (2 * kBins + 4) * 4) / 4); }

inline int64_t cand_cap(int64_t max_len) { return max_len; }

size_t split_topk_ws_bytes(int64_t T, int64_t max_len) {
  const int chunk = split_chunk(max_len);
  const int64_t nchunk = (max_len + chunk - 1) / chunk;
  return al((size_t)T * (2 * kBins + 4) * 4) + al((size_t)T * 8 * 4) + al((size_t)T * nchunk * 4 * 4) +
         al((size_t)T * cand_cap(max_len) * 8);
}

SplitTopkWs split_topk_carve(void* base, int64_t T, int64_t max_len) {
  SplitTopkWs w{};
  w.chunk = split_chunk(max_len);
  w.nchunk = (int)((max_len + w.chunk - 1) / w.chunk);
  w.cap = cand_cap(max_len);
  char* p = static_cast<char*>(base);
  // zeroed region first: histograms and counters
  w.hist = reinterpret_cast<uint32_t*>(p);
  w.hist2 = w.hist + T * kBins;
  w.counter = w.hist2 + T * kBins;
  p += al((size_t)T * (2 * kBins + 4) * 4);
  w.state = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * 8 * 4);
  w.ndef = reinterpret_cast<uint32_t*>(p);   // (and after it, per chunk, three words of the MISA† selection)
  p += al((size_t)T * w.nchunk * 4 * 4);
  w.cand = reinterpret_cast<uint32_t*>(p);
  return w;
}

hipError_t launch_topk_split(const TopkArgs& a, const SplitTopkWs& w, bool hist_done, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  dim3 grid(w.nchunk, (unsigned)a.T);
  RescoreArgs none{};
  // rows of scores in place (not of candidate slots), up to kOneLaunchRows of
  // them: one launch after the histogram, its last workgroup per row selecting
  const bool one = !a.imap && a.T <= kOneLaunchRows;
  if (w.chunk == kThreads * 4) {
    if (!hist_done) hipLaunchKernelGGL(split_hist_kernel<4>, grid, dim3(kThreads), 0, st, a, w);
  } else {
    if (!hist_done) hipLaunchKernelGGL(split_hist_kernel<1>, grid, dim3(kThreads), 0, st, a, w);
  }
  if (one) {
    // chunks of 4096 scores whatever the histogram's chunking: fewer members
    // for the last workgroup to gather (chunk indices stay below w.nchunk)
    dim3 g4((unsigned)((w.nchunk * (int64_t)w.chunk + kThreads * 4 - 1) / (kThreads * 4)), (unsigned)a.T);
    hipLaunchKernelGGL((split_select_kernel<4, 32, 1, false>), g4, dim3(kThreads), 0, st, a, w, none, nullptr);
  } else if (w.chunk == kThreads * 4) {
    hipLaunchKernelGGL(split_filter_kernel<4>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL((split_compact_kernel<4, 32, 1, false>), grid, dim3(kThreads), 0, st, a, w, none);
  } else {
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

namespace {
template <int EPT, int D>
void launch_hier_d(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, float* mscore, hipStream_t st) {
  dim3 grid(w.nchunk, (unsigned)a.T);
  switch ((r.H + 15) / 16) {
    case 1: hipLaunchKernelGGL((split_select_kernel<EPT, D, 1, true>), grid, dim3(kThreads), 0, st, a, w, r, mscore); break;
    case 2: hipLaunchKernelGGL((split_select_kernel<EPT, D, 2, true>), grid, dim3(kThreads), 0, st, a, w, r, mscore); break;
    case 3: hipLaunchKernelGGL((split_select_kernel<EPT, D, 3, true>), grid, dim3(kThreads), 0, st, a, w, r, mscore); break;
    default: hipLaunchKernelGGL((split_select_kernel<EPT, D, 4, true>), grid, dim3(kThreads), 0, st, a, w, r, mscore); break;
  }
}
template <int EPT>
hipError_t launch_hier_e(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, float* mscore,
                         hipStream_t st) {
  switch (r.d) {
    case 32: launch_hier_d<EPT, 32>(a, w, r, mscore, st); break;
    case 64: launch_hier_d<EPT, 64>(a, w, r, mscore, st); break;
    case 128: launch_hier_d<EPT, 128>(a, w, r, mscore, st); break;
    case 256: launch_hier_d<EPT, 256>(a, w, r, mscore, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_hier_select(const TopkArgs& a, const SplitTopkWs& w, const RescoreArgs& r, float* mscore,
                              hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (a.imap || a.k > 8192 || r.ftopk > a.k) return hipErrorInvalidValue;
  return w.chunk == kThreads * 4 ? launch_hier_e<4>(a, w, r, mscore, st) : launch_hier_e<1>(a, w, r, mscore, st);
}

bool split_topk_always_ok(int64_t max_len) { return max_len <= (int64_t)kMaxChunks * kThreads * 4; }

}  // namespace misa
