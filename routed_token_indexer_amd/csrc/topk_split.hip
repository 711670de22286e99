// Split per-query top-k for few, long score rows (decode: a handful of queries
// over 10^4..10^6 tokens), where one workgroup per row would leave the chip idle.
//
// Same selection rule as the per-row kernels (MISA pages: the indexer keeps the
// top-k tokens of each query; order by score descending, token index
// ascending; output in ascending token index, -1 padded), computed by launches
// over (row, chunk) grids:
//   1. hist     each chunk adds its LDS histogram of the key's top 12 bits into
//               the row's global histogram (atomics; the decode scoring kernel
//               usually builds it instead).
//   2. filter   each chunk reads the finished histogram, finds the threshold
//               bin b1, counts its keys above b1, appends the keys of bin b1
//               (key, index) to the row's candidate list and counts their next
//               12 key bits into the row's level-2 histogram. The last chunk of
//               the row to finish resolves the exact threshold key from the
//               level-2 histogram (and, when its threshold bin is not kept
//               whole, the low 8 bits of that bin's few candidates) and turns
//               the per-chunk counts into per-chunk output offsets.
//   3. compact  each chunk writes its kept indices in index order from its
//               offset (ballots inside waves, counts across waves).
// Within a launch, chunks hand data to the last one through device-coherent
// stores (sc1: written through to memory, which every XCD's loads with sc1
// see) completed before an atomic arrival count; the L2 write-back fence that a
// release would add costs more than the whole selection on gfx950.
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
constexpr int kCandReg = 8 * kThreads;       // candidates the last chunk holds in registers

// state[t][*]: written by the last chunk of the filter launch
enum { ST_THR = 0, ST_KREM = 1 };
// counter[t][*] (zero on entry)
enum { CT_CAND = 0, CT_DONE = 1 };

__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this thread's stores have completed (for the sc1 stores above:
// reached memory).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// Every chunk finds the row's threshold bin b1 from the finished histogram,
// counts its keys above b1 and appends the keys of bin b1 (key, index) to the
// row's candidate list (one cursor reservation per workgroup), and counts key
// bits 8..19 of those keys into the row's level-2 histogram. The last chunk of
// the row to arrive then
//   - resolves the threshold key thr: the level-2 threshold bin b2 (all the
//     candidates share the top 12 bits b1); when b2 is not kept whole, a
//     256-bin histogram of the low 8 bits of its keys (usually one or two)
//     gives the rest, and how many keys equal to thr are kept (krem; all of
//     them when b2 is kept whole);
//   - counts the kept candidates of every chunk, and writes each chunk's output
//     offset (keys kept in the chunks before it) and the number of keys equal
//     to thr in front of it, for the compaction launch.
template <int EPT>
__global__ __launch_bounds__(kThreads) void split_filter_kernel(TopkArgs a, SplitTopkWs w) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t wcnt[kWaves], wdef[kWaves], wbase[kWaves];
  __shared__ uint32_t s_last;
  // the last chunk only
  __shared__ uint32_t s_p[kCandReg];   // level-3 histogram, then the list prefix
  __shared__ uint32_t wsum2[3][kWaves], sh2[4], sh3[4];
  __shared__ uint32_t cgt[kMaxChunks], ceq[kMaxChunks];
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
  for (int k = 0; k < kBins / kThreads; ++k) lh[tid + k * kThreads] = hv[k];
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
  // level 2: bits 8..19 of the keys of bin b1 (device-scope atomics, complete
  // before this chunk's arrival below)
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
    store_coherent(reinterpret_cast<uint64_t*>(w.seg) + t * w.nchunk + c, ((uint64_t)tot << 32) | b);
    for (int ww = 0; ww < kWaves; ++ww) {
      wbase[ww] = b;
      b += wcnt[ww];
    }
    store_coherent(w.ndef + t * w.nchunk + c, nd);
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
      store_coherent(cand + pos, ((uint64_t)(uint32_t)(base + 64 * j) << 32) | u[j]);
    run += (uint32_t)__popcll(mk[j]);
  }
  // ---- arrival: this chunk's list entries and count are in memory before it counts
  wait_stores();
  __syncthreads();
  const int nact = (int)((n + kThreads * EPT - 1) / (kThreads * EPT));
  if (tid == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(w.counter + t * 4 + CT_DONE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == (uint32_t)(nact - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the last chunk: exact threshold among the m candidates of bin b1.
  // Thread i holds list entries 8i .. 8i + 7, so that per-chunk counts are
  // differences of one prefix sum over the list order (each chunk appended its
  // candidates as one run).
  const uint32_t m = m_all < (uint32_t)w.cap ? m_all : (uint32_t)w.cap;
  const bool inreg = m <= (uint32_t)kCandReg;
  uint64_t cv[8];
  // unconditional loads from a clamped index (m >= 1: bin b1 holds the krem1-th
  // key), so that all of them go out before the first wait
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t i = (uint32_t)(8 * tid + j);
    const uint64_t x = load_coherent(cand + (i < m ? i : m - 1u));
    cv[j] = (inreg && i < m) ? x : 0ull;
  }
  const int tc = tid < nact ? tid : 0;
  const uint32_t nd_l = load_coherent(w.ndef + t * w.nchunk + tc);
  const uint64_t sg_l = load_coherent(reinterpret_cast<const uint64_t*>(w.seg) + t * w.nchunk + tc);
  // the level-2 histogram, requested with the list (one round trip for all)
  constexpr int H2PT = kBins / kThreads;
  uint32_t h2v[H2PT];
#pragma unroll
  for (int k = 0; k < H2PT; ++k) h2v[k] = load_coherent(w.hist2 + t * kBins + tid + k * kThreads);
  // visit(f): f(key, index) for each of this thread's candidates
  auto visit = [&](auto&& f) {
    if (inreg) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((uint32_t)(8 * tid + j) < m) f((uint32_t)cv[j], (uint32_t)(cv[j] >> 32));
    } else {
      for (uint32_t i = tid; i < m; i += kThreads) {
        const uint64_t x = load_coherent(cand + i);
        f((uint32_t)x, (uint32_t)(x >> 32));
      }
    }
  };
  if (!inreg)
    for (int i = tid; i < kMaxChunks; i += kThreads) {
      cgt[i] = 0;
      ceq[i] = 0;
    }
  // level 2: the threshold sub-bin b2 of bits 8..19 among the m keys of bin b1
  uint32_t* const h3 = s_p;   // level 3: 256 bins of the low 8 bits
  const uint32_t nd_c = tid < nact ? nd_l : 0u;
  const uint64_t sg = tid < nact ? sg_l : 0ull;
#pragma unroll
  for (int k = 0; k < H2PT; ++k) lh[tid + k * kThreads] = h2v[k];
  if (tid < 256) h3[tid] = 0u;
  __syncthreads();
  find_threshold(lh, kBins, krem1, wsum2[0], sh2);
  const uint32_t b2 = sh2[0], krem2 = sh2[1];
  uint32_t thr, krem_eq;
  if (sh2[2]) {
    // the sub-bin is kept whole: every key from its lowest value up
    thr = (b1 << 20) | (b2 << 8);
    krem_eq = 0xffffffffu;
  } else {
    // level 3: the low 8 bits of the (usually few) keys of sub-bin b2
    visit([&](uint32_t key, uint32_t) {
      if (((key >> 8) & 0xfffu) == b2) atomicAdd(&h3[key & 0xffu], 1u);
    });
    __syncthreads();
    find_threshold(h3, 256, krem2, wsum2[1], sh3);
    thr = (b1 << 20) | (b2 << 8) | sh3[0];
    krem_eq = sh3[1];   // all 32 bits resolved: the first krem_eq keys equal to thr
  }
  // ---- kept candidates of every chunk (keys above thr, keys equal to thr)
  uint32_t gt_c = 0, eq_c = 0;
  if (inreg) {
    // prefix over the list of (above << 16 | equal), m <= 8192 keeps both
    // halves below 2^16; the level-3 histogram is free again
    uint32_t* P = s_p;
    uint32_t loc[8], run = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t key = (uint32_t)cv[j];
      const bool ok = (uint32_t)(8 * tid + j) < m;
      run += ok ? (((key > thr) ? 1u << 16 : 0u) | (key == thr ? 1u : 0u)) : 0u;
      loc[j] = run;
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan(run, wsum2[0], tot);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((uint32_t)(8 * tid + j) < m) P[8 * tid + j] = pre + loc[j];
    __syncthreads();
    if (tid < nact) {
      const uint32_t start = (uint32_t)sg, cnt = (uint32_t)(sg >> 32);
      const uint32_t hiv = cnt ? P[start + cnt - 1] : 0u, lov = (cnt && start) ? P[start - 1] : 0u;
      gt_c = nd_c + ((hiv - lov) >> 16);
      eq_c = (hiv - lov) & 0xffffu;
    }
  } else {
    // long lists: one LDS atomic per (wave, chunk) group of list entries
    constexpr int CH = kThreads * EPT;
    auto count_chunks = [&](uint64_t x, bool valid) {   // called by the whole wave
      const uint32_t key = (uint32_t)x;
      const int cc = valid ? (int)((uint32_t)(x >> 32) / CH) : -1;
      const uint64_t mg = __ballot(valid && key > thr), mq = __ballot(valid && key == thr);
      uint64_t pending = __ballot(valid);
      while (pending) {
        const int leader = __ffsll((unsigned long long)pending) - 1;
        const int lc = __builtin_amdgcn_readlane(cc, leader);
        const uint64_t mask = __ballot(cc == lc) & pending;
        if (lane == leader) {
          const uint32_t ng = (uint32_t)__popcll(mg & mask), nq = (uint32_t)__popcll(mq & mask);
          if (ng) atomicAdd(&cgt[lc], ng);
          if (nq) atomicAdd(&ceq[lc], nq);
        }
        pending &= ~mask;
      }
    };
    for (uint32_t b0 = 0; b0 < m; b0 += kThreads) {
      const uint32_t i = b0 + tid;
      count_chunks(i < m ? load_coherent(cand + i) : 0ull, i < m);
    }
    __syncthreads();
    if (tid < nact) {
      gt_c = nd_c + cgt[tid];
      eq_c = ceq[tid];
    }
  }
  uint32_t eq_before;
  const uint32_t gt_before = block_excl_scan2(gt_c, eq_c, &wsum2[1][0], eq_before);
  if (tid < nact) {
    w.selb[t * w.nchunk + tid] = gt_before + (eq_before < krem_eq ? eq_before : krem_eq);
    w.eqb[t * w.nchunk + tid] = eq_before;
  }
  if (tid == 0) {
    w.state[t * 8 + ST_THR] = thr;
    w.state[t * 8 + ST_KREM] = krem_eq;
  }
}

// Every chunk writes its kept indices in index order: the keys above the row's
// threshold key thr, and of the keys equal to thr those ranked (in index
// order) below krem. Its output offset and the number of keys equal to thr in
// front of it come from the filter's last chunk.
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
      if (os) os[e] = sc;
      if constexpr (RESCORE) s_tok[e - e0] = (int)e;
    }
    if constexpr (RESCORE) {
      off = (uint32_t)e0;
      nsel = e1 > e0 ? (uint32_t)(e1 - e0) : 0u;
      stage_q();
      __syncthreads();
    }
    // padding [n, k), spread over the row's chunks
    for (int64_t j = n + (int64_t)c * kThreads + tid; j < a.k; j += (int64_t)w.nchunk * kThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.f;
      if constexpr (RESCORE) {
        r.scores[t * (int64_t)a.k + j] = -INFINITY;
        if (r.hist) atomicAdd(&lh[score_key(-INFINITY) >> 20], 1u);
      }
    }
    if constexpr (!RESCORE) return;
  } else {
    if (e0 >= n) return;
    const uint32_t* st = w.state + t * 8;
    const uint32_t ustar = st[ST_THR], krem = st[ST_KREM];
    const uint32_t sel_before = w.selb[t * w.nchunk + c], eq_before = w.eqb[t * w.nchunk + c];
    uint32_t u[EPT];
    bool in[EPT];
    load_chunk<EPT>(row, e0, n, u, in);
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
    if (!r.hist) return;
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
  // shorter rows are selected by one workgroup each, out of registers
  return T <= 4096 && max_len > topk_row_reg_max() && max_len <= (int64_t)kMaxChunks * kThreads * 4;
}

int64_t split_topk_zero_words(int64_t T) { return (int64_t)(al((size_t)T * (2 * kBins + 4) * 4) / 4); }

inline int64_t cand_cap(int64_t max_len) { return max_len; }

size_t split_topk_ws_bytes(int64_t T, int64_t max_len) {
  const int chunk = split_chunk(max_len);
  const int64_t nchunk = (max_len + chunk - 1) / chunk;
  return al((size_t)T * (2 * kBins + 4) * 4) + al((size_t)T * 8 * 4) + 3 * al((size_t)T * nchunk * 4) +
         al((size_t)T * nchunk * 8) + al((size_t)T * cand_cap(max_len) * 8);
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
  w.ndef = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.selb = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.eqb = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.seg = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 8);
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
