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

namespace misa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;
constexpr int kMaxChunks = 1024;

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

// Exclusive prefix sum over the 256 threads (ascending thread id); also returns the total.
__device__ __forceinline__ uint32_t excl_scan256(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = wsum[w];
    pre += w < wave ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return pre + inc - v;
}

// Digit d of an nb-bin histogram (scanned from the top) at which the running
// count reaches krem: count(bins > d) < krem <= count(bins >= d). Every thread
// returns the same (digit, krem - count(bins > d)).
template <int NB>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t krem, uint32_t* wsum, uint32_t* sh,
                                           uint32_t& digit, uint32_t& krem_out) {
  constexpr int PER = NB / kThreads;   // bins per thread (>= 1)
  const int tid = threadIdx.x;
  uint32_t c[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = hist[NB - 1 - (PER * tid + j)];
    mine += c[j];
  }
  uint32_t total;
  uint32_t above = excl_scan256(mine, wsum, total);
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

// The chunk of a workgroup is 256 * EPT consecutive scores; wave w owns the
// contiguous run [64 * EPT * w, 64 * EPT * (w + 1)) of it, lane l holds
// elements 64 * j + l of that run (j < EPT): every load is a coalesced 256-byte
// row, and index order is (wave, j, lane). All of a thread's loads are issued
// before any of them is used.
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
// counts its keys above b1 and appends the keys of bin b1 to the row's list
// (one cursor reservation per workgroup).
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
    const uint32_t tot = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    uint32_t b = tot ? atomicAdd(w.counter + t * 4 + CT_CAND, tot) : 0u;
    for (int ww = 0; ww < kWaves; ++ww) {
      wbase[ww] = b;
      b += wcnt[ww];
    }
    w.ndef[t * w.nchunk + c] = wdef[0] + wdef[1] + wdef[2] + wdef[3];
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

// Visit the m candidates of a row, 8 per thread per round with all loads issued first.
template <typename F>
__device__ __forceinline__ void for_candidates(const uint2* cand, uint32_t m, F&& f) {
  for (uint32_t b = 0; b < m; b += 8 * kThreads) {
    uint2 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t i = b + q * kThreads + threadIdx.x;
      v[q] = i < m ? cand[i] : uint2{0u, 0xffffffffu};
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (v[q].y != 0xffffffffu) f(v[q].x, v[q].y);
  }
}

// Every chunk resolves the row's exact k-th key u* from the candidate list
// (12 + 8 more bits), derives its own output offset from the counts of the
// chunks before it, then writes its selected indices in index order.
template <int EPT>
__global__ __launch_bounds__(kThreads) void split_compact_kernel(TopkArgs a, SplitTopkWs w) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t gtc[kMaxChunks], eqc[kMaxChunks];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t sh[4];
  __shared__ uint32_t wgt[kWaves], weq[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  if (n <= a.k) {
    const int64_t e1 = min(e0 + CH, n);
    for (int64_t e = e0 + tid; e < e1; e += kThreads) {
      int32_t id;
      float sc;
      out_entry(imap, p, e, score_key(row[e]), id, sc);
      oi[e] = id;
      if (os) os[e] = sc;
    }
    // padding [n, k), spread over the row's chunks
    for (int64_t j = n + (int64_t)c * kThreads + tid; j < a.k; j += (int64_t)w.nchunk * kThreads) {
      oi[j] = -1;
      if (os) os[j] = 0.f;
    }
    return;
  }
  if (e0 >= n) return;
  uint32_t u[EPT];
  bool in[EPT];
  load_chunk<EPT>(row, e0, n, u, in);
  const uint32_t* st = w.state + t * 8;
  const uint32_t b1 = st[ST_B1], m = min(st[ST_M], (uint32_t)w.cap);
  uint32_t krem = st[ST_KREM1];
  const uint2* cand = reinterpret_cast<const uint2*>(w.cand) + t * w.cap;
  // ---- exact k-th key: level 2 (bits 19..8), level 3 (bits 7..0) on the candidates
  uint32_t prefix = b1 << 20;
  for (int i = tid; i < kBins; i += kThreads) lh[i] = 0;
  for (int i = tid; i < c; i += kThreads) {
    gtc[i] = 0;
    eqc[i] = 0;
  }
  __syncthreads();
  for_candidates(cand, m, [&](uint32_t uu, uint32_t) { atomicAdd(&lh[(uu >> 8) & 0xfffu], 1u); });
  __syncthreads();
  uint32_t d2, krem2;
  find_digit<kBins>(lh, krem, wsum, sh, d2, krem2);
  prefix |= d2 << 8;
  krem = krem2;
  for (int i = tid; i < 256; i += kThreads) lh[i] = 0;
  __syncthreads();
  for_candidates(cand, m, [&](uint32_t uu, uint32_t) {
    if ((uu & 0xffffff00u) == prefix) atomicAdd(&lh[uu & 0xffu], 1u);
  });
  __syncthreads();
  uint32_t d3, krem3;
  find_digit<256>(lh, krem, wsum, sh, d3, krem3);
  const uint32_t ustar = prefix | d3;
  krem = krem3;   // keys equal to u* that are kept (the lowest indices)
  // ---- candidates above / equal to u* in the chunks before this one
  for_candidates(cand, m, [&](uint32_t uu, uint32_t e) {
    const int cc = (int)(e / (uint32_t)CH);
    if (cc < c) {
      if (uu > ustar) atomicAdd(&gtc[cc], 1u);
      else if (uu == ustar) atomicAdd(&eqc[cc], 1u);
    }
  });
  __syncthreads();
  // in chunk order: equal keys before chunk cc, and how many of them are kept
  constexpr int PER = kMaxChunks / kThreads;
  uint32_t eq_loc[PER], nd_loc[PER];
  uint32_t eq_mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int cc = PER * tid + j;
    eq_loc[j] = cc < c ? eqc[cc] : 0u;
    nd_loc[j] = cc < c ? w.ndef[t * w.nchunk + cc] + gtc[cc] : 0u;
    eq_mine += eq_loc[j];
  }
  uint32_t eq_tot;
  uint32_t eq_before = excl_scan256(eq_mine, wsum, eq_tot);
  uint32_t sel_mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t take = eq_before >= krem ? 0u : min(eq_loc[j], krem - eq_before);
    sel_mine += nd_loc[j] + take;
    eq_before += eq_loc[j];
  }
  uint32_t sel_tot;
  (void)excl_scan256(sel_mine, wsum, sel_tot);
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
  uint32_t eq_run = eq_tot, sel_run = sel_tot;
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
    }
    eq_run += (uint32_t)__popcll(meq);
    sel_run += (uint32_t)__popcll(msel);
  }
}

// Scores per chunk: 4096 (16 per thread) for long rows, 1024 for shorter ones
// so that a row still spreads over several workgroups.
inline int split_ept(int64_t max_len) { return max_len >= 65536 ? 16 : 4; }
inline int split_chunk(int64_t max_len) { return kThreads * split_ept(max_len); }

inline size_t al(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool use_split_topk(int64_t T, int64_t max_len) {
  // rows of up to 12288 scores are selected from LDS by one workgroup each
  return T <= 4096 && max_len > 12288 && max_len <= (int64_t)kMaxChunks * kThreads * 16;
}

int64_t split_topk_zero_words(int64_t T) { return (int64_t)(al((size_t)T * (kBins + 4) * 4) / 4); }

size_t split_topk_ws_bytes(int64_t T, int64_t max_len) {
  const int chunk = split_chunk(max_len);
  const int64_t nchunk = (max_len + chunk - 1) / chunk;
  return al((size_t)T * (kBins + 4) * 4) + al((size_t)T * 8 * 4) + 3 * al((size_t)T * nchunk * 4) +
         al((size_t)T * max_len * 8);
}

SplitTopkWs split_topk_carve(void* base, int64_t T, int64_t max_len) {
  SplitTopkWs w{};
  w.chunk = split_chunk(max_len);
  w.nchunk = (int)((max_len + w.chunk - 1) / w.chunk);
  w.cap = max_len;
  char* p = static_cast<char*>(base);
  // zeroed region first: histogram and counters
  w.hist = reinterpret_cast<uint32_t*>(p);
  w.counter = w.hist + T * kBins;
  p += al((size_t)T * (kBins + 4) * 4);
  w.state = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * 8 * 4);
  w.ndef = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.off = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.eqb = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)T * w.nchunk * 4);
  w.cand = reinterpret_cast<uint32_t*>(p);
  return w;
}

hipError_t launch_topk_split(const TopkArgs& a, const SplitTopkWs& w, bool hist_done, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  dim3 grid(w.nchunk, (unsigned)a.T);
  if (w.chunk == kThreads * 16) {
    if (!hist_done) hipLaunchKernelGGL(split_hist_kernel<16>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL(split_filter_kernel<16>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL(split_compact_kernel<16>, grid, dim3(kThreads), 0, st, a, w);
  } else {
    if (!hist_done) hipLaunchKernelGGL(split_hist_kernel<4>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL(split_filter_kernel<4>, grid, dim3(kThreads), 0, st, a, w);
    hipLaunchKernelGGL(split_compact_kernel<4>, grid, dim3(kThreads), 0, st, a, w);
  }
  return hipGetLastError();
}

}  // namespace misa
