// Per-query top-k of the indexer scores.
//
// MISA pages (MISA abstract; gist.science "Probleemstelling" and "Methodologie:
// MISA"): the indexer keeps the top-k tokens per query, one set shared by all
// heads. Tokens are ordered by (score descending, token index ascending) and the
// first min(k, n) are kept; the set is written in ascending token index, padded
// with -1. Scores compare as reals (-0 == +0).
//
// One workgroup per row. Rows of up to 32K scores keep their keys (an
// order-preserving 32-bit map of the scores) in registers: one LDS histogram
// finds the bin of the k-th key, the few keys of that bin are ranked exactly,
// and one ballot pass writes the kept set in index order (topk_row_reg_kernel).
// Rows of heavy ties, and longer rows, take an exact three-level radix select
// (12 + 12 + 8 bits) whose index-ordered compaction lets the lowest indices win
// among equal keys (topk_row_kernel; a row of at most kRowCap scores is staged
// once into LDS, longer rows are re-read in each pass).
#include "misa_common.hpp"
#include "misa_internal.hpp"
#include "misa_select.hpp"

namespace misa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kRowCap = 12288;   // scores staged in LDS (48 KiB)

// Row geometry: n scores (the visible prefix, or kc candidate slots), and the
// visible prefix p used to map candidate slots back to token ids.
__device__ __forceinline__ void row_geometry(const TopkArgs& a, int64_t t, int64_t& n, int& p) {
  p = query_prefix_len(a.q_seq, a.q_len, a.nseq, a.Lmax, t);
  if (p < 0) {
    p = 0;
    n = 0;
    return;
  }
  n = a.imap ? a.kc : p;
}

// Output token id of score slot e (-1 for a skipped candidate) and its score.
__device__ __forceinline__ void out_entry(const TopkArgs& a, const int32_t* imap, int p, int64_t e, uint32_t u,
                                          int32_t& id, float& sc) {
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

// Exclusive prefix sum over the workgroup's threads (ascending thread id).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum) {
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
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  __syncthreads();
  return pre + inc - v;
}

// Exact top-k of row t by one 1024-thread workgroup, rows of any length.
__device__ __forceinline__ void topk_row_general(const TopkArgs& a, int64_t t) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t rowk[kRowCap];
  __shared__ uint32_t wsum[kTopkWaves];
  __shared__ uint32_t wgt[kTopkWaves], weq[kTopkWaves];
  __shared__ uint32_t sh_digit, sh_krem, s_m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t n;
  int p;
  row_geometry(a, t, n, p);
  const int k = a.k;
  const float* row = a.scores + t * a.stride;
  int32_t* oi = a.idx + t * (int64_t)k;
  float* os = a.score ? a.score + t * (int64_t)k : nullptr;
  const int32_t* imap = a.imap ? a.imap + t * (int64_t)a.kc : nullptr;

  if (n <= k) {
    for (int j = tid; j < k; j += kTopkThreads) {
      if (j < n) {
        int32_t id;
        float sc;
        out_entry(a, imap, p, j, score_key(row[j]), id, sc);
        oi[j] = id;
        if (os) os[j] = sc;
      } else {
        oi[j] = -1;
        if (os) os[j] = 0.f;
      }
    }
    return;
  }

  const bool inlds = n <= kRowCap;
  if (inlds) {
    for (int64_t e0 = 0; e0 < n; e0 += 4 * kTopkThreads) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t e = e0 + q * kTopkThreads + tid;
        v[q] = e < n ? row[e] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t e = e0 + q * kTopkThreads + tid;
        if (e < n) rowk[e] = score_key(v[q]);
      }
    }
    __syncthreads();
  }
  auto key_at = [&](int64_t e) -> uint32_t { return inlds ? rowk[e] : score_key(row[e]); };

  // ---- radix select of the k-th largest key: levels of 12, 12 and 8 key bits,
  // each a histogram of the keys that match the digits found so far
  uint32_t prefix = 0, pmask = 0;
  uint32_t krem = (uint32_t)k;
  const int shifts[3] = {20, 8, 0};
  const int nbins[3] = {4096, 4096, 256};
  auto level = [&](int pass, auto&& feed) {   // feed(add) calls add(key) for every key counted
    const int shift = shifts[pass], nb = nbins[pass];
    for (int i = tid; i < nb; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    feed([&](uint32_t u) {
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    });
    __syncthreads();
    // thread i owns bins [nb - 4(i+1), nb - 4i), scanned from the top
    const int ngrp = nb / 4;
    uint32_t c[4] = {0, 0, 0, 0};
    if (tid < ngrp) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[nb - 1 - (4 * tid + j)];
    }
    const uint32_t mine = c[0] + c[1] + c[2] + c[3];
    uint32_t above = block_excl_scan(mine, wsum);
    if (tid < ngrp) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < krem && above + c[j] >= krem) {
          sh_digit = (uint32_t)(nb - 1 - (4 * tid + j));
          sh_krem = krem - above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem = sh_krem;
    __syncthreads();
  };
  auto row_keys = [&](auto&& add) {
    for (int64_t e = tid; e < n; e += kTopkThreads) add(key_at(e));
  };
  // index-ordered output: wave w owns a contiguous segment and needs the counts of
  // keys above the k-th key (wgt) and equal to it (weq) in every segment
  const int64_t seg = ((n + kTopkWaves - 1) / kTopkWaves + 63) / 64 * 64;
  const int64_t s0 = wave * seg, s1 = min(s0 + seg, n);
  bool counted = false;
  level(0, row_keys);
  if (!inlds) {
    // A row in memory: a second pass (in the same strided order as the first)
    // lists the keys of the threshold bin with their indices in LDS, each wave
    // in a region of its own (no atomics), and counts every segment's keys in
    // higher bins; the last two levels then run over the lists, and the
    // segments' counts come from them: the row is read three times instead of
    // five. A wave with more keys in the bin than its region holds sends the row
    // through the levels over the row.
    constexpr int kPerWave = kRowCap / 2 / kTopkWaves;
    uint32_t* const lkey = rowk + wave * 2 * kPerWave;
    uint32_t* const lidx = lkey + kPerWave;
    const uint32_t b1 = prefix >> 20;
    if (tid < kTopkWaves) {
      wgt[tid] = 0u;
      weq[tid] = 0u;
    }
    if (tid == 0) s_m = 0u;
    __syncthreads();
    uint32_t nl = 0;   // keys this wave has listed so far (lane 0's copy is the wave's)
    // the segment of element e, followed along the stride (no division per element)
    int sg = 0;
    int64_t sg_end = seg;
    for (int64_t e = tid; e < n; e += kTopkThreads) {
      while (e >= sg_end) {
        ++sg;
        sg_end += seg;
      }
      const uint32_t u = key_at(e);
      if ((u >> 20) > b1) atomicAdd(&wgt[sg], 1u);
      const bool inb = (u >> 20) == b1;
      const uint64_t mb = __ballot(inb);
      const uint32_t pos = nl + lanes_below(mb);
      if (inb && pos < (uint32_t)kPerWave) {
        lkey[pos] = u;
        lidx[pos] = (uint32_t)e;
      }
      nl += (uint32_t)__popcll(mb);
    }
    nl = (uint32_t)__builtin_amdgcn_readfirstlane((int)nl);
    __shared__ uint32_t s_nl[kTopkWaves];
    if (lane == 0) {
      s_nl[wave] = nl;
      if (nl > (uint32_t)kPerWave) s_m = 1u;
    }
    __syncthreads();
    if (s_m == 0u) {
      // entry j of wave w's list: key at rowk[2 w kPerWave + j], index kPerWave further
      auto list_keys = [&](auto&& add) {
        for (int i = tid; i < kTopkWaves * kPerWave; i += kTopkThreads) {
          const int w = i / kPerWave, j = i % kPerWave;
          if ((uint32_t)j < s_nl[w]) add(rowk[2 * w * kPerWave + j]);
        }
      };
      level(1, list_keys);
      level(2, list_keys);
      const uint32_t us = prefix;
      for (int i = tid; i < kTopkWaves * kPerWave; i += kTopkThreads) {
        const int w = i / kPerWave, j = i % kPerWave;
        if ((uint32_t)j >= s_nl[w]) continue;
        const uint32_t u = rowk[2 * w * kPerWave + j];
        const int ls = (int)(rowk[2 * w * kPerWave + kPerWave + j] / (uint32_t)seg);   // the entry's segment
        if (u > us) atomicAdd(&wgt[ls], 1u);
        else if (u == us) atomicAdd(&weq[ls], 1u);
      }
      __syncthreads();
      counted = true;
    }
  }
  if (!counted) {
    level(1, row_keys);
    level(2, row_keys);
  }
  const uint32_t ustar = prefix;   // the k-th key; krem keys equal to it are kept

  if (!counted) {
    uint32_t cgt = 0, ceq = 0;
    for (int64_t e = s0 + lane; e < s1; e += 64) {
      const uint32_t u = key_at(e);
      cgt += u > ustar ? 1u : 0u;
      ceq += u == ustar ? 1u : 0u;
    }
    cgt = wave_sum(cgt);
    ceq = wave_sum(ceq);
    if (lane == 0) {
      wgt[wave] = cgt;
      weq[wave] = ceq;
    }
    __syncthreads();
  }
  uint32_t eq_run = 0, sel_run = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t take = eq_run >= krem ? 0u : min(weq[w], krem - eq_run);
    sel_run += wgt[w] + take;
    eq_run += weq[w];
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int64_t e0 = s0; e0 < s1; e0 += 64) {
    const int64_t e = e0 + lane;
    const bool in = e < s1;
    const uint32_t u = in ? key_at(e) : 0u;
    const bool gt = in && u > ustar;
    const bool eq = in && u == ustar;
    const uint64_t meq = __ballot(eq);
    const uint32_t eq_rank = eq_run + (uint32_t)__popcll(meq & lt);
    const bool sel = gt || (eq && eq_rank < krem);
    const uint64_t msel = __ballot(sel);
    const uint32_t pos = sel_run + (uint32_t)__popcll(msel & lt);
    if (sel && pos < (uint32_t)k) {
      int32_t id;
      float sc;
      out_entry(a, imap, p, e, u, id, sc);
      oi[pos] = id;
      if (os) os[pos] = sc;
    }
    eq_run += (uint32_t)__popcll(meq);
    sel_run += (uint32_t)__popcll(msel);
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(TopkArgs a) { topk_row_general(a, blockIdx.x); }

// First output of a row that the register-resident kernel left to the general
// select (no valid output is below -1).
constexpr int32_t kFallbackMark = INT32_MIN;
constexpr int kFallbackRows = 64;   // rows checked per workgroup

// Rows marked by the register-resident kernel, redone by the general select:
// each workgroup reads the first output of kFallbackRows rows.
__global__ __launch_bounds__(kTopkThreads) void topk_fallback_kernel(TopkArgs a) {
  __shared__ uint64_t s_mask;
  const int64_t t0 = (int64_t)blockIdx.x * kFallbackRows;
  if (threadIdx.x < 64) {
    const int64_t t = t0 + threadIdx.x;
    const bool marked = t < a.T && a.idx[t * (int64_t)a.k] == kFallbackMark;
    const uint64_t m = __ballot(marked);
    if (threadIdx.x == 0) s_mask = m;
  }
  __syncthreads();
  uint64_t m = s_mask;
  while (m) {
    const int i = __ffsll((unsigned long long)m) - 1;
    m &= m - 1;
    topk_row_general(a, t0 + i);
    __syncthreads();   // LDS of the general select is reused by the next row
  }
}

// Exact select over the whole register-resident row (the fast path's fallback):
// range [lo, hi] of the row's keys, radix levels on v = key - lo from the top of
// that range, then the ascending-slot output of every v above the prefix and the
// first krem equal to it. fresh_nvalid / fresh_nvs give the lane's and the
// wave's count of slots in the row; emit(j, sel, run) writes slot j.
template <int EPT, int NT, int NH, typename FV, typename FS, typename Emit>
__device__ __forceinline__ void general_select(const uint32_t (&u)[EPT], FV fresh_nvalid, FS fresh_nvs, int k,
                                               RadixScratch<NT, NH>& rs, uint32_t* wmin, uint32_t* wmax,
                                               uint32_t* wgt, uint32_t* weq, Emit emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();   // the fast path's list (in the histograms) is no longer read
  radix_clear(rs);
  uint32_t lo = 0xffffffffu, hi = 0u;
  {
    const int nv = fresh_nvalid(), ns = fresh_nvs();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if (j >= ns) continue;
      lo = min(lo, j < nv ? u[j] : 0xffffffffu);
      hi = max(hi, j < nv ? u[j] : 0u);
    }
  }
  block_minmax<NT>(lo, hi, wmin, wmax);   // its barrier also orders the clear
  const int nbits = hi == lo ? 0 : 32 - __clz(hi - lo);

  uint32_t prefix, pmask, krem = (uint32_t)k;
  bool full;
  radix_select(
      [&](auto&& f) {
        const int nv = fresh_nvalid(), ns = fresh_nvs();
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          if (j >= ns) continue;
          if (j < nv) f(u[j] - lo);
        }
      },
      nbits, prefix, pmask, krem, full, rs);

  // ---- ascending-slot output: values above the prefix, then the first krem equal to it
  auto is_gt = [&](int j, int nv) { return j < nv && ((u[j] - lo) & pmask) > prefix; };
  auto is_eq = [&](int j, int nv) { return j < nv && ((u[j] - lo) & pmask) == prefix; };
  uint32_t cgt = 0, ceq = 0;
  int nv = fresh_nvalid(), ns = fresh_nvs();
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if (j >= ns) continue;
    cgt += (uint32_t)__popcll(__ballot(is_gt(j, nv)));
    ceq += (uint32_t)__popcll(__ballot(is_eq(j, nv)));
  }
  if (lane == 0) {
    wgt[wave] = cgt;
    weq[wave] = ceq;
  }
  __syncthreads();
  uint32_t eq_run = 0, sel_run = 0;
  for (int ww = 0; ww < wave; ++ww) {
    const uint32_t take = eq_run >= krem ? 0u : min(weq[ww], krem - eq_run);
    sel_run += wgt[ww] + take;
    eq_run += weq[ww];
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  nv = fresh_nvalid();
  ns = fresh_nvs();
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if (j >= ns) continue;
    const bool gt = is_gt(j, nv);
    const bool eq = is_eq(j, nv);
    const uint64_t meq = __ballot(eq);
    const uint32_t eq_rank = eq_run + (uint32_t)__popcll(meq & lt);
    emit(j, gt || (eq && eq_rank < krem), sel_run);
    eq_run += (uint32_t)__popcll(meq);
  }
}

// Register-resident variant for rows of at most NT * EPT scores: every key
// stays in the registers of its lane for the whole select, wave w owning the
// contiguous run [64 * EPT * w, 64 * EPT * (w + 1)) with lane l holding elements
// 64 * j + l of it. Slots past the row hold key 0 and are skipped wave by wave.
//
// Fast path (a handful of VALU operations per score, the rest is per row):
//  1. one LDS histogram of 4096 bins over the row's key range [lo, hi], or over
//     the 2^kWinBits keys below hi when the range is wider (lower keys fall into
//     bin 0), gives the bin d of the k-th largest key and how many of that bin
//     are still needed (a threshold in a clamped bin 0 takes a second histogram
//     of that bin's keys over their own range);
//  2. keys above bin d are kept (counted per wave with ballots); the keys of bin
//     d, about a handful for real scores, go to an LDS list with their slots;
//  3. each listed key gets its exact rank in (key descending, slot ascending)
//     order; the last kept one gives the threshold key and the slot cutoff among
//     keys equal to it, and the kept ones add to their wave's count;
//  4. one pass writes every key > threshold, or == threshold at a slot <=
//     cutoff, at its ballot position (ascending slot order).
// The select falls back to an exact multi-level radix over the whole row when
// bin d holds more than kCandCap keys (heavy ties, e.g. exactly representable
// grids) or the row holds the padding key itself.
constexpr int kNonTemporal = 2;   // buffer cache policy bit: streaming access
constexpr int kWinBits = 26;     // window of 2^26 key units: 8 octaves of positive floats
constexpr int kBinShift = kWinBits - 12;
constexpr int kCandCap = 512;    // keys of the threshold bin ranked in LDS

// The register-resident select of row t (the body of topk_row_reg_kernel).
template <int EPT, bool GATHER, int NT, bool MANY>
__device__ __attribute__((always_inline)) void topk_row_reg_row(const TopkArgs& a, int64_t t) {
  constexpr int NW = NT / 64;
  // the few-rows variants run the fallback in place; the many-rows (MANY) variants
  // mark the row for topk_fallback_kernel and keep their registers for the fast
  // path: at most 64 per lane, so that eight waves per SIMD are resident
  constexpr bool kInlineFallback = !MANY;
  constexpr bool kPrefetchIds = GATHER && EPT <= 16;   // token ids held beside the keys
  __shared__ __attribute__((aligned(16))) RadixScratch<NT, (NT == 1024 && !MANY) ? 3 : 1> rs;
  __shared__ uint32_t wmin[NW], wmax[NW];
  __shared__ uint32_t wgt[NW], weq[NW];
  __shared__ uint32_t s_m, s_thr, s_cut;
  static_assert(2 * kCandCap <= kSelBins, "candidate list lives in the first histogram");
  uint32_t* const c_key = &rs.hist[0][0];          // after the level-1 scan
  uint32_t* const c_slot = &rs.hist[0][kCandCap];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t n;
  int p;
  row_geometry(a, t, n, p);
  if (n <= a.len_lo || n > a.len_hi) return;   // the other launch's row
  const int k = a.k;
  const float* row = a.scores + t * a.stride;
  int32_t* oi = a.idx + t * (int64_t)k;
  float* os = a.score ? a.score + t * (int64_t)k : nullptr;
  const int32_t* imap = a.imap ? a.imap + t * (int64_t)a.kc : nullptr;

  if (n <= k) {
    // the whole row, then -1 padding: four slots per thread requested at once
    // (clamped reads), so that the copy takes one memory round trip per 4 * NT
    // slots instead of one per slot
    constexpr int U = 4;
    const int nl = (int)n;
    for (int j0 = 0; j0 < k; j0 += U * NT) {
      float v[U];
      int32_t m[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * NT + tid;
        const int jc = j < nl ? j : 0;
        v[u] = nl > 0 ? row[jc] : 0.f;
        m[u] = (imap && nl > 0) ? imap[jc] : 0;
      }
      // all of them consumed from here on (an s_waitcnt the compiler sees: it
      // would otherwise also wait for the stores below before each use)
      __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * NT + tid;
        if (j >= k) continue;
        int32_t id = -1;
        float sc = 0.f;
        if (j < nl) {
          sc = key_score(score_key(v[u]));
          id = j;
          if (imap) {
            const bool ok = m[u] >= 0 && m[u] < p;
            id = ok ? m[u] : -1;
            sc = ok ? sc : 0.f;
          }
        }
        oi[j] = id;
        if (os) os[j] = sc;
      }
    }
    return;
  }

  // ---- every request at once: the keys and (gather rows) their token ids
  const int base = wave * 64 * EPT + lane;   // slot of element j: base + 64 * j (n < 2^31)
  // elements j < nvalid of this lane lie in the row (one count instead of an index per element)
  const int nvalid = n > base ? (int)min((int64_t)EPT, (n - base + 63) / 64) : 0;
  // lane 0 has the most; slots j >= nvs are empty in the whole wave and skipped by a scalar branch
  const int nvs = __builtin_amdgcn_readfirstlane(nvalid);
  // each pass takes fresh copies of nvalid / nvs that the compiler cannot see through,
  // so it recomputes the slot masks (one compare each) instead of keeping up to 64 of
  // them live in scalar registers across the whole kernel
  auto fresh_nvalid = [&]() {
    int x = nvalid;
    asm volatile("" : "+v"(x));
    return x;
  };
  auto fresh_nvs = [&]() {
    int x = nvs;
    asm volatile("" : "+s"(x));
    return x;
  };
  // loads through range-checked views of the row: one 32-bit lane offset and a
  // uniform per-element offset instead of a 64-bit address per element
  uint32_t u[EPT];
  int32_t ids[kPrefetchIds ? EPT : 1];
  const auto rview = buffer_view(row, (uint32_t)(n * 4));
  const auto iview = buffer_view(imap, GATHER ? (uint32_t)(n * 4) : 0u);
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if (j >= nvs) continue;
    // raw bits (keys in place below); non-temporal: every score is read once
    u[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rview, (int)((uint32_t)base * 4u), (int)(256u * j),
                                                          kNonTemporal);
    if constexpr (kPrefetchIds) ids[j] = (int32_t)buffer_load_u32(iview, (uint32_t)base * 4u, 256u * j);
  }
  if (tid == 0) s_m = 0u;
  radix_clear(rs);
  uint32_t lo = 0xffffffffu, hi = 0u;
  {
    const int nv = fresh_nvalid(), ns = fresh_nvs();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if (j >= ns) continue;
      const bool in = j < nv;
      u[j] = in ? score_key(__uint_as_float(u[j])) : 0u;
      hi = max(hi, u[j]);
      lo = min(lo, in ? u[j] : 0xffffffffu);
    }
  }
  // every load has been consumed: say so to the compiler's wait tracking (an
  // s_waitcnt it sees), which otherwise cannot match the skipped slots of the passes
  // below to those of the loads and waits for all memory operations, the earlier
  // output stores included, before each slot of the output loop
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  block_minmax<NT>(lo, hi, wmin, wmax);   // its barrier also orders the histogram clear

  // ---- 1. level-1 histogram of the keys <= wtop: over the range [lo, wtop] when
  // it spans at most kWinBits bits (bins of 2^shift keys from lo), else over the
  // window of 2^kWinBits keys below wtop with every lower key in bin 0. Padding
  // slots (key 0, the (-n) mod 64 slots after the row's last element) land in
  // bin 0 and are taken out of it again. A threshold in a clamped bin 0 gives a
  // second histogram over that bin's keys (wtop = its top), now unclamped.
  constexpr uint32_t kWin = (1u << kWinBits) - 1u;
  auto adaptive_shift = [](uint32_t range) { return max(0, (range == 0u ? 0 : 32 - __clz(range)) - 12); };
  uint32_t wtop = hi;
  bool clamped = hi - lo > kWin;
  uint32_t wbase = clamped ? hi - kWin : lo;
  int shift = clamped ? kBinShift : adaptive_shift(hi - lo);
  if (tid == 0) atomicSub(&rs.hist[0][0], (uint32_t)(-n & 63));
  {
    const int ns = fresh_nvs();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if (j >= ns) continue;
      const uint32_t d = __builtin_elementwise_sub_sat(u[j], wbase) >> shift;
      atomicAdd(&rs.hist[0][d], 1u);
    }
  }
  __syncthreads();
  find_threshold<NT>(rs.hist[0], kSelBins, (uint32_t)k, rs.wsum[0], rs.out[0]);
  uint32_t d1 = rs.out[0][0], krem1 = rs.out[0][1];
  if (d1 == 0u && clamped) {
    wtop = wbase + ((1u << shift) - 1u);   // <= hi: bin 0 holds keys below it
    clamped = false;
    wbase = lo;
    shift = adaptive_shift(wtop - lo);
    for (int i = tid; i < kSelBins; i += NT) rs.hist[0][i] = 0u;   // find_threshold has read them
    __syncthreads();
    if (tid == 0) atomicSub(&rs.hist[0][0], (uint32_t)(-n & 63));
    const int ns = fresh_nvs();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if (j >= ns) continue;
      if (u[j] <= wtop) atomicAdd(&rs.hist[0][__builtin_elementwise_sub_sat(u[j], wbase) >> shift], 1u);
    }
    __syncthreads();
    find_threshold<NT>(rs.hist[0], kSelBins, krem1, rs.wsum[1], rs.out[1]);
    d1 = rs.out[1][0];
    krem1 = rs.out[1][1];
  }

  // ---- output of slot j where sel holds: ascending slot order from pos
  auto emit = [&](int j, bool sel, uint32_t& run) {
    const uint64_t msel = __ballot(sel);
    const uint32_t pos =
        run + __builtin_amdgcn_mbcnt_hi((uint32_t)(msel >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msel, 0u));
    if (sel && pos < (uint32_t)k) {
      int32_t id = base + 64 * j;
      float sc = key_score(u[j]);
      if constexpr (GATHER) {
        int32_t v;
        if constexpr (kPrefetchIds) v = ids[j];
        else v = (int32_t)buffer_load_u32(iview, (uint32_t)base * 4u, 256u * j);
        const bool ok = v >= 0 && v < p;
        id = ok ? v : -1;
        sc = ok ? sc : 0.f;
      }
      oi[pos] = id;
      if (os) os[pos] = sc;
    }
    run += (uint32_t)__popcll(msel);
  };

  // bin 0 is exact unless it holds clamped keys; a row key equal to the padding
  // key 0 (float bits 0xffffffff) leaves it to the general select too
  if (d1 != 0u || (!clamped && lo != 0u)) {
    // ---- 2. keys above bin d are kept; keys of bin d are listed
    const uint32_t klo = wbase + (d1 << shift);
    const uint32_t span = (1u << shift) - 1u;
    const uint32_t khi = wtop - klo < span ? wtop : klo + span;   // no wrap past 2^32 - 1
    uint32_t cgt = 0;
    {
      const int ns = fresh_nvs();
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        if (j >= ns) continue;
        cgt += (uint32_t)__popcll(__ballot(u[j] > khi));
        const bool c = u[j] - klo <= khi - klo;   // klo <= key <= khi; padding (key 0) is below klo > 0
        const uint64_t mc = __ballot(c);
        if (mc) {
          uint32_t off = 0;
          if (lane == 0) off = atomicAdd(&s_m, (uint32_t)__popcll(mc));
          off = (uint32_t)__shfl(off, 0, kWave) +
                __builtin_amdgcn_mbcnt_hi((uint32_t)(mc >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mc, 0u));
          if (c && off < (uint32_t)kCandCap) {
            c_key[off] = u[j];
            c_slot[off] = (uint32_t)(base + 64 * j);
          }
        }
      }
    }
    if (lane == 0) {
      wgt[wave] = cgt;
      weq[wave] = 0u;
    }
    __syncthreads();
    const uint32_t m = s_m;
    if (m <= (uint32_t)kCandCap) {
      // ---- 3. exact rank of each listed key; the krem1 first are kept. A few
      // keys: a thread per key walks the list; more: a wave per key, its lanes
      // comparing 64 others at a time
      auto keep = [&](uint32_t r, uint32_t ki, uint32_t si) {
        if (r < krem1) atomicAdd(&weq[si / (64u * EPT)], 1u);
        if (r == krem1 - 1u) {
          s_thr = ki;
          s_cut = si;
        }
      };
      if (m <= 32u) {
        if ((uint32_t)tid < m) {
          const uint32_t ki = c_key[tid], si = c_slot[tid];
          uint32_t r = 0;
          if constexpr (!MANY) {
            // the list read 4 slots at a time (16-byte broadcast reads; slots
            // past m are in the list's storage and masked); the many-row
            // variants lack the registers to hold these loads in flight
#pragma unroll
            for (int g = 0; g < 8; ++g) {
              const u32x4 kk = *reinterpret_cast<const u32x4*>(c_key + 4 * g);
              const u32x4 ss = *reinterpret_cast<const u32x4*>(c_slot + 4 * g);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                r += ((uint32_t)(4 * g + e) < m && (kk[e] > ki || (kk[e] == ki && ss[e] < si))) ? 1u : 0u;
            }
          } else {
            for (uint32_t q = 0; q < m; ++q)
              r += (c_key[q] > ki || (c_key[q] == ki && c_slot[q] < si)) ? 1u : 0u;
          }
          keep(r, ki, si);
        }
      } else {
        for (uint32_t i = wave; i < m; i += NW) {
          const uint32_t ki = c_key[i], si = c_slot[i];
          uint32_t r = 0;
          for (uint32_t q0 = 0; q0 < m; q0 += 64) {
            const uint32_t q = q0 + lane;
            bool before = false;
            if (q < m) before = c_key[q] > ki || (c_key[q] == ki && c_slot[q] < si);
            r += (uint32_t)__popcll(__ballot(before));
          }
          if (lane == 0) keep(r, ki, si);
        }
      }
      __syncthreads();
      const uint32_t thr = s_thr;
      const int cut = (int)s_cut - base;   // kept keys equal to thr: 64 * j <= cut
      uint32_t run = 0;
      for (int ww = 0; ww < wave; ++ww) run += wgt[ww] + weq[ww];
      // ---- 4. ascending-slot output
      const int ns = fresh_nvs();
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        if (j >= ns) continue;
        emit(j, (u[j] > thr) | ((u[j] == thr) & (64 * j <= cut)), run);
      }
      return;
    }
  }
  if constexpr (kInlineFallback)
    general_select<EPT, NT>(u, fresh_nvalid, fresh_nvs, k, rs, wmin, wmax, wgt, weq, emit);
  else if (tid == 0)
    oi[0] = kFallbackMark;
}

template <int EPT, bool GATHER, int NT, bool MANY>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(MANY ? 8 : NT / 256))) void topk_row_reg_kernel(
    TopkArgs a) {
  // causal batches: longest rows first, unless the launch takes only the shorter
  // rows (then the rows it leaves alone, the longer ones, come last and fill the tail)
  topk_row_reg_row<EPT, GATHER, NT, MANY>(a, a.len_hi != INT64_MAX ? (int64_t)blockIdx.x
                                                                        : (int64_t)a.T - 1 - blockIdx.x);
}

}  // namespace

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t st) {
  if (words <= 0) return hipSuccess;
  const int64_t g = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)g), dim3(256), 0, st, p, words);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int64_t max_len = a.imap ? a.kc : a.Lmax;
  const dim3 grid((unsigned)a.T), block(kTopkThreads);
  // many rows (prefill): 256- and 512-thread workgroups (one histogram), so that
  // several rows per CU are in flight; few rows: 1024 threads for the shortest
  // latency per row
#define MISA_TOPK_REG(EPT_, NT_)                                                          \
  if (max_len <= (EPT_) * (NT_)) {                                                        \
    if (a.imap)                                                                           \
      hipLaunchKernelGGL((topk_row_reg_kernel<EPT_, true, NT_, false>), grid, dim3(NT_), 0, st, a);  \
    else                                                                                  \
      hipLaunchKernelGGL((topk_row_reg_kernel<EPT_, false, NT_, false>), grid, dim3(NT_), 0, st, a); \
    return hipGetLastError();                                                             \
  }
  if (a.T >= 256) {
    // rows the register-resident kernel leaves to the general select are marked
    // and redone by topk_fallback_kernel (usually none: a launch that only reads)
    bool done = false;
#define MISA_TOPK_MANY(EPT_, NT_)                                                        \
    if (!done && max_len <= (EPT_) * (NT_)) {                                            \
      if (a.imap)                                                                        \
        hipLaunchKernelGGL((topk_row_reg_kernel<EPT_, true, NT_, true>), grid, dim3(NT_), 0, st, a);  \
      else                                                                               \
        hipLaunchKernelGGL((topk_row_reg_kernel<EPT_, false, NT_, true>), grid, dim3(NT_), 0, st, a); \
      done = true;                                                                       \
    }
    MISA_TOPK_MANY(16, 256)
    MISA_TOPK_MANY(32, 256)
    if (!done && max_len <= 32 * 512) {
      // rows of up to 8192 scores on 256-thread workgroups (eight per CU), longer
      // ones on 512-thread workgroups (four per CU): two launches over the batch,
      // each leaving the other's rows alone. A causal batch has rows of every
      // length, and its shorter half then runs twice as many rows per CU
      TopkArgs s = a, l = a;
      s.len_hi = 32 * 256;
      l.len_lo = 32 * 256;
      if (a.imap) {
        hipLaunchKernelGGL((topk_row_reg_kernel<32, true, 256, true>), grid, dim3(256), 0, st, s);
        hipLaunchKernelGGL((topk_row_reg_kernel<32, true, 512, true>), grid, dim3(512), 0, st, l);
      } else {
        hipLaunchKernelGGL((topk_row_reg_kernel<32, false, 256, true>), grid, dim3(256), 0, st, s);
        hipLaunchKernelGGL((topk_row_reg_kernel<32, false, 512, true>), grid, dim3(512), 0, st, l);
      }
      done = true;
    }
#undef MISA_TOPK_MANY
    if (done) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(topk_fallback_kernel, dim3((unsigned)((a.T + kFallbackRows - 1) / kFallbackRows)),
                         block, 0, st, a);
      return hipGetLastError();
    }
  }
  MISA_TOPK_REG(4, 1024)
  MISA_TOPK_REG(8, 1024)
  MISA_TOPK_REG(16, 1024)
  MISA_TOPK_REG(32, 1024)
#undef MISA_TOPK_REG
  hipLaunchKernelGGL(topk_row_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

int64_t topk_row_reg_max() { return 32 * kTopkThreads; }

}  // namespace misa
