// Per-query top-k of the indexer scores.
//
// MISA pages (MISA abstract; gist.science "Probleemstelling" and "Methodologie:
// MISA"): the indexer keeps the top-k tokens per query, one set shared by all
// heads. Tokens are ordered by (score descending, token index ascending) and the
// first min(k, n) are kept; the set is written in ascending token index, padded
// with -1. Scores compare as reals (-0 == +0).
//
// One workgroup per row: a three-level radix select over an order-preserving
// 32-bit key (12 + 12 + 8 bits, LDS histograms) finds the k-th key u* and how
// many keys equal to u* are kept; then each wave compacts its contiguous
// segment in index order with ballots, so the lowest indices among equal keys
// win and the output comes out sorted. A row of at most kRowCap scores is
// staged once into LDS as keys and every pass runs out of LDS; longer rows are
// re-read from global memory in each pass.
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

__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(TopkArgs a) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t rowk[kRowCap];
  __shared__ uint32_t wsum[kTopkWaves];
  __shared__ uint32_t wgt[kTopkWaves], weq[kTopkWaves];
  __shared__ uint32_t sh_digit, sh_krem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
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

  // ---- radix select of the k-th largest key
  uint32_t prefix = 0, pmask = 0;
  uint32_t krem = (uint32_t)k;
  const int shifts[3] = {20, 8, 0};
  const int nbins[3] = {4096, 4096, 256};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass], nb = nbins[pass];
    for (int i = tid; i < nb; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t e = tid; e < n; e += kTopkThreads) {
      const uint32_t u = key_at(e);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
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
  }
  const uint32_t ustar = prefix;   // the k-th key; krem keys equal to it are kept

  // ---- index-ordered compaction: wave w owns a contiguous segment
  const int64_t seg = ((n + kTopkWaves - 1) / kTopkWaves + 63) / 64 * 64;
  const int64_t s0 = wave * seg, s1 = min(s0 + seg, n);
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

// Register-resident variant for rows of at most kTopkThreads * EPT scores
// (EPT <= 32): every key stays in the registers of its lane for the whole
// select, wave w owning the contiguous run [64 * EPT * w, 64 * EPT * (w + 1))
// with lane l holding elements 64 * j + l of it.
// The radix levels run on v = key - min(key) over the row's nbits-bit range,
// 12 bits per level from the top of that range: scores concentrated in a few
// octaves then spread over the histogram instead of piling into a handful of
// exponent bins (which serializes the LDS atomics and leaves large threshold
// bins), and the select usually ends after one or two levels.
template <int EPT, bool GATHER>
__global__ __launch_bounds__(kTopkThreads) void topk_row_reg_kernel(TopkArgs a) {
  constexpr bool kPrefetchIds = GATHER && EPT <= 16;   // token ids held beside the keys
  __shared__ RadixScratch rs;
  __shared__ uint32_t wmin[kSelWaves], wmax[kSelWaves];
  __shared__ uint32_t wgt[kSelWaves], weq[kSelWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
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

  // ---- every request at once: the keys and (gather rows) their token ids
  const int64_t base = (int64_t)wave * 64 * EPT + lane;
  auto in_row = [&](int j) { return base + 64 * j < n; };
  uint32_t u[EPT];
  int32_t ids[kPrefetchIds ? EPT : 1];
  {
    float v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int64_t e = base + 64 * j;
      v[j] = row[e < n ? e : 0];
      if constexpr (kPrefetchIds) ids[j] = imap[e < n ? e : 0];
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) u[j] = score_key(v[j]);
  }
  radix_clear(rs);
  // ---- key range of the row (element 0 exists, so it stands in for the tail)
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const uint32_t x = in_row(j) ? u[j] : u[0];
    lo = min(lo, x);
    hi = max(hi, x);
  }
  block_minmax(lo, hi, wmin, wmax);
  const int nbits = hi == lo ? 0 : 32 - __clz(hi - lo);
#pragma unroll
  for (int j = 0; j < EPT; ++j) u[j] -= lo;   // v = key - min; slots past the row are never visited

  uint32_t prefix, pmask, krem = (uint32_t)k;
  bool full;
  radix_select(
      [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < EPT; ++j)
          if (in_row(j)) f(u[j]);
      },
      nbits, prefix, pmask, krem, full, rs);

  // ---- index-ordered compaction: values above the prefix, then the first krem equal to it
  auto is_gt = [&](int j) { return in_row(j) && (u[j] & pmask) > prefix; };
  auto is_eq = [&](int j) { return in_row(j) && (u[j] & pmask) == prefix; };
  uint32_t cgt = 0, ceq = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    cgt += (uint32_t)__popcll(__ballot(is_gt(j)));
    ceq += (uint32_t)__popcll(__ballot(is_eq(j)));
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
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const bool gt = is_gt(j);
    const bool eq = is_eq(j);
    const uint64_t meq = __ballot(eq);
    const uint32_t eq_rank = eq_run + (uint32_t)__popcll(meq & lt);
    const bool sel = gt || (eq && eq_rank < krem);
    const uint64_t msel = __ballot(sel);
    const uint32_t pos = sel_run + (uint32_t)__popcll(msel & lt);
    if (sel && pos < (uint32_t)k) {
      int32_t id = (int32_t)(base + 64 * j);
      float sc = key_score(u[j] + lo);
      if constexpr (GATHER) {
        int32_t v;
        if constexpr (kPrefetchIds) v = ids[j];
        else v = imap[base + 64 * j];
        const bool ok = v >= 0 && v < p;
        id = ok ? v : -1;
        sc = ok ? sc : 0.f;
      }
      oi[pos] = id;
      if (os) os[pos] = sc;
    }
    eq_run += (uint32_t)__popcll(meq);
    sel_run += (uint32_t)__popcll(msel);
  }
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
#define MISA_TOPK_REG(EPT_)                                                     \
  if (max_len <= (EPT_) * kTopkThreads) {                                       \
    if (a.imap)                                                                 \
      hipLaunchKernelGGL((topk_row_reg_kernel<EPT_, true>), grid, block, 0, st, a);  \
    else                                                                        \
      hipLaunchKernelGGL((topk_row_reg_kernel<EPT_, false>), grid, block, 0, st, a); \
    return hipGetLastError();                                                   \
  }
  MISA_TOPK_REG(4)
  MISA_TOPK_REG(8)
  MISA_TOPK_REG(16)
  MISA_TOPK_REG(32)
#undef MISA_TOPK_REG
  hipLaunchKernelGGL(topk_row_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

int64_t topk_row_reg_max() { return 32 * kTopkThreads; }

}  // namespace misa
