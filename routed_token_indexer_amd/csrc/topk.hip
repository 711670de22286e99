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
// win and the output comes out sorted.
#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ int64_t row_length(const TopkArgs& a, int64_t t) {
  if (a.row_len) return a.row_len[t];
  const int seq = a.q_seq[t];
  if (seq < 0 || seq >= a.nseq) return 0;
  const int p = a.q_len[t];
  return p < 0 ? 0 : (p > a.Lmax ? a.Lmax : p);
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
  __shared__ uint32_t wsum[kTopkWaves];
  __shared__ uint32_t wgt[kTopkWaves], weq[kTopkWaves];
  __shared__ uint32_t sh_digit, sh_krem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t n = row_length(a, t);
  const int k = a.k;
  const float* row = a.scores + t * a.stride;
  int32_t* oi = a.idx + t * (int64_t)k;
  float* os = a.score ? a.score + t * (int64_t)k : nullptr;
  const int32_t* imap = a.imap ? a.imap + t * (int64_t)a.kc : nullptr;

  if (n <= k) {
    for (int j = tid; j < k; j += kTopkThreads) {
      if (j < n) {
        oi[j] = imap ? imap[j] : j;
        if (os) os[j] = key_score(score_key(row[j]));
      } else {
        oi[j] = -1;
        if (os) os[j] = 0.f;
      }
    }
    return;
  }

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
      const uint32_t u = score_key(row[e]);
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
    const uint32_t u = score_key(row[e]);
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
    const float sv = in ? row[e] : 0.f;
    const uint32_t u = score_key(sv);
    const bool gt = in && u > ustar;
    const bool eq = in && u == ustar;
    const uint64_t meq = __ballot(eq);
    const uint32_t eq_rank = eq_run + (uint32_t)__popcll(meq & lt);
    const bool sel = gt || (eq && eq_rank < krem);
    const uint64_t msel = __ballot(sel);
    const uint32_t pos = sel_run + (uint32_t)__popcll(msel & lt);
    if (sel && pos < (uint32_t)k) {
      oi[pos] = imap ? imap[e] : (int32_t)e;
      if (os) os[pos] = key_score(u);
    }
    eq_run += (uint32_t)__popcll(meq);
    sel_run += (uint32_t)__popcll(msel);
  }
}

__global__ __launch_bounds__(64) void cand_count_kernel(const int32_t* __restrict__ cand, int kc,
                                                        const int32_t* __restrict__ q_seq,
                                                        const int32_t* __restrict__ q_len, int64_t T,
                                                        int64_t nseq, int64_t Lmax, int32_t* __restrict__ row_len) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  const int seq = q_seq[t];
  int p = q_len[t];
  if (seq < 0 || seq >= nseq) p = 0;
  p = p < 0 ? 0 : (p > Lmax ? (int)Lmax : p);
  const int32_t* c = cand + t * (int64_t)kc;
  int n = kc;
  for (int j0 = 0; j0 < kc; j0 += 64) {
    const int j = j0 + lane;
    bool ok = true;
    if (j < kc) {
      const int v = c[j];
      const int prev = j > 0 ? c[j - 1] : -1;
      ok = v >= 0 && v < p && v > prev;
    }
    const uint64_t bad = __ballot(!ok);
    if (bad) {
      n = j0 + __ffsll((unsigned long long)bad) - 1;
      break;
    }
  }
  if (lane == 0) row_len[t] = n;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)a.T), dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_cand_count(const int32_t* cand, int kc, const int32_t* q_seq, const int32_t* q_len,
                             int64_t T, int64_t nseq, int64_t Lmax, int32_t* row_len, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(cand_count_kernel, dim3((unsigned)T), dim3(64), 0, st, cand, kc, q_seq, q_len, T, nseq,
                     Lmax, row_len);
  return hipGetLastError();
}

}  // namespace misa
