// Selection building blocks of the top-k kernels: workgroups of NT threads
// (1024 by default), order-preserving 32-bit keys (score_key), radix levels over
// LDS histograms.
//
// The selection rule (MISA pages: the indexer keeps the top-k tokens of each
// query, ordered by score descending and token index ascending) is resolved as
// a key threshold: every key above it is kept, and of the keys equal to it the
// krem with the lowest indices.
#pragma once

#include "misa_common.hpp"

namespace misa {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 4096;   // bins of one radix level (12 bits)

// Inclusive prefix sum over the 64 lanes of a wave: row shifts by 1, 2, 4, 8
// inside each 16-lane row, then lane 15 of rows 0 / 2 into rows 1 / 3 and lane
// 31 into rows 2 and 3 (DPP; an out-of-row source reads the 0 given as `old`).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return (uint32_t)x;
}

// Exclusive prefix sum over the workgroup in thread order, and the total.
// One barrier; wsum[NT / 64] must not be reused before every thread has
// passed the next barrier.
template <int NT = kSelThreads>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w4 = 0; w4 < NW; w4 += 4) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(wsum + w4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pre += (w4 + i) < wave ? x[i] : 0u;
      tot += x[i];
    }
  }
  total = tot;
  return pre + inc - v;
}

// Two exclusive prefix sums at once (one barrier): returns a's and sets b's.
// wsum2 holds 2 * kSelWaves words (1024-thread workgroups).
__device__ __forceinline__ uint32_t block_excl_scan2(uint32_t a, uint32_t b, uint32_t* wsum2, uint32_t& b_excl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) {
    wsum2[wave] = ia;
    wsum2[kSelWaves + wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
#pragma unroll
  for (int w4 = 0; w4 < kSelWaves; w4 += 4) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(wsum2 + w4);
    const u32x4 y = *reinterpret_cast<const u32x4*>(wsum2 + kSelWaves + w4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa += (w4 + i) < wave ? x[i] : 0u;
      pb += (w4 + i) < wave ? y[i] : 0u;
    }
  }
  b_excl = pb + ib - b;
  return pa + ia - a;
}

// Threshold bin of a histogram of nb <= kSelBins bins scanned from the top: the
// bin d with count(bins > d) < krem <= count(bins >= d). Writes out[0] = d,
// out[1] = krem - count(bins > d) and out[2] = 1 if bin d is kept whole (its
// count equals out[1]). Requires count(all bins) >= krem >= 1. Two barriers;
// the caller reads out[] after the second.
template <int NT = kSelThreads>
__device__ __forceinline__ void find_threshold(const uint32_t* hist, int nb, uint32_t krem, uint32_t* wsum,
                                               uint32_t* out) {
  constexpr int PMAX = kSelBins / NT;   // bins per thread at most
  const int tid = threadIdx.x;
  const int per = nb > NT ? nb / NT : 1;
  uint32_t c[PMAX], mine = 0;
#pragma unroll
  for (int jj = 0; jj < PMAX; ++jj) {
    const int b = per * tid + jj;
    c[jj] = (jj < per && b < nb) ? hist[nb - 1 - b] : 0u;
    mine += c[jj];
  }
  uint32_t tot;
  uint32_t above = block_excl_scan<NT>(mine, wsum, tot);
#pragma unroll
  for (int jj = 0; jj < PMAX; ++jj) {
    if (above < krem && above + c[jj] >= krem) {
      out[0] = (uint32_t)(nb - 1 - (per * tid + jj));
      out[1] = krem - above;
      out[2] = (krem - above == c[jj]) ? 1u : 0u;
    }
    above += c[jj];
  }
  __syncthreads();
}

// find_threshold by the calling wave alone, for nb <= 256 bins (four per
// lane; no barrier inside: the caller puts one before out[] is read).
__device__ __forceinline__ void find_threshold_wave(const uint32_t* hist, int nb, uint32_t krem, uint32_t* out) {
  constexpr int PER = 4;
  const int lane = threadIdx.x & 63;
  uint32_t c[PER], mine = 0;
#pragma unroll
  for (int jj = 0; jj < PER; ++jj) {
    const int b = PER * lane + jj;
    c[jj] = b < nb ? hist[nb - 1 - b] : 0u;
    mine += c[jj];
  }
  uint32_t above = wave_incl_scan(mine) - mine;
#pragma unroll
  for (int jj = 0; jj < PER; ++jj) {
    if (above < krem && above + c[jj] >= krem) {
      out[0] = (uint32_t)(nb - 1 - (PER * lane + jj));
      out[1] = krem - above;
      out[2] = (krem - above == c[jj]) ? 1u : 0u;
    }
    above += c[jj];
  }
}

// Scratch of radix_select for NT threads: NH histograms (one per level, or a
// single one cleared between levels), a scan and a result slot per level.
template <int NT = kSelThreads, int NH = 3>
struct RadixScratch {
  uint32_t hist[NH][kSelBins];
  uint32_t wsum[3][NT / 64];
  uint32_t out[3][4];
};

// Zeroes the histograms (the caller puts a barrier before radix_select).
template <int NT, int NH>
__device__ __forceinline__ void radix_clear(RadixScratch<NT, NH>& rs) {
  for (int i = threadIdx.x; i < NH * kSelBins; i += NT) (&rs.hist[0][0])[i] = 0u;
}

// Radix select among values v in [0, 2^nbits) (nbits <= 32) that each thread
// visits with visit(f) (f(v) for each of its values). Levels of up to 12 bits
// from the top bit down find where the krem-th largest value lies (krem: on
// entry, how many values to keep, at least 1 and at most their number); a level
// whose threshold bin is kept whole ends the select. On return (same in every
// thread) the kept values are those with (v & pmask) > prefix, then krem of
// those with (v & pmask) == prefix (the lowest indices first). `full` tells
// whether every one of the nbits bits was resolved. xn further copies of the
// value xv take part (counted by thread 0), ranked after every visited value.
template <int NT, int NH, typename Visit>
__device__ __forceinline__ void radix_select(Visit visit, int nbits, uint32_t& prefix, uint32_t& pmask,
                                             uint32_t& krem, bool& full, RadixScratch<NT, NH>& rs,
                                             uint32_t xv = 0u, uint32_t xn = 0u) {
  prefix = 0;
  pmask = 0;
  full = true;
#pragma unroll
  for (int lv = 0; lv < 3; ++lv) {
    const int top = nbits - 12 * lv;   // bits still unresolved
    if (top <= 0) break;
    const int width = top < 12 ? top : 12;
    const int shift = top - width;
    const uint32_t dm = (1u << width) - 1u;
    uint32_t* h = rs.hist[NH == 1 ? 0 : lv];
    if (NH == 1 && lv > 0) {   // one histogram: clear the previous level's counts first
      for (int i = threadIdx.x; i < kSelBins; i += NT) h[i] = 0u;
      __syncthreads();
    }
    const uint32_t pf = prefix, pm = pmask;
    visit([&](uint32_t v) {
      if ((v & pm) == pf) atomicAdd(&h[(v >> shift) & dm], 1u);
    });
    if (threadIdx.x == 0 && xn && (xv & pm) == pf) atomicAdd(&h[(xv >> shift) & dm], xn);
    __syncthreads();
    find_threshold<NT>(h, 1 << width, krem, rs.wsum[lv], rs.out[lv]);
    prefix |= rs.out[lv][0] << shift;
    pmask |= dm << shift;
    krem = rs.out[lv][1];
    if (rs.out[lv][2] && shift > 0) {
      full = false;   // the threshold bin is kept whole: its lower bits do not matter
      break;
    }
  }
}

// Minimum and maximum over the workgroup (one barrier; wmin / wmax of NT / 64).
template <int NT = kSelThreads>
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t* wmin, uint32_t* wmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, kWave));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, kWave));
  }
  if (lane == 0) {
    wmin[wave] = lo;
    wmax[wave] = hi;
  }
  __syncthreads();
  lo = wmin[0];
  hi = wmax[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    lo = min(lo, wmin[w]);
    hi = max(hi, wmax[w]);
  }
}

}  // namespace misa
