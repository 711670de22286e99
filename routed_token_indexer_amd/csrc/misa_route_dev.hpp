// Device building blocks of the block-pooled router, shared by the router
// kernels and the fused decode step so that every path computes the same
// per-head aggregates, bit for bit (same loads, MFMA sequence and sums).
#pragma once

#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {

__device__ __forceinline__ void query_prefix(const RouteArgs& a, int64_t t, int& seq, int& p) {
  if (t >= a.T) {
    seq = -1;
    p = 0;
    return;
  }
  seq = a.q_seq[t];
  p = a.q_len[t];
  if (seq < 0 || seq >= a.nseq) {
    seq = -1;
    p = 0;
  }
  p = p < 0 ? 0 : (p > a.Lmax ? (int)a.Lmax : p);
}

// bf16 round-to-nearest-even of x, and of the remainder x - hi.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void split_hi_lo(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne_bits(x);
  const float r = x - __uint_as_float(hi << 16);
  lo = bf16_rne_bits(r);
}

// Sum of the partial block's keys into s[0..D) (all lanes of one wave), rows in
// order. The loads go out 16 rows at a time (a load per row and wait would make
// the sum one memory round trip per key); only the adds are sequential.
template <int D>
__device__ __forceinline__ void wave_tail_sum(const RouteArgs& a, int seq, int start, int n_tail, float* s) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = D / 64 > 0 ? D / 64 : 1;
  constexpr int RB = 16;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  if (n_tail > 0 && lane * PER < D) {
    const uint16_t* kp = a.k + ((int64_t)seq * a.Lmax + start) * D + lane * PER;
    for (int r0 = 0; r0 < n_tail; r0 += RB) {
      uint16_t v[RB][PER];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int r = min(r0 + rr, n_tail - 1);   // rows past the tail re-read the last one and are not added
#pragma unroll
        for (int i = 0; i < PER; ++i) v[rr][i] = kp[(int64_t)r * D + i];
      }
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const bool in = r0 + rr < n_tail;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const float x = __uint_as_float((uint32_t)v[rr][i] << 16);
          acc[i] = in ? acc[i] + x : acc[i];
        }
      }
    }
  }
  if (lane * PER < D) {
#pragma unroll
    for (int i = 0; i < PER; ++i) s[lane * PER + i] = acc[i];
  }
}

// Tail dot x_g = q_g . S_tail for lane g < H (q read from global, S_tail in LDS).
template <int D>
__device__ __forceinline__ float tail_dot(const RouteArgs& a, int64_t t, int lane, const float* s) {
  float x = 0.f;
  if (lane < a.H) {
    const u32x4* qrow = reinterpret_cast<const u32x4*>(a.q + (t * a.H + lane) * D);
    u32x4 qv[D / 8];   // the whole row requested at once
#pragma unroll
    for (int i = 0; i < D / 8; ++i) qv[i] = qrow[i];
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const u32x4 v = qv[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x = fmaf(bf16_lo(v[e]), s[8 * i + 2 * e], x);
        x = fmaf(bf16_hi(v[e]), s[8 * i + 2 * e + 1], x);
      }
    }
  }
  return x;
}

// Per-head sums over block tiles [jb, je) (tiles of 16 blocks, stepping `stride`
// tiles) of max(q_g . Kbar_j, 0), for the RTQ row tiles of query t.
// On return, lanes with (lane & 15) == 0 of group g hold rows 4g..4g+3 of each tile.
template <int D, int RTQ>
__device__ __forceinline__ void block_affinity(const RouteArgs& a, int64_t t, int seq, int jb, int je, int stride,
                                               float (&rs)[RTQ][4]) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  u32x4 afrag[RTQ][KS];
#pragma unroll
  for (int r = 0; r < RTQ; ++r) {
    const int head = 16 * r + col;
    const bool hv = seq >= 0 && head < a.H;
    const uint16_t* qp = a.q + (t * a.H + (hv ? head : 0)) * D + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hv) v = *reinterpret_cast<const u32x4*>(qp + ks * 32);
      afrag[r][ks] = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) rs[r][j] = 0.f;
  }
  const int64_t nblk = a.Lmax / a.B;
  for (int j0 = jb; j0 < je; j0 += 16 * stride) {
    const int j = j0 + col;
    const bool bv = j < je;
    const float* kb = a.kbar + ((int64_t)(seq < 0 ? 0 : seq) * nblk + (bv ? j : 0)) * D + grp * 8;
    u32x4 bhi[KS], blo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      floatx4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
      if (bv) {
        v0 = *reinterpret_cast<const floatx4*>(kb + ks * 32);
        v1 = *reinterpret_cast<const floatx4*>(kb + ks * 32 + 4);
      }
      uint32_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        split_hi_lo(v0[e], h[e], l[e]);
        split_hi_lo(v1[e], h[4 + e], l[4 + e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bhi[ks][e] = h[2 * e] | (h[2 * e + 1] << 16);
        blo[ks][e] = l[2 * e] | (l[2 * e + 1] << 16);
      }
    }
#pragma unroll
    for (int r = 0; r < RTQ; ++r) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = mfma_16x16x32(afrag[r][ks], bhi[ks], acc);
        acc = mfma_16x16x32(afrag[r][ks], blo[ks], acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) rs[r][jj] += relu(acc[jj]);
    }
  }
  // sum over the 16 block columns (fixed xor tree)
#pragma unroll
  for (int r = 0; r < RTQ; ++r)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float v = rs[r][jj];
      v += __shfl_xor(v, 1, kWave);
      v += __shfl_xor(v, 2, kWave);
      v += __shfl_xor(v, 4, kWave);
      v += __shfl_xor(v, 8, kWave);
      rs[r][jj] = v;
    }
}

}  // namespace misa
