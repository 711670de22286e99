// Proxy-query shared scan with per-query refinement (PIVOT-Refine).
//
// PIVOT (thelatestinai.com paper cards, the PIVOT abstract) folds a group of
// nearby queries into one proxy query, lets the proxy scan the full prefix
// once to obtain a candidate set, and (Refine) has every query of the group
// re-score those candidates with its own indexer and keep its own top-k. Groups
// are runs of G consecutive queries. The page does not say how the proxy is
// formed; this library takes the sum of the group's per-head queries, rounded
// to bf16 (nearest, ties to even) for the indexer, with the sum of their head
// weights: the mean up to the positive factor G, which changes no ranking and
// needs no division. The proxy scans the longest prefix of its group.
//
// pivot_proxy_kernel: one thread per (group, head, 8 dims) sums the group's
// query pieces in query order in fp32 (eight pieces requested at a time); the group's first thread of each head
// sums the weights, and thread 0 of the group writes its sequence (that of its
// first query) and longest prefix. pivot_broadcast_kernel copies each group's
// candidate row to its queries.
#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {
namespace {

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void pivot_proxy_kernel(PivotArgs a) {
  const int ppr = a.d / 8;                        // 8-dim pieces per head row
  const int64_t per = (int64_t)a.H * ppr;         // pieces per group
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.ng * per) return;
  const int64_t g = i / per;
  const int64_t r = i % per;                      // head r / ppr, piece r % ppr
  const int64_t t0 = g * a.G;
  const int64_t t1 = t0 + a.G < a.T ? t0 + a.G : a.T;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // eight queries' pieces in flight at a time (clamped reads), added in query order
  for (int64_t tb = t0; tb < t1; tb += 8) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t t = tb + j < t1 ? tb + j : t0;
      v[j] = *reinterpret_cast<const u32x4*>(a.q + (t * per + r) * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (tb + j >= t1) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(v[j][e]);
        acc[2 * e + 1] += bf16_hi(v[j][e]);
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = bf16_rne_bits(acc[2 * e]) | (bf16_rne_bits(acc[2 * e + 1]) << 16);
  *reinterpret_cast<u32x4*>(a.qp + (g * per + r) * 8) = o;
  if (r % ppr == 0) {
    const int hd = (int)(r / ppr);
    float ws = 0.f;
    for (int64_t t = t0; t < t1; ++t) ws += a.w[t * a.H + hd];
    a.wp[g * a.H + hd] = ws;
  }
  if (r == 0) {
    int len = 0;
    for (int64_t t = t0; t < t1; ++t) len = a.q_len[t] > len ? a.q_len[t] : len;
    a.gseq[g] = a.q_seq[t0];
    a.glen[g] = len;
  }
}

// one workgroup per (query, 1024 candidate slots): four slots per thread
__global__ __launch_bounds__(256) void pivot_broadcast_kernel(const int32_t* __restrict__ gcand,
                                                              int32_t* __restrict__ cand, int64_t T, int G, int kc) {
  const int64_t nchunk = (kc + 1023) / 1024;
  const int64_t t = blockIdx.x / nchunk;
  const int64_t src = (t / G) * kc, dst = t * kc;
  const int i0 = (int)(blockIdx.x % nchunk) * 1024 + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = i0 + 256 * j;
    if (i < kc) cand[dst + i] = gcand[src + i];
  }
}

}  // namespace

hipError_t launch_pivot_proxy(const PivotArgs& a, hipStream_t st) {
  if (a.ng == 0) return hipSuccess;
  const int64_t n = a.ng * (int64_t)a.H * (a.d / 8);
  hipLaunchKernelGGL(pivot_proxy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pivot_broadcast(const int32_t* gcand, int32_t* cand, int64_t T, int G, int kc, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t n = T * ((kc + 1023) / 1024);
  hipLaunchKernelGGL(pivot_broadcast_kernel, dim3((unsigned)n), dim3(256), 0, st, gcand, cand, T, G, kc);
  return hipGetLastError();
}

}  // namespace misa
