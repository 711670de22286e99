// Block mean-pooling of the indexer keys.
//
// MISA pages (gist.science "Methodologie: MISA", block-pooled router): the
// prefix is cut into blocks of B tokens and the router works on the mean-pooled
// keys of those blocks. This kernel stores the fp32 means of the complete
// blocks of every sequence; a query's partial last block is pooled by the
// router itself.
//
// One wave per (sequence, block): each lane reads 16 contiguous bytes of a key
// row per load, so a wave instruction covers 1 KiB of consecutive key rows, and
// eight such loads per lane are in flight at once; the per-lane fp32 sums (rows
// in order) are combined with a fixed xor tree (deterministic order).
#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ k, int64_t Lmax, int64_t nblk,
                                                   int B, float* __restrict__ kbar, int64_t total) {
  constexpr int LPR = D / 8;       // lanes per key row
  constexpr int RPI = 64 / LPR;    // rows per wave instruction
  const int lane = threadIdx.x & 63;
  const int64_t gb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gb >= total) return;
  const int64_t seq = gb / nblk, j = gb % nblk;
  const int sub = lane / LPR, c8 = (lane % LPR) * 8;
  const uint16_t* base = k + (seq * Lmax + j * B) * D + c8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // RB rows per lane in flight (clamped reads), then added in row order: one
  // memory round trip per RB * RPI rows instead of one per RPI rows
  constexpr int RB = 8;
  for (int r0 = sub; r0 < B; r0 += RB * RPI) {
    u32x4 v[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int r = r0 + u * RPI;
      v[u] = *reinterpret_cast<const u32x4*>(base + (int64_t)(r < B ? r : sub) * D);
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (r0 + u * RPI >= B) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(v[u][e]);
        acc[2 * e + 1] += bf16_hi(v[u][e]);
      }
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], off, kWave);
  if (sub == 0) {
    float* o = kbar + gb * D + c8;
    const float fb = (float)B;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = acc[i] / fb;
  }
}

}  // namespace

hipError_t launch_pool(const uint16_t* k, int64_t nseq, int64_t Lmax, int d, int B, float* kbar,
                       hipStream_t st) {
  const int64_t nblk = Lmax / B;
  const int64_t total = nseq * nblk;
  if (total == 0) return hipSuccess;
  dim3 grid((unsigned)((total + 3) / 4));
  switch (d) {
    case 32: hipLaunchKernelGGL(pool_kernel<32>, grid, dim3(256), 0, st, k, Lmax, nblk, B, kbar, total); break;
    case 64: hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(256), 0, st, k, Lmax, nblk, B, kbar, total); break;
    case 128: hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(256), 0, st, k, Lmax, nblk, B, kbar, total); break;
    case 256: hipLaunchKernelGGL(pool_kernel<256>, grid, dim3(256), 0, st, k, Lmax, nblk, B, kbar, total); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace misa
