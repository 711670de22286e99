// Block mean-pooling of the indexer keys.
//
// MISA pages (gist.science "Methodologie: MISA", block-pooled router): the
// prefix is cut into blocks of B tokens and the router works on the mean-pooled
// keys of those blocks. This kernel stores the fp32 means of the complete
// blocks of every sequence; a query's partial last block is pooled by the
// router itself.
//
// misa_pool_update pools only the blocks that an append to the key cache
// completed, so that a decode loop keeps the pooled keys current at the cost of
// one block per sequence every B tokens.
//
// One wave per (sequence, block): each lane reads 16 contiguous bytes of a key
// row per load, so a wave instruction covers 1 KiB of consecutive key rows, and
// sixteen such loads per lane are in flight at once; the per-lane fp32 sums (rows
// in order) are combined with a fixed xor tree (deterministic order).
#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {
namespace {

// Mean of block j of sequence seq into kbar[seq][j] (one wave; nblk = Lmax / B
// blocks per sequence in kbar). The same code serves the full pooling and the
// incremental update, so both write the same bits.
template <int D>
__device__ __forceinline__ void pool_block(const uint16_t* __restrict__ k, int64_t Lmax, int64_t nblk, int B,
                                           float* __restrict__ kbar, int64_t seq, int64_t j) {
  constexpr int LPR = D / 8;       // lanes per key row
  constexpr int RPI = 64 / LPR;    // rows per wave instruction
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, c8 = (lane % LPR) * 8;
  const uint16_t* base = k + (seq * Lmax + j * B) * D + c8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // RB rows per lane in flight (clamped reads), then added in row order: one
  // memory round trip per RB * RPI rows instead of one per RPI rows (a block of
  // 64 rows of d = 128 in one trip)
  constexpr int RB = 16;
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
    float* o = kbar + (seq * nblk + j) * D + c8;
    const float fb = (float)B;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = acc[i] / fb;
  }
}

// every complete block: one wave per (sequence, block)
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ k, int64_t Lmax, int64_t nblk,
                                                   int B, float* __restrict__ kbar, int64_t total) {
  const int64_t gb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gb >= total) return;
  pool_block<D>(k, Lmax, nblk, B, kbar, gb / nblk, gb % nblk);
}

// the blocks an append completed: wave (n, i) pools block prev / B + i of
// sequence n if it ends inside (prev, next] (nb waves per sequence cover every
// such block when next - prev <= max_new, nb = max_new / B + 1)
template <int D>
__global__ __launch_bounds__(256) void pool_update_kernel(const uint16_t* __restrict__ k, int64_t nseq, int64_t Lmax,
                                                          int64_t nblk, int B, const int32_t* __restrict__ prev_len,
                                                          const int32_t* __restrict__ new_len, int nb,
                                                          float* __restrict__ kbar) {
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= nseq * nb) return;
  const int64_t n = gw / nb;
  const int i = (int)(gw % nb);
  const int prev = prev_len[n], next = new_len[n];
  if (prev < 0 || next < prev || next > Lmax) return;   // not a valid append: nothing to pool
  const int64_t j = prev / B + i;
  if ((j + 1) * B > next) return;   // block still open after the append
  pool_block<D>(k, Lmax, nblk, B, kbar, n, j);
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

hipError_t launch_pool_update(const uint16_t* k, int64_t nseq, int64_t Lmax, int d, int B, const int32_t* prev_len,
                              const int32_t* new_len, int max_new, float* kbar, hipStream_t st) {
  const int64_t nblk = Lmax / B;
  if (nseq == 0 || nblk == 0) return hipSuccess;
  const int nb = max_new / B + 1;
  const dim3 grid((unsigned)((nseq * nb + 3) / 4));
#define MISA_POOL_UPDATE(D_)                                                                          \
  hipLaunchKernelGGL(pool_update_kernel<D_>, grid, dim3(256), 0, st, k, nseq, Lmax, nblk, B, prev_len, new_len, nb, \
                     kbar)
  switch (d) {
    case 32: MISA_POOL_UPDATE(32); break;
    case 64: MISA_POOL_UPDATE(64); break;
    case 128: MISA_POOL_UPDATE(128); break;
    case 256: MISA_POOL_UPDATE(256); break;
    default: return hipErrorInvalidValue;
  }
#undef MISA_POOL_UPDATE
  return hipGetLastError();
}

}  // namespace misa
