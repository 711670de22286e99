// Block filter composed with head routing: the coarse stage of a two-stage
// (block, then token) indexer search.
//
// HISA (thelatestinai.com paper cards, the HISA abstract) scores pooled block
// representations, drops the weak blocks and runs the indexer only on the
// tokens of the retained ones. The gist.science MISA summary presents head
// routing as combinable with such token-axis schemes ("Betekenis en Claims").
// Here the coarse score of complete block j of a query is the routed indexer
// formula on the block's mean key,
//     b_j = sum over the routed heads g (in the given order) of w_g * max(q_g . Kbar_j, 0),
// the m best complete blocks are kept (ties to the lower block id, by the
// ordinary top-k over the rows of b), and the partial last block is always
// kept. The candidate list of a query is then the token ids of its retained
// blocks followed by those of its partial block, ascending, -1 padded; the
// routed scoring and top-k of the fine stage run over that list in gather mode.
//
// block_score_kernel: one wave per (64 blocks, query). Lane j owns block j:
// its pooled key row is read with 16-byte loads (the row stays in the lane's
// registers four values at a time) and multiplied by the routed query rows,
// which sit in LDS as bf16 and are read as broadcasts. Eight heads are summed
// per pass over the row. The cost is a few µs of latency: 1024 pooled rows of
// d = 128 are 512 KiB per query.
#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {

// the routed query rows of block_score_kernel, [h][d] bf16 (dynamic LDS)
extern __shared__ __attribute__((aligned(16))) uint16_t block_q_lds[];

namespace {

constexpr int kBlockWave = 64;   // blocks per workgroup (one wave)
constexpr int kHeadGroup = 8;    // heads summed per pass over a pooled row

template <int D>
__global__ __launch_bounds__(kBlockWave) void block_score_kernel(BlockArgs a) {
  uint16_t* const s_q = block_q_lds;
  // 1-D grid: query t, chunk of 64 of its blocks
  const int64_t nchunk = a.nblk > 0 ? (a.nblk + kBlockWave - 1) / kBlockWave : 1;
  const int64_t t = blockIdx.x / nchunk;
  const int64_t chunk = blockIdx.x % nchunk;
  const int lane = threadIdx.x;
  const int p = query_prefix_len(a.q_seq, a.q_len, a.nseq, a.Lmax, t);
  const int nb = p < 0 ? 0 : p / a.B;
  if (chunk == 0 && lane == 0) a.blen[t] = nb;
  const int64_t j0 = chunk * kBlockWave;
  if (j0 >= nb) return;
  const int64_t seq = a.q_seq[t];
  const int h = a.h;
  const int32_t* hrow = a.heads + t * h;
  // stage the routed rows, 8 bf16 per 16-byte piece (an id outside [0, H)
  // stages zeros and contributes nothing)
  constexpr int PPR = D / 8;
  for (int i = lane; i < h * PPR; i += kBlockWave) {
    const int g = hrow[i / PPR];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (g >= 0 && g < a.H) v = *reinterpret_cast<const u32x4*>(a.q + (t * a.H + g) * D + (i % PPR) * 8);
    *reinterpret_cast<u32x4*>(s_q + (i / PPR) * D + (i % PPR) * 8) = v;
  }
  __syncthreads();
  const int64_t j = j0 + lane;
  const bool ok = j < nb;
  const float* krow = a.kbar + (seq * a.nblk + (ok ? j : j0)) * D;
  float b = 0.f;
  for (int g0 = 0; g0 < h; g0 += kHeadGroup) {
    float acc[kHeadGroup];
#pragma unroll
    for (int e = 0; e < kHeadGroup; ++e) acc[e] = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; c += 4) {
      const floatx4 kv = *reinterpret_cast<const floatx4*>(krow + c);
#pragma unroll
      for (int e = 0; e < kHeadGroup; ++e) {
        if (g0 + e < h) {
          const uint2 qq = *reinterpret_cast<const uint2*>(s_q + (g0 + e) * D + c);
          float x = acc[e];
          x = fmaf(bf16_lo(qq.x), kv[0], x);
          x = fmaf(bf16_hi(qq.x), kv[1], x);
          x = fmaf(bf16_lo(qq.y), kv[2], x);
          x = fmaf(bf16_hi(qq.y), kv[3], x);
          acc[e] = x;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kHeadGroup; ++e) {
      if (g0 + e < h) {
        const int g = hrow[g0 + e];
        if (g >= 0 && g < a.H) b += a.w[t * a.H + g] * relu(acc[e]);
      }
    }
  }
  if (ok) a.bscore[t * a.nblk + j] = b;
}

// cand[t][i]: token i of the retained blocks (in block order), then the
// partial block's tokens, then -1. The retained block list is ascending with
// its nk = min(m, complete blocks) valid entries first.
__global__ __launch_bounds__(256) void block_expand_kernel(BlockArgs a, const int32_t* __restrict__ blocks, int m,
                                                           int32_t* __restrict__ cand, int kc) {
  const int64_t nchunk = (kc + 255) / 256;
  const int64_t t = blockIdx.x / nchunk;
  const int i = (int)(blockIdx.x % nchunk) * 256 + threadIdx.x;
  if (i >= kc) return;
  const int p = query_prefix_len(a.q_seq, a.q_len, a.nseq, a.Lmax, t);
  const int nb = p < 0 ? 0 : p / a.B;
  const int nk = nb < m ? nb : m;
  const int nfull = nk * a.B;
  int32_t v = -1;
  if (i < nfull)
    v = blocks[t * m + i / a.B] * a.B + i % a.B;
  else if (i < nfull + (p - nb * a.B))
    v = nb * a.B + (i - nfull);
  cand[t * (int64_t)kc + i] = v;
}

}  // namespace

hipError_t launch_block_score(const BlockArgs& a, int d, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  // at least one workgroup per query: it writes the query's block count
  const int64_t nchunk = a.nblk > 0 ? (a.nblk + kBlockWave - 1) / kBlockWave : 1;
  const dim3 grid((unsigned)(nchunk * a.T));
  const size_t lds = (size_t)a.h * d * sizeof(uint16_t);
  switch (d) {
    case 32: hipLaunchKernelGGL(block_score_kernel<32>, grid, dim3(kBlockWave), lds, st, a); break;
    case 64: hipLaunchKernelGGL(block_score_kernel<64>, grid, dim3(kBlockWave), lds, st, a); break;
    case 128: hipLaunchKernelGGL(block_score_kernel<128>, grid, dim3(kBlockWave), lds, st, a); break;
    case 256: hipLaunchKernelGGL(block_score_kernel<256>, grid, dim3(kBlockWave), lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_block_expand(const BlockArgs& a, const int32_t* blocks, int m, int32_t* cand, int kc,
                               hipStream_t st) {
  if (a.T == 0 || kc == 0) return hipSuccess;
  const dim3 grid((unsigned)((kc + 255) / 256 * a.T));
  hipLaunchKernelGGL(block_expand_kernel, grid, dim3(256), 0, st, a, blocks, m, cand, kc);
  return hipGetLastError();
}

}  // namespace misa
