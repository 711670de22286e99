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
// the m best complete blocks are kept (ties to the lower block id; by
// block_select_kernel below, or by the ordinary top-k over the rows of b for
// rows of more than 4096 blocks), and the partial last block is always kept. The candidate list of a query is then the token ids of its retained
// blocks followed by those of its partial block, ascending, -1 padded; the
// routed scoring and top-k of the fine stage run over that list in gather mode.
//
// block_score_kernel: one workgroup of four waves per (64 blocks, query). The
// 64 pooled key rows (contiguous in memory) are read once, coalesced, into an
// LDS tile (16-byte pieces XOR-swizzled by row, so that the row reads below are
// conflict-free; d = 256 in four quarters). Lane j of every wave then takes row j
// into registers, and wave w multiplies it by the routed query rows w, w + 4,
// ... (bf16 in LDS, read as broadcasts). The per-head dots meet in LDS, where
// wave 0 applies the ReLU and the weights in head order.
#include "misa_common.hpp"
#include "misa_internal.hpp"
#include "misa_select.hpp"

namespace misa {

// dynamic LDS of block_score_kernel: the routed query rows [h][d] bf16, then
// the per-head dots [h][64] fp32
extern __shared__ __attribute__((aligned(16))) uint16_t block_q_lds[];

namespace {

constexpr int kBlockWave = 64;   // blocks per workgroup
constexpr int kBlockWaves = 4;   // waves per workgroup (heads split among them)

template <int D>
__global__ __launch_bounds__(64 * kBlockWaves) void block_score_kernel(BlockArgs a) {
  // row floats staged at once: with h = 64 routed rows the tile, the query
  // rows and the dots fill at most 64 KiB of LDS
  constexpr int HALF = D == 256 ? 64 : D;
  constexpr int NV = HALF / 4;              // 16-byte pieces of a staged row
  constexpr int NT = 64 * kBlockWaves;
  __shared__ floatx4 s_k[kBlockWave * NV];  // [64 rows][NV pieces], piece u of row r at u ^ (r & 7)
  uint16_t* const s_q = block_q_lds;                                     // [h][D] bf16
  float* const s_dot = reinterpret_cast<float*>(block_q_lds + a.h * D);  // [h][64] fp32
  // 1-D grid: query t, chunk of 64 of its blocks
  const int64_t nchunk = a.nblk > 0 ? (a.nblk + kBlockWave - 1) / kBlockWave : 1;
  const int64_t t = blockIdx.x / nchunk;
  const int64_t chunk = blockIdx.x % nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = query_prefix_len(a.q_seq, a.q_len, a.nseq, a.Lmax, t);
  const int nb = p < 0 ? 0 : p / a.B;
  if (chunk == 0 && tid == 0) a.blen[t] = nb;
  const int64_t j0 = chunk * kBlockWave;
  if (j0 >= nb) return;
  const int64_t seq = a.q_seq[t];
  const int h = a.h;
  const int32_t* hrow = a.heads + t * h;
  const float* kseq = a.kbar + seq * a.nblk * D;
  // tile loads: piece i of the tile is row i / NV (clamped to the last visible
  // block), piece i % NV
  constexpr int PPT = kBlockWave * NV / NT;   // pieces per thread
  auto load_tile = [&](int c0, floatx4* v) {
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int i = tid + NT * r;
      const int64_t row = j0 + i / NV < nb ? j0 + i / NV : nb - 1;
      v[r] = *reinterpret_cast<const floatx4*>(kseq + row * D + c0 + 4 * (i % NV));
    }
  };
  auto store_tile = [&](const floatx4* v) {
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int i = tid + NT * r;
      const int row = i / NV, u = i % NV;
      s_k[row * NV + (u ^ (row & 7))] = v[r];
    }
  };
  floatx4 tv[PPT];
  load_tile(0, tv);
  // stage the routed rows, 8 bf16 per 16-byte piece (an id outside [0, H)
  // stages zeros and contributes nothing)
  constexpr int PPR = D / 8;
  for (int i = tid; i < h * PPR; i += NT) {
    const int g = hrow[i / PPR];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (g >= 0 && g < a.H) v = *reinterpret_cast<const u32x4*>(a.q + (t * a.H + g) * D + (i % PPR) * 8);
    *reinterpret_cast<u32x4*>(s_q + (i / PPR) * D + (i % PPR) * 8) = v;
  }
#pragma unroll
  for (int c0 = 0; c0 < D; c0 += HALF) {
    if (c0 > 0) {
      load_tile(c0, tv);
      __syncthreads();   // every wave has read the previous half from the tile
    }
    store_tile(tv);
    __syncthreads();
    floatx4 kv[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) kv[u] = s_k[lane * NV + (u ^ (lane & 7))];
    for (int g = wave; g < h; g += kBlockWaves) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const uint2 qq = *reinterpret_cast<const uint2*>(s_q + g * D + c0 + 4 * u);
        float x = acc[u & 3];
        x = fmaf(bf16_lo(qq.x), kv[u][0], x);
        x = fmaf(bf16_hi(qq.x), kv[u][1], x);
        x = fmaf(bf16_lo(qq.y), kv[u][2], x);
        x = fmaf(bf16_hi(qq.y), kv[u][3], x);
        acc[u & 3] = x;
      }
      const float dot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      s_dot[g * 64 + lane] = c0 == 0 ? dot : s_dot[g * 64 + lane] + dot;   // only this wave owns head g
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const int64_t j = j0 + lane;
  float b = 0.f;
  for (int g = 0; g < h; ++g) {
    const int hg = hrow[g];
    if (hg >= 0 && hg < a.H) b += a.w[t * a.H + hg] * relu(s_dot[g * 64 + lane]);
  }
  if (j < nb) a.bscore[t * a.nblk + j] = b;
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

// The m best complete blocks of one query and its candidate list, in one
// workgroup of 1024 threads (rows of at most kSelMaxBlocks block scores).
// Thread i holds blocks 4i .. 4i + 3, so thread order is block order. A radix
// select over the order-preserving keys finds the threshold; the kept blocks
// (keys above it, then the lowest-id ones equal to it) get their output slots
// from two prefix sums in thread order, so the list comes out ascending. The
// candidate list is then written from the kept list in LDS, coalesced.
constexpr int kSelEPT = 4;
constexpr int kSelMaxBlocks = kSelEPT * kSelThreads;

__global__ __launch_bounds__(kSelThreads) void block_select_kernel(BlockArgs a, int m, int32_t* __restrict__ blocks,
                                                                  int32_t* __restrict__ cand, int kc) {
  __shared__ RadixScratch<kSelThreads, 1> rs;
  __shared__ __attribute__((aligned(16))) uint32_t wsum2[2 * kSelWaves];
  __shared__ int32_t s_blk[kSelMaxBlocks];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = query_prefix_len(a.q_seq, a.q_len, a.nseq, a.Lmax, t);
  const int nb = p < 0 ? 0 : p / a.B;
  const int ntail = p < 0 ? 0 : p - nb * a.B;
  const int nk = nb < m ? nb : m;
  uint32_t u[kSelEPT];
#pragma unroll
  for (int r = 0; r < kSelEPT; ++r) {
    const int j = kSelEPT * tid + r;
    u[r] = j < nb ? score_key(a.bscore[t * a.nblk + j]) : 0u;
  }
  const bool all = nb <= m;
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)nk;
  if (!all) {
    radix_clear(rs);
    __syncthreads();
    bool full;
    radix_select<kSelThreads, 1>(
        [&](auto f) {
#pragma unroll
          for (int r = 0; r < kSelEPT; ++r)
            if (kSelEPT * tid + r < nb) f(u[r]);
        },
        32, prefix, pmask, krem, full, rs);
  }
  // 2 = above the threshold (kept), 1 = equal to it (kept if among the first krem), 0 = below
  auto cls = [&](int r) -> int {
    if (kSelEPT * tid + r >= nb) return 0;
    if (all || (u[r] & pmask) > prefix) return 2;
    return (u[r] & pmask) == prefix ? 1 : 0;
  };
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int r = 0; r < kSelEPT; ++r) {
    const int c = cls(r);
    ngt += c == 2 ? 1u : 0u;
    neq += c == 1 ? 1u : 0u;
  }
  uint32_t eq_before;
  const uint32_t gt_before = block_excl_scan2(ngt, neq, wsum2, eq_before);
  uint32_t pos = gt_before + (eq_before < krem ? eq_before : krem);
  uint32_t er = eq_before;
#pragma unroll
  for (int r = 0; r < kSelEPT; ++r) {
    const int c = cls(r);
    bool keep = c == 2;
    if (c == 1) keep = er++ < krem;
    if (keep) {
      const int j = kSelEPT * tid + r;
      s_blk[pos] = j;
      blocks[t * m + pos] = j;
      ++pos;
    }
  }
  for (int i = nk + tid; i < m; i += kSelThreads) blocks[t * m + i] = -1;
  __syncthreads();
  const int nfull = nk * a.B;
  int32_t* crow = cand + t * (int64_t)kc;
  for (int i = tid; i < kc; i += kSelThreads) {
    int32_t v = -1;
    if (i < nfull)
      v = s_blk[i / a.B] * a.B + i % a.B;
    else if (i < nfull + ntail)
      v = nb * a.B + (i - nfull);
    crow[i] = v;
  }
}

}  // namespace

bool block_select_fused(const BlockArgs& a) { return a.nblk <= kSelMaxBlocks; }

hipError_t launch_block_select(const BlockArgs& a, int m, int32_t* blocks, int32_t* cand, int kc, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (!block_select_fused(a)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_select_kernel, dim3((unsigned)a.T), dim3(kSelThreads), 0, st, a, m, blocks, cand, kc);
  return hipGetLastError();
}

hipError_t launch_block_score(const BlockArgs& a, int d, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  // at least one workgroup per query: it writes the query's block count
  const int64_t nchunk = a.nblk > 0 ? (a.nblk + kBlockWave - 1) / kBlockWave : 1;
  const dim3 grid((unsigned)(nchunk * a.T)), block(64 * kBlockWaves);
  const size_t lds = (size_t)a.h * d * sizeof(uint16_t) + (size_t)a.h * 64 * sizeof(float);
  switch (d) {
    case 32: hipLaunchKernelGGL(block_score_kernel<32>, grid, block, lds, st, a); break;
    case 64: hipLaunchKernelGGL(block_score_kernel<64>, grid, block, lds, st, a); break;
    case 128: hipLaunchKernelGGL(block_score_kernel<128>, grid, block, lds, st, a); break;
    case 256: hipLaunchKernelGGL(block_score_kernel<256>, grid, block, lds, st, a); break;
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
