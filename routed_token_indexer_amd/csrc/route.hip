// Block-pooled head router of MISA.
//
// MISA pages (MISA abstract; gist.science "Methodologie: MISA"): the prefix of
// length p is split into M = ceil(p / B) blocks, the router computes per-head
// affinities against the mean-pooled keys, aggregates them into one importance
// per head and keeps the top-h heads; its cost is O(H_I * M).
//
// The aggregate is the head's own indexer term on the pooled keys,
//     r_g = w_g * sum_{j < M} max(q_g . Kbar_j, 0),
// where the last block may be partial (mean over its visible tokens). Heads are
// ranked by rho_g = n_tail * r_g (n_tail = size of the partial block, 1 if none):
//     rho_g = w_g * (n_tail * sum_{complete j} max(q_g . Kbar_j, 0) + max(q_g . S_tail, 0)),
// with S_tail the plain sum of the partial block's keys. Multiplying every r_g by
// the same positive n_tail keeps the ranking and removes the division, so on
// inputs whose products and sums are exact in fp32 the ranking is exact too.
// Ties go to the lower head id; the routed set is written in ascending head id.
//
// The affinities q_g . Kbar_j run on the matrix cores: the query's head rows
// are MFMA A-fragments, 16 pooled blocks form a B tile. Pooled keys are fp32,
// so each B value is split into bf16 hi + lo (two MFMAs): hi + lo carries 16
// significant bits, and pooled keys of small-integer inputs are exact in hi.
//   decode  (few queries, long prefixes): a workgroup takes one query and a
//           chunk of blocks, its waves split the blocks; a second small kernel
//           sums the chunk partials in chunk order and selects the heads.
//   prefill (many queries): a workgroup takes four consecutive queries, one
//           per wave; the pooled keys of their sequence are staged in LDS as
//           hi / lo tiles once for all of them, and each wave selects its
//           query's heads.
#include "misa_common.hpp"
#include "misa_internal.hpp"
#include "misa_score_dev.hpp"
#include "misa_route_dev.hpp"

namespace misa {
namespace {

// Rank heads by rho (ties: lower id) and write the routed set. Runs in one
// wave; lane g < H holds head g's complete-block aggregate A and partial-block dot x.
__device__ __forceinline__ void route_select_w(const RouteArgs& a, int64_t t, int lane, float w, float A, float x,
                                               int n_tail) {
  int pos;
  float r;
  const bool sel = route_rank(a.H, a.h, lane, w, A, x, n_tail, pos, r);
  if (sel) a.heads[t * a.h + pos] = lane;
  if (lane < a.H && a.router_key) a.router_key[t * a.H + lane] = r;
}
__device__ __forceinline__ void route_select(const RouteArgs& a, int64_t t, int lane, float A, float x,
                                             int n_tail) {
  route_select_w(a, t, lane, lane < a.H ? a.w[t * a.H + lane] : 0.f, A, x, n_tail);
}

// decode: grid (nchunk, T); the four waves split the chunk's blocks.
template <int D, int RTQ>
__global__ __launch_bounds__(256) void route_decode_kernel(RouteArgs a) {
  __shared__ float red[4][64];
  __shared__ float stail[D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x;
  int seq, p;
  query_prefix(a, t, seq, p);
  const int nfull = p / a.B;
  const int jb = c * a.chunk_blocks + wave * 16;
  const int je = min((c + 1) * a.chunk_blocks, nfull);
  float rs[RTQ][4];
  block_affinity<D, RTQ>(a, t, seq, jb, je, 4, rs);
  if ((lane & 15) == 0) {
#pragma unroll
    for (int r = 0; r < RTQ; ++r)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) red[wave][16 * r + 4 * (lane >> 4) + jj] = rs[r][jj];
  }
  __syncthreads();
  const int tid = threadIdx.x;
  const float A = tid < 64 ? ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid] : 0.f;
  if (a.fused) {
    // fused decode pipeline: emit the chunk partial and (chunk 0) the partial-block
    // dot; the scoring kernel sums them and selects the heads. Every workgroup also
    // clears a slice of the later launches' zero-initialised state.
    if (tid < a.H) a.partial[(t * a.nchunk + c) * a.H + tid] = A;
    const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
    for (int z = 0; z < 2; ++z)
      for (int64_t i = lin * 256 + tid; i < a.zero_words[z]; i += nwg * 256) a.zero[z][i] = 0u;
    if (c != 0 || wave != 0) return;
    const int n_tail = p - nfull * a.B;
    wave_tail_sum<D>(a, seq, nfull * a.B, n_tail, stail);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float x = n_tail > 0 ? tail_dot<D>(a, t, lane, stail) : 0.f;
    if (lane < a.H) a.xtail[t * a.H + lane] = x;
    return;
  }
  if (a.nchunk > 1) {
    if (tid < a.H) a.partial[(t * a.nchunk + c) * a.H + tid] = A;
    return;
  }
  if (wave != 0) return;
  const int n_tail = p - nfull * a.B;
  wave_tail_sum<D>(a, seq, nfull * a.B, n_tail, stail);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float x = n_tail > 0 ? tail_dot<D>(a, t, lane, stail) : 0.f;
  route_select(a, t, lane, A, x, n_tail);
}

// decode, several chunks: sum the partials in chunk order, add the tail, select.
template <int D>
__global__ __launch_bounds__(64) void route_final_kernel(RouteArgs a) {
  __shared__ float stail[D];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  int seq, p;
  query_prefix(a, t, seq, p);
  const int nfull = p / a.B;
  const int n_tail = p - nfull * a.B;
  const float A = sum_partials(a.partial, t, a.nchunk, a.H, lane);
  wave_tail_sum<D>(a, seq, nfull * a.B, n_tail, stail);
  __syncthreads();
  const float x = n_tail > 0 ? tail_dot<D>(a, t, lane, stail) : 0.f;
  route_select(a, t, lane, A, x, n_tail);
}

// prefill, tiled: grid (ceil(T / (4 * QPW))); a workgroup routes QPW consecutive
// queries per wave. When they all read one sequence, every 64-block chunk of its
// pooled keys is split into bf16 hi / lo once and staged in LDS (16-byte piece p
// of block row j at slot p ^ (j & SWM): an XOR swizzle that stays inside the
// row), and each 16-block tile feeds the MFMAs of every query's head rows; a
// query adds only its complete blocks. Per query the tiles, their order and the
// MFMA sequence are those of block_affinity, so the aggregates are the same bit
// for bit; the partial block is staged and summed while the query rows load.
// Workgroups whose queries span several sequences route each query on its own
// wave (block_affinity over its blocks).
template <int D, int RTQ, int QPW>
__global__ __launch_bounds__(256, 2) void route_prefill_tiled_kernel(RouteArgs a) {
  constexpr int KS = D / 32;
  constexpr int PPR = D / 8;                 // 16-byte bf16 pieces per pooled row
  constexpr int SB = 64;                     // pooled blocks per LDS stage
  constexpr int QT = 4 * QPW;
  constexpr int SPT = SB * PPR / 256;        // staged pieces per thread
  constexpr int SWM = (PPR < 16 ? PPR : 16) - 1;   // XOR swizzle within the row
  static_assert(SPT >= 1 && PPR <= 32, "staging");
  __shared__ __attribute__((aligned(16))) uint16_t s_hi[SB * D], s_lo[SB * D];
  __shared__ float red[QT][64];
  __shared__ float stail[QT][D];
  __shared__ int s_seq[QT], s_nfull[QT], s_ntail[QT], s_shared_seq, s_nmax;
  __shared__ __attribute__((aligned(16))) uint16_t s_tail[SB * D];   // rows of the staged partial block
  __shared__ int s_tst, s_tlen;   // staged partial block: first block index, rows (0: none)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * QT;
  if (tid < QT) {
    int seq, p;
    query_prefix(a, t0 + tid, seq, p);
    s_seq[tid] = seq;
    s_nfull[tid] = p / a.B;
    s_ntail[tid] = p - (p / a.B) * a.B;
  }
  __syncthreads();
  if (tid == 0) {
    int sq = -2, nmax = 0;
    for (int i = 0; i < QT; ++i) {
      if (s_seq[i] < 0) continue;
      sq = (sq == -2 || sq == s_seq[i]) ? s_seq[i] : -3;
      nmax = max(nmax, s_nfull[i]);
    }
    s_shared_seq = sq;   // -2: no valid query, -3: several sequences
    s_nmax = nmax;
  }
  __syncthreads();
  const int seq_all = s_shared_seq;

  // per query of this wave: head aggregates in red[], then tail, ranking, routed set
  auto finish = [&](int i) {
    const int ql = wave * QPW + i;
    const int64_t t = t0 + ql;
    if (t >= a.T) return;
    int seq, p;
    query_prefix(a, t, seq, p);
    const int nfull = p / a.B;
    const int n_tail = p - nfull * a.B;
    wave_tail_sum<D>(a, seq, nfull * a.B, n_tail, stail[ql]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float A = red[ql][lane];
    const float x = n_tail > 0 ? tail_dot<D>(a, t, lane, stail[ql]) : 0.f;
    route_select(a, t, lane, A, x, n_tail);
  };
  auto put_red = [&](int ql, const float (&rs)[RTQ][4]) {
    if (col == 0) {
#pragma unroll
      for (int r = 0; r < RTQ; ++r)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) red[ql][16 * r + 4 * grp + jj] = rs[r][jj];
    }
  };

  if (seq_all == -3) {   // several sequences: each query on its own
#pragma unroll 1
    for (int i = 0; i < QPW; ++i) {
      const int ql = wave * QPW + i;
      const int64_t t = t0 + ql;
      if (t >= a.T) break;
      int seq, p;
      query_prefix(a, t, seq, p);
      float rs[RTQ][4];
      block_affinity<D, RTQ>(a, t, seq, 0, p / a.B, 1, rs);
      put_red(ql, rs);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      finish(i);
    }
    return;
  }

  // ---- one sequence. The rows of the queries' partial block (consecutive
  // positions share it, except across a block boundary) are requested first,
  // then the head weights and the query rows; staging the partial block and
  // summing it per query then overlap the wait for the query rows, since loads
  // complete in order
  if (tid == 0) {
    int st = -1, len = 0;
    for (int q = 0; q < QT; ++q) {
      if (s_seq[q] < 0 || s_ntail[q] == 0) continue;
      if (st < 0 || st == s_nfull[q]) {
        st = s_nfull[q];
        len = max(len, s_ntail[q]);
      }
    }
    s_tst = st;
    s_tlen = len <= SB ? len : 0;
  }
  __syncthreads();
  const int tst = s_tst, tlen = s_tlen;
  u32x4 tr[SPT];
  {
    const uint16_t* src = a.k + ((int64_t)(seq_all < 0 ? 0 : seq_all) * a.Lmax + (int64_t)(tst < 0 ? 0 : tst) * a.B) * D;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int pc = tid + 256 * s;
      if (pc < tlen * PPR) tr[s] = *reinterpret_cast<const u32x4*>(src + (int64_t)pc * 8);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // (a volatile load from a clamped index: issued here, not moved next to its use)
  float wq[QPW];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int64_t t = t0 + wave * QPW + i;
    const bool ok = t < a.T && lane < a.H;
    const float v = *reinterpret_cast<const volatile float*>(a.w + (ok ? t * a.H + lane : 0));
    wq[i] = ok ? v : 0.f;
  }
  u32x4 afrag[QPW][RTQ][KS];
  int nf[QPW];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int ql = wave * QPW + i;
    const int64_t t = t0 + ql;
    const bool tv = t < a.T && s_seq[ql] >= 0;
    nf[i] = tv ? s_nfull[ql] : 0;
#pragma unroll
    for (int r = 0; r < RTQ; ++r) {
      const int head = 16 * r + col;
      const bool hv = tv && head < a.H;
      const uint16_t* qp = a.q + ((hv ? t : 0) * a.H + (hv ? head : 0)) * D + grp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qp + ks * 32);
        afrag[i][r][ks] = hv ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  const int nmax = s_nmax;
  const int64_t nblk_seq = a.Lmax / a.B;
  const float* kb_seq = a.kbar + (int64_t)(seq_all < 0 ? 0 : seq_all) * nblk_seq * D;
  floatx4 sv[SPT][2];
  auto stage_load = [&](int c0) {   // pooled rows [c0, c0 + SB) (rows past nmax read row 0)
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int pc = tid + 256 * s;
      const int jr = pc / PPR, piece = pc % PPR;
      const float* kp = kb_seq + (int64_t)(c0 + jr < nmax ? c0 + jr : 0) * D + piece * 8;
      sv[s][0] = *reinterpret_cast<const floatx4*>(kp);
      sv[s][1] = *reinterpret_cast<const floatx4*>(kp + 4);
    }
  };
  auto stage_store = [&](int c0) {   // as hi / lo (rows past nmax are zero)
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int pc = tid + 256 * s;
      const int jr = pc / PPR, piece = pc % PPR;
      const bool bv = c0 + jr < nmax;
      uint32_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        split_hi_lo(bv ? sv[s][0][e] : 0.f, h[e], l[e]);
        split_hi_lo(bv ? sv[s][1][e] : 0.f, h[4 + e], l[4 + e]);
      }
      u32x4 hv4, lv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv4[e] = h[2 * e] | (h[2 * e + 1] << 16);
        lv4[e] = l[2 * e] | (l[2 * e + 1] << 16);
      }
      const int slot = piece ^ (jr & SWM);
      *reinterpret_cast<u32x4*>(s_hi + jr * D + slot * 8) = hv4;
      *reinterpret_cast<u32x4*>(s_lo + jr * D + slot * 8) = lv4;
    }
  };
  // the first stage is requested with the rest, so that every load of the
  // prologue is in flight at once
  if (nmax > 0) stage_load(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < SPT; ++s) {
    const int pc = tid + 256 * s;
    if (pc < tlen * PPR) *reinterpret_cast<u32x4*>(s_tail + pc * 8) = tr[s];
  }
  if (nmax > 0) stage_store(0);
  __syncthreads();
  // per query: the partial-block sum S_tail, rows in order (the adds of
  // wave_tail_sum), from the staged rows 16 at a time so that the LDS reads
  // overlap; a second distinct partial block is summed from memory
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int ql = wave * QPW + i;
    const int seq = s_seq[ql];
    const int nfull = seq < 0 ? 0 : s_nfull[ql];
    const int n_tail = seq < 0 || t0 + ql >= a.T ? 0 : s_ntail[ql];
    if (n_tail == 0) continue;
    if (tlen > 0 && tst == nfull) {
      constexpr int PER = D / 64 > 0 ? D / 64 : 1;
      constexpr int RB = 16;
      if (lane * PER < D) {
        float acc[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = 0.f;
        for (int r0 = 0; r0 < n_tail; r0 += RB) {
          uint16_t v[RB][PER];
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) {
            const int r = min(r0 + rr, n_tail - 1);   // rows past the tail re-read the last one, not added
#pragma unroll
            for (int e = 0; e < PER; ++e) v[rr][e] = s_tail[r * D + lane * PER + e];
          }
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) {
            const bool in = r0 + rr < n_tail;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
              const float x = __uint_as_float((uint32_t)v[rr][e] << 16);
              acc[e] = in ? acc[e] + x : acc[e];
            }
          }
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) stail[ql][lane * PER + e] = acc[e];
      }
    } else {
      wave_tail_sum<D>(a, seq, nfull * a.B, n_tail, stail[ql]);
    }
  }
  float rs[QPW][RTQ][4];
#pragma unroll
  for (int i = 0; i < QPW; ++i)
#pragma unroll
    for (int r = 0; r < RTQ; ++r)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) rs[i][r][jj] = 0.f;
  for (int c0 = 0; c0 < nmax; c0 += SB) {
    if (c0 > 0) {
      stage_load(c0);
      stage_store(c0);
      __syncthreads();
    }
    const int nb = min(SB, nmax - c0);
    for (int jt = 0; jt < nb; jt += 16) {
      const int jr = jt + col;
      u32x4 bhi[KS], blo[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int slot = (4 * ks + grp) ^ (jr & SWM);
        bhi[ks] = *reinterpret_cast<const u32x4*>(s_hi + jr * D + slot * 8);
        blo[ks] = *reinterpret_cast<const u32x4*>(s_lo + jr * D + slot * 8);
      }
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        const bool jv = c0 + jr < nf[i];
#pragma unroll
        for (int r = 0; r < RTQ; ++r) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            acc = mfma_16x16x32(afrag[i][r][ks], bhi[ks], acc);
            acc = mfma_16x16x32(afrag[i][r][ks], blo[ks], acc);
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) rs[i][r][jj] += jv ? relu(acc[jj]) : 0.f;
        }
      }
    }
    __syncthreads();   // the stage is rewritten next
  }
  // sum over the 16 block columns: the pairs of block_affinity's xor tree, as
  // DPP moves inside each 16-lane row. After the steps over lane ^ 1 and
  // lane ^ 2 every lane of a quad holds the same value, so its mirror partner
  // in the other quad (and then in the other half row) gives the same sum as
  // the lane ^ 4 (lane ^ 8) partner, bit for bit
#define MISA_DPP_ADD(v, ctrl) ((v) + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), (ctrl), 0xf, 0xf, false)))
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
#pragma unroll
    for (int r = 0; r < RTQ; ++r)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v = rs[i][r][jj];
        v = MISA_DPP_ADD(v, 0xb1);    // quad_perm [1, 0, 3, 2]: lane ^ 1
        v = MISA_DPP_ADD(v, 0x4e);    // quad_perm [2, 3, 0, 1]: lane ^ 2
        v = MISA_DPP_ADD(v, 0x141);   // row_half_mirror
        v = MISA_DPP_ADD(v, 0x140);   // row_mirror
        rs[i][r][jj] = v;
      }
    put_red(wave * QPW + i, rs[i]);
  }
#undef MISA_DPP_ADD
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // per query: the tail dot x_g = q_g . S_tail from the A fragments already in
  // registers (lane (col, grp) holds k-slots 32 ks + 8 grp .. + 8 of head
  // 16 r + col; the four groups' parts are added across lanes), instead of
  // reading the query rows from memory a second time
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int ql = wave * QPW + i;
    const int64_t t = t0 + ql;
    if (t >= a.T) break;
    const int n_tail = s_seq[ql] < 0 ? 0 : s_ntail[ql];
    float x = 0.f;
    if (n_tail > 0) {
      float xr[RTQ];
#pragma unroll
      for (int r = 0; r < RTQ; ++r) xr[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const floatx4 s0 = *reinterpret_cast<const floatx4*>(&stail[ql][32 * ks + 8 * grp]);
        const floatx4 s1 = *reinterpret_cast<const floatx4*>(&stail[ql][32 * ks + 8 * grp + 4]);
#pragma unroll
        for (int r = 0; r < RTQ; ++r) {
          const u32x4 v = afrag[i][r][ks];
          float acc = xr[r];
          acc = fmaf(bf16_lo(v[0]), s0[0], acc);
          acc = fmaf(bf16_hi(v[0]), s0[1], acc);
          acc = fmaf(bf16_lo(v[1]), s0[2], acc);
          acc = fmaf(bf16_hi(v[1]), s0[3], acc);
          acc = fmaf(bf16_lo(v[2]), s1[0], acc);
          acc = fmaf(bf16_hi(v[2]), s1[1], acc);
          acc = fmaf(bf16_lo(v[3]), s1[2], acc);
          acc = fmaf(bf16_hi(v[3]), s1[3], acc);
          xr[r] = acc;
        }
      }
#pragma unroll
      for (int r = 0; r < RTQ; ++r) {
        xr[r] += __shfl_xor(xr[r], 16, kWave);
        xr[r] += __shfl_xor(xr[r], 32, kWave);
      }
      // lane g = 16 * grp + col takes head g: row tile grp
#pragma unroll
      for (int r = 0; r < RTQ; ++r)
        if (grp == r) x = xr[r];
    }
    route_select_w(a, t, lane, wq[i], red[ql][lane], x, n_tail);
  }
}

template <int D, int RTQ>
hipError_t launch_rtq(const RouteArgs& a, bool prefill, hipStream_t st) {
  if (prefill && !a.fused) {
    // one query per wave: 155 registers at d = 128, three workgroups per CU (two
    // queries per wave share more staging but leave two)
    constexpr int QPW = 1;
    hipLaunchKernelGGL((route_prefill_tiled_kernel<D, RTQ, QPW>), dim3((unsigned)((a.T + 4 * QPW - 1) / (4 * QPW))),
                       dim3(256), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((route_decode_kernel<D, RTQ>), dim3(a.nchunk, (unsigned)a.T), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nchunk == 1 || a.fused) return e;
  hipLaunchKernelGGL((route_final_kernel<D>), dim3((unsigned)a.T), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_route_d(const RouteArgs& a, bool prefill, hipStream_t st) {
  switch ((a.H + 15) / 16) {
    case 1: return launch_rtq<D, 1>(a, prefill, st);
    case 2: return launch_rtq<D, 2>(a, prefill, st);
    case 3: return launch_rtq<D, 3>(a, prefill, st);
    default: return launch_rtq<D, 4>(a, prefill, st);
  }
}

}  // namespace

bool route_is_prefill(int64_t T, int64_t nseq) { return T >= 64 && T >= 8 * nseq; }

// Chunking of the pooled blocks in decode: 64 blocks per wave-set step; enough
// chunks to give the chip about 256 workgroups. Prefill needs no partials.
size_t route_partial_floats(int64_t T, int H, int64_t Lmax, int B, int* nchunk, int* chunk_blocks) {
  const int64_t mmax = Lmax / B;
  int64_t cb = 64;
  while (cb < mmax && ((mmax + cb - 1) / cb) * T > 256) cb *= 2;
  const int64_t nc = mmax < 1 ? 1 : (mmax + cb - 1) / cb;
  *nchunk = (int)nc;
  *chunk_blocks = (int)cb;
  return nc > 1 ? (size_t)T * (size_t)nc * (size_t)H : 0;
}

hipError_t launch_route(const RouteArgs& a, int d, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool prefill = route_is_prefill(a.T, a.nseq);
  switch (d) {
    case 32: return launch_route_d<32>(a, prefill, st);
    case 64: return launch_route_d<64>(a, prefill, st);
    case 128: return launch_route_d<128>(a, prefill, st);
    case 256: return launch_route_d<256>(a, prefill, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace misa
