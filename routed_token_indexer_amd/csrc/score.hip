// Token scoring of the MISA / DSA indexer on the gfx950 matrix cores.
//
// MISA pages (MISA abstract; gist.science "Methodologie: MISA", sparse token
// scoring): only the routed heads score every prefix token. The score of token s
// for query t with head set R is
//     S[t][s] = sum_{g in R} w[t][g] * max(q[t][g] . k[s], 0).
// The dense DSA indexer ("Probleemstelling") is the same with R = all H heads,
// and the MISA† fine stage ("Hiërarchische Variant") applies it to a candidate
// list instead of the whole prefix.
//
// The query's gathered head rows are MFMA A-fragments held in registers; keys
// stream from HBM as B-fragments, 16 keys per 16x16x32 MFMA column tile; ReLU,
// the head weight and the head sum are applied to the accumulators in
// registers and one fp32 score per (query, key) is stored. Lane i of a wave
// supplies A row / B column (i % 16) and k-slots 8 * (i / 16) .. + 8 of each
// 32-dim step, so one load instruction reads 64 contiguous bytes of each of 16
// keys.
//   decode kernel  one query per workgroup and a chunk of its keys (decode
//                  batches and candidate lists); can also build the level-1
//                  histogram of the split top-k for the scores it writes.
//   wide kernel    a tile of consecutive queries of one sequence per workgroup
//                  (causal prefill), so each key tile loaded serves the whole
//                  query tile.
#include <hip/hip_ext.h>

#include "misa_common.hpp"
#include "misa_internal.hpp"
#include "misa_score_dev.hpp"

namespace misa {

namespace {

// Row length of query t (tokens it can see, or valid candidates) and its key
// sequence; seq = -1 marks an absent or invalid query (it produces nothing).
__device__ __forceinline__ void query_info(const ScoreArgs& a, int64_t t, int& seq, int& n) {
  seq = -1;
  n = 0;
  if (t >= a.T) return;
  const int sq = a.q_seq[t];
  if (sq < 0 || sq >= a.nseq) return;
  seq = sq;
  const int p = a.q_len[t];
  n = p < 0 ? 0 : (p > a.Lmax ? (int)a.Lmax : p);
}

// prefill: grid (key chunks, query tiles). A workgroup is 4 waves; wave w owns
// the 16 * RT gathered head rows of QW consecutive queries, held as MFMA A
// fragments for the whole launch. The workgroup's chunk of keys streams through
// LDS in blocks of 64 keys, double buffered: one global load per key per
// workgroup, and every wave multiplies each block into all of its rows.
// Queries of several sequences in one tile are handled by one pass over the
// keys per distinct sequence (rows of other sequences store nothing).
template <int D, int NHP, int RT, int KB>
__global__ __launch_bounds__(256, 2) void score_prefill_kernel(ScoreArgs a) {
  constexpr int KS = D / 32;                  // 32-wide k-steps
  constexpr int QW = (16 * RT) / NHP;         // queries per wave
  constexpr int QT = 4 * QW;                  // queries per workgroup
  // Row layout. Grouped (up to 16 rows per query, when a wave's tiles split evenly):
  // tile r = M4 * i + f holds queries 4i .. 4i + 3 of the wave, row rho being head
  // slot 4f + rho % 4 of query 4i + rho / 4, so the MFMA output rows 4g .. 4g + 3 of
  // lane group g are 4 head slots of one query and its full head sum is a sum over
  // f inside the lane (no cross-lane step; every lane stores). Otherwise rows run
  // query-major (row R of the wave is slot R % NHP of query R / NHP) and the head
  // sum crosses lane groups.
  constexpr int M4 = NHP / 4;
  constexpr bool GROUPED = NHP <= 16 && RT % M4 == 0;
  constexpr int NOUT = GROUPED ? RT / M4 : (NHP <= 8 ? RT : QW);   // output slots of one lane
  // KB: keys per LDS block
  // LDS key rows: d = 128 rows are unpadded with 16-byte piece p of row k at slot
  // p ^ (k & 15) (row-wise writes and MFMA-layout reads both spread over all
  // banks); other widths use a 16-byte pad per row
  constexpr bool SWZ = D == 128;
  constexpr int LDK = SWZ ? D : D + 8;        // LDS row stride (bf16)
  constexpr int PPR = D / 8;                  // 16-byte pieces per key row
  constexpr int LPT = KB * PPR / 256;         // pieces each thread moves per block
  static_assert(QW >= 1 && (16 * RT) % NHP == 0 && LPT >= 1, "tiling");
  constexpr int NROW = 4 * 16 * RT;           // head rows of the workgroup
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][KB * LDK];
  __shared__ __attribute__((aligned(16))) float s_w[NROW];   // row weights (0 for padding rows)
  __shared__ int s_head[NROW];                                // row head ids (-1: padding row)
  __shared__ int s_seq[QT], s_n[QT];
  __shared__ int s_pseq[QT], s_pn[QT], s_np;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  // grid (tiles, chunks): consecutive workgroups take consecutive tiles of one
  // chunk, so the round-robin spread over the XCDs mixes tiles of every length on
  // every XCD (with the chunk as the fast index, one XCD would get every chunk-0
  // workgroup and another only the few long tiles' last chunks)
  const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;   // longest prefixes first
  const int64_t t0 = tile * QT;
  const int chunk_id = blockIdx.y;

  // query (within the workgroup) and head slot of workgroup row R
  auto row_query = [&](int R) {
    const int wv = R / (16 * RT), Rw = R % (16 * RT);
    return wv * QW + (GROUPED ? 4 * ((Rw / 16) / M4) + (Rw % 16) / 4 : Rw / NHP);
  };
  auto row_slot = [&](int R) {
    const int Rw = R % (16 * RT);
    return GROUPED ? 4 * ((Rw / 16) % M4) + (Rw % 4) : Rw % NHP;
  };

  // ---- 1. query rows' sequences and lengths, raw head ids (all requested at once)
  __shared__ int s_nmax, s_smin, s_smax;
  if (tid == 0) {
    s_nmax = 0;
    s_smin = 0x7fffffff;
    s_smax = -1;
  }
  constexpr int RPT = (NROW + 255) / 256;
  int graw[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int R = tid + 256 * i;
    const int64_t t = t0 + row_query(R);
    const int hs = row_slot(R);
    const int64_t tc = t < a.T ? t : 0;
    const int hc = hs < a.hh ? hs : 0;
    const int32_t* hp = a.heads ? a.heads + tc * a.hh + hc : a.q_seq + tc;
    const int g = *hp;
    graw[i] = (R < NROW && t < a.T && hs < a.hh) ? (a.heads ? g : hs) : -1;
  }
  int my_seq = -1, my_n = 0;
  if (tid < QT) query_info(a, t0 + tid, my_seq, my_n);
  __syncthreads();
  if (tid < QT) {
    s_seq[tid] = my_seq;
    s_n[tid] = my_n;
    if (my_seq >= 0) {
      atomicMax(&s_nmax, my_n);
      atomicMin(&s_smin, my_seq);
      atomicMax(&s_smax, my_seq);
    }
  }
  __syncthreads();
  // a chunk past every prefix of the tile has nothing to do
  const int c_begin = chunk_id * a.chunk;
  if (c_begin >= s_nmax) return;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int R = tid + 256 * i;
    if (R < NROW) {
      const int g = graw[i];
      s_head[R] = (s_seq[row_query(R)] >= 0 && g >= 0 && g < a.H) ? g : -1;
    }
  }
  if (tid == 0) {
    if (s_smin == s_smax) {   // one sequence: one pass over its keys
      s_pseq[0] = s_smin;
      s_pn[0] = s_nmax;
      s_np = 1;
    } else {                  // several: one pass per distinct sequence, each up to its longest prefix
      int np = 0;
      for (int i = 0; i < QT; ++i) {
        const int sq = s_seq[i];
        if (sq < 0) continue;
        int j = 0;
        while (j < np && s_pseq[j] != sq) ++j;
        if (j == np) {
          s_pseq[np] = sq;
          s_pn[np] = 0;
          ++np;
        }
        s_pn[j] = max(s_pn[j], s_n[i]);
      }
      s_np = np;
    }
  }
  __syncthreads();

  // ---- 2. A fragments of this wave's rows and the row weights (clamped, unconditional loads)
  u32x4 afrag[RT][KS];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int R = wave * 16 * RT + 16 * r + col;
    const int head = s_head[R];
    const uint16_t* qp = a.q + ((head < 0 ? 0 : (t0 + row_query(R)) * a.H + head) * D) + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + ks * 32);
      afrag[r][ks] = head < 0 ? u32x4{0u, 0u, 0u, 0u} : v;
    }
  }
  float wv[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int R = tid + 256 * i;
    const int head = R < NROW ? s_head[R] : -1;
    const float v = a.w[head < 0 ? 0 : (t0 + row_query(R)) * a.H + head];
    wv[i] = head < 0 ? 0.f : v;
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    if (tid + 256 * i < NROW) s_w[tid + 256 * i] = wv[i];
  // the lane's output slot i is query out_q(i) of the workgroup (rows 4 * grp .. + 3 of
  // each tile after the head sum); writer lanes hold each sum once
  auto out_q = [&](int i) {
    return wave * QW + (GROUPED ? 4 * i + grp : (NHP == 4 ? 4 * i + grp : (NHP == 8 ? 2 * i + (grp >> 1) : i)));
  };
  const bool writer = GROUPED || NHP == 4 ? true : (NHP == 8 ? (grp & 1) == 0 : grp == 0);
  // weights of the lane's accumulator rows (4 * grp .. + 3 of each tile), kept in registers
  __syncthreads();
  floatx4 wreg[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) wreg[r] = *reinterpret_cast<const floatx4*>(&s_w[wave * 16 * RT + 16 * r + 4 * grp]);
  // scores of the workgroup's query rows through a range-checked buffer view: a
  // store outside a query's visible prefix (or chunk) goes to an offset past the
  // view and is dropped, so the store needs no branch
  const int64_t nrow_out = a.T - t0 < QT ? a.T - t0 : QT;
  const auto oview = buffer_view(a.out + t0 * a.out_stride, (uint32_t)(nrow_out * a.out_stride * 4));
  const int np = s_np;

  for (int pi = 0; pi < np; ++pi) {
    const int sq = s_pseq[pi];
    if (c_begin >= s_pn[pi]) continue;
    const int c_end = min(c_begin + a.chunk, s_pn[pi]);
    const uint16_t* kseq = a.k + (int64_t)sq * a.Lmax * D;
    const int nblk = (c_end - c_begin + KB - 1) / KB;
    // per output slot: keys below lim are this lane's to store in this pass, at byte
    // offset voff + 4 * key in the view
    int lim[NOUT];
    uint32_t voff[NOUT];
    int lim_min = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NOUT; ++i) {
      const int q = out_q(i);
      lim[i] = (writer && s_seq[q] == sq) ? min(s_n[q], c_end) : 0;
      lim_min = min(lim_min, lim[i]);
      voff[i] = (uint32_t)((int64_t)q * a.out_stride * 4);
    }
    // blocks below every slot's limit store without masks (grouped rows only: there
    // every lane is a writer)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off, kWave));
    // staging of one key block: thread pieces tid + 256 * i (row, 16-byte column)
    auto load_block = [&](int b, u32x4 (&v)[LPT]) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int pc = tid + 256 * i;
        int s = c_begin + b * KB + pc / PPR;
        s = s < a.Lmax ? s : (int)a.Lmax - 1;
        v[i] = *reinterpret_cast<const u32x4*>(kseq + (int64_t)s * D + (pc % PPR) * 8);
      }
    };
    auto store_block = [&](uint16_t* buf, const u32x4 (&v)[LPT]) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int pc = tid + 256 * i;
        const int row = pc / PPR, piece = pc % PPR;
        *reinterpret_cast<u32x4*>(buf + row * LDK + (SWZ ? piece ^ (row & 15) : piece) * 8) = v[i];
      }
    };
    // Blocks in flight in registers while block b is multiplied: two where the
    // registers allow (one block of MFMA work is shorter than a key load's latency
    // under load), else one.
    constexpr int PF = NHP <= 16 && RT <= 4 ? 2 : 1;
    u32x4 nv[PF][LPT];
    {
      u32x4 v[LPT];
      load_block(0, v);
#pragma unroll
      for (int j = 0; j < PF; ++j) load_block(1 + j < nblk ? 1 + j : 0, nv[(1 + j) % PF]);
      store_block(s_k[0], v);
    }
    __syncthreads();
    // one block: cur holds block b + 1 (the register sets are named statically, the
    // loop below alternates them; an index computed at run time would move them
    // through indexed register access and wait for every load)
    auto block_step = [&](int b, u32x4 (&cur)[LPT]) {
      const uint16_t* buf = s_k[b & 1];
      const int base = c_begin + b * KB;
      const bool unmasked = base + KB <= lim_min;
      // Tiles are software-pipelined: the MFMAs of tile kt + 1 go out next to the
      // epilogue (ReLU, weights, head sum, stores) of tile kt, which does not depend
      // on them, so neither waits on the other's latency; within a tile the k-step
      // is outer, so consecutive MFMAs feed different accumulators.
      auto mma = [&](int kt, floatx4 (&acc)[RT]) {
        u32x4 bv[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          bv[ks] = *reinterpret_cast<const u32x4*>(buf + (kt * 16 + col) * LDK +
                                                   (SWZ ? (4 * ks + grp) ^ col : 4 * ks + grp) * 8);
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int r = 0; r < RT; ++r) acc[r] = mfma_16x16x32(afrag[r][ks], bv[ks], acc[r]);
      };
      auto epi = [&](int kt, const floatx4 (&acc)[RT]) {
        float part[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r)
          part[r] = wreg[r][0] * relu(acc[r][0]) + wreg[r][1] * relu(acc[r][1]) + wreg[r][2] * relu(acc[r][2]) +
                    wreg[r][3] * relu(acc[r][3]);
        // head sum per query: within the lane (4 rows), across lane groups, across tiles
        float val[NOUT];
        if constexpr (GROUPED) {
#pragma unroll
          for (int i = 0; i < NOUT; ++i) {
            float v = part[M4 * i];
#pragma unroll
            for (int f = 1; f < M4; ++f) v += part[M4 * i + f];
            val[i] = v;
          }
        } else if constexpr (NHP == 4) {
#pragma unroll
          for (int r = 0; r < RT; ++r) val[r] = part[r];
        } else if constexpr (NHP == 8) {
#pragma unroll
          for (int r = 0; r < RT; ++r) val[r] = part[r] + __shfl_xor(part[r], 16, kWave);
        } else {
          constexpr int m = NHP / 16;
#pragma unroll
          for (int q = 0; q < QW; ++q) {
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < m; ++i) v += part[q * m + i];
            v += __shfl_xor(v, 16, kWave);
            v += __shfl_xor(v, 32, kWave);
            val[q] = v;
          }
        }
        const int s_out = base + kt * 16 + col;
        if (GROUPED && unmasked) {
#pragma unroll
          for (int i = 0; i < NOUT; ++i) buffer_store_f32(val[i] + 0.f, oview, voff[i] + (uint32_t)s_out * 4u);
        } else {
#pragma unroll
          for (int i = 0; i < NOUT; ++i)
            buffer_store_f32(val[i] + 0.f, oview, s_out < lim[i] ? voff[i] + (uint32_t)s_out * 4u : 0xfffffff0u);
        }
      };
      floatx4 acc0[RT], acc1[RT];
      mma(0, acc0);
#pragma unroll
      for (int kt = 0; kt < KB / 16; kt += 2) {
        if (kt + 1 < KB / 16) mma(kt + 1, acc1);
        epi(kt, acc0);
        if (kt + 2 < KB / 16) mma(kt + 2, acc0);
        if (kt + 1 < KB / 16) epi(kt + 1, acc1);
      }
      store_block(s_k[(b + 1) & 1], cur);
      load_block(b + 1 + PF < nblk ? b + 1 + PF : 0, cur);   // block b + 1 + PF takes the freed registers
      __syncthreads();
    };
    int b = 0;
    if constexpr (PF == 2) {
      for (; b + 1 < nblk; b += 2) {
        block_step(b, nv[1]);
        block_step(b + 1, nv[0]);
      }
      if (b < nblk) block_step(b, nv[1]);
    } else {
      for (; b < nblk; ++b) block_step(b, nv[0]);
    }
  }
}

// decode: grid (key chunks, T); one query per workgroup, its rows padded to RT tiles.
// Startup is ordered for a memory system that the key stream is about to
// saturate: everything that does not depend on the query's sequence (its H
// query rows, which are staged in LDS, its weights, the routed head ids or the
// router's chunk partials) is requested first, then the first key tiles, and
// only then are the routed heads selected and the A fragments read from LDS.
// Every iteration prefetches the next iteration's keys before computing the
// current one. With a.partial set, the workgroup selects the query's routed
// heads itself from the router's chunk partials (the fused decode pipeline).
template <int D, int RT, bool GATHER, bool HIST>
__global__ __launch_bounds__(256) void score_decode_kernel(ScoreArgs a) {
  constexpr int KT = 4;           // 16-key tiles per wave iteration: 64 keys, one per lane at the end
  constexpr int LDQ = D + 8;      // LDS row stride of the staged query rows (bf16)
  constexpr int QV = D / 8;       // 16-byte pieces per query row
  constexpr int QPT = (64 * QV + 255) / 256;   // staging pieces per thread (H <= 64)
  // d = 128 over contiguous keys streams row blocks through a swizzled LDS stage
  // (16 KiB per wave), which also holds the staged query rows before the stream
  // starts (gathered candidate rows keep the direct MFMA-layout loads)
  constexpr bool kStage = D == 128 && !GATHER;
  constexpr int kQBytes = 64 * LDQ * 2;
  constexpr int kBufBytes = kStage ? (4 * 1024 * 16 > kQBytes ? 4 * 1024 * 16 : kQBytes) : kQBytes;
  // level-1 histogram: two 16-bit bin counts per word (a chunk has at most 16384 keys)
  __shared__ uint32_t lh[HIST ? 2048 : 1];
  __shared__ __align__(16) uint8_t s_buf[kBufBytes];
  uint16_t* const s_q = reinterpret_cast<uint16_t*>(s_buf);
  __shared__ float s_w[64];
  __shared__ int s_heads[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t t = blockIdx.y;
  const bool fused_route = a.partial != nullptr;

  // 1. requests that do not depend on the sequence
  u32x4 qv[QPT];
  const int nqv = a.H * QV;
  const uint16_t* qsrc = a.q + t * a.H * D;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = threadIdx.x + 256 * j;
    qv[j] = *reinterpret_cast<const u32x4*>(qsrc + (int64_t)(i < nqv ? i : 0) * 8);
  }
  // Issued by every lane from clamped, in-bounds addresses (a conditional load
  // would make the compiler wait for it before the key requests go out); the
  // pointer selects only depend on kernel arguments.
  const int gl = lane < a.H ? lane : a.H - 1;
  const float wg = a.w[t * a.H + gl];
  const float x = (fused_route ? a.xtail : a.w)[t * a.H + gl];
  PartialBatch pb;
  load_partials(fused_route ? a.partial : a.w, t, fused_route ? a.nchunk_r : 1, a.H, lane, pb);
  const int32_t* hp = a.heads ? a.heads + t * a.hh + (lane < a.hh ? lane : a.hh - 1) : a.q_seq + t;
  const int hv = *hp;
  const int head_in = a.heads ? hv : lane;

  int seq = a.q_seq[t];
  int p = a.q_len[t];
  if (seq < 0 || seq >= a.nseq) {
    seq = -1;
    p = 0;
  }
  p = p < 0 ? 0 : (p > a.Lmax ? (int)a.Lmax : p);
  const int n = GATHER ? (seq < 0 ? 0 : a.kc) : p;
  const int c_begin = blockIdx.x * a.chunk;
  if (c_begin >= n && !(fused_route && blockIdx.x == 0)) return;
  const int c_end = min(c_begin + a.chunk, n);
  const uint16_t* kseq = a.k + (int64_t)(seq < 0 ? 0 : seq) * a.Lmax * D + grp * 8;
  const int32_t* crow = GATHER ? a.cand + t * a.kc : nullptr;
  auto key_of = [&](int s) -> int {
    if constexpr (GATHER) {
      const int id = crow[s];
      return (id >= 0 && id < p) ? id : -1;
    } else {
      return s;
    }
  };
  // c_begin < max_len <= Lmax, so row c_begin of the (clamped) sequence exists
  const int fallback = GATHER ? 0 : c_begin;

  // 2. consume the small loads before any key request of this wave goes out
  // (workgroups dispatched a little later would otherwise find their small
  // loads queued behind tens of MiB of key requests): stage the query rows and
  // weights, and (wave 0) sum the router's partials.
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < nqv) *reinterpret_cast<u32x4*>(s_q + (i / QV) * LDQ + (i % QV) * 8) = qv[j];
  }
  float A = 0.f;
  if (wave == 0) {
    if (lane < a.H) s_w[lane] = wg;
    if (fused_route) A = finish_partials(a.partial, t, a.nchunk_r, a.H, lane, pb);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. the first two iterations' key tiles (two in flight per wave)
  constexpr int kStep = 4 * 16 * KT;   // keys per workgroup iteration
  const int base0 = c_begin + wave * 16 * KT;
  const uint16_t* kseq_rows = a.k + (int64_t)(seq < 0 ? 0 : seq) * a.Lmax * D;
  KeyTiles<D, kStage ? 1 : KT> ta, tb;
  RowBlock128 ra, rb;
  if constexpr (kStage) {
    load_row_block128(kseq_rows, base0, c_end, lane, key_of, fallback, ra);
    load_row_block128(kseq_rows, base0 + kStep, c_end, lane, key_of, fallback, rb);
  } else {
    load_key_tiles<D, KT>(kseq, base0, c_end, col, key_of, fallback, ta);
    load_key_tiles<D, KT>(kseq, base0 + kStep, c_end, col, key_of, fallback, tb);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 4. select the heads while the keys stream in
  if (wave == 0) {
    if (fused_route) {
      const int n_tail = p - (p / a.B) * a.B;
      int pos;
      float r;
      const bool sel = route_rank(a.H, a.hh, lane, wg, A, x, n_tail, pos, r);
      if (sel) s_heads[pos] = lane;
      if (blockIdx.x == 0) {
        if (sel && a.heads_out) a.heads_out[t * a.hh + pos] = lane;
        if (lane < a.H && a.router_key) a.router_key[t * a.H + lane] = r;
      }
    } else if (lane < a.hh) {
      s_heads[lane] = (head_in >= 0 && head_in < a.H) ? head_in : -1;
    }
  }
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < 2048; i += 256) lh[i] = 0;
  }
  __syncthreads();
  if (c_begin >= n) return;

  u32x4 afrag[RT][D / 32];
  float wrow[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = 16 * r + col;
    const int head = row < a.hh ? s_heads[row] : -1;
    const uint16_t* qa = s_q + (head < 0 ? 0 : head) * LDQ + grp * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qa + ks * 32);
      afrag[r][ks] = head < 0 ? u32x4{0u, 0u, 0u, 0u} : v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row2 = 16 * r + 4 * grp + j;
      const int hd = row2 < a.hh ? s_heads[row2] : -1;
      wrow[r][j] = hd < 0 ? 0.f : s_w[hd];
    }
  }

  // Scores of this chunk go through a buffer view of [c_begin, c_end), so the
  // stores of lanes past c_end are dropped by the range check instead of being
  // branched around: the loop body stays straight-line and the compiler can
  // count the loads in flight exactly.
  const auto ov = buffer_view(a.out + t * a.out_stride + c_begin, (uint32_t)(c_end - c_begin) * 4u);
  auto put = [&](float v, int b) {
    const int s = b + lane;
    buffer_store_f32(v, ov, (uint32_t)(s - c_begin) * 4u);
    if constexpr (HIST) {
      const uint32_t bin = score_key(v) >> 20;
      atomicAdd(&lh[bin >> 1], (s < c_end ? 1u : 0u) << (16 * (bin & 1u)));
    }
  };
  auto emit = [&](const KeyTiles<D, KT>& tiles, int b) { put(score_four_tiles<D, RT>(afrag, wrow, tiles, grp), b); };
  // Two register sets alternate, so no in-flight tile is ever copied (a copy
  // would wait for its load). The iteration count is uniform over the
  // workgroup; each wave masks its own tail through c_end. Inside the loop the
  // loads are unconditional (an odd count prefetches one spare iteration of
  // in-bounds rows).
  const int nit = (c_end - c_begin + kStep - 1) / kStep;
  int it = 0;
  if constexpr (kStage) {
    // a block goes to this wave's LDS stage, the registers take the block after
    // next, and the block is scored from LDS (LDS operations of a wave run in
    // order, so the stage is not rewritten before its reads)
    __syncthreads();   // every wave has read the staged query rows
    u32x4* const s_blk = reinterpret_cast<u32x4*>(s_buf) + wave * 1024;
    auto valid_bits = [&](int b) {
      uint32_t bits = 0;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int s = b + 16 * kt + col;
        bits |= (s < c_end && key_of(s) >= 0) ? 1u << kt : 0u;
      }
      return bits;
    };
    auto score_staged = [&](int b) {
      put(score_four_tiles_staged<RT>(afrag, wrow, s_blk, grp, col, valid_bits(b)), b);
    };
    for (; it + 2 < nit; it += 2) {
      const int b = base0 + it * kStep;
      stage_row_block128(s_blk, ra, lane);
      load_row_block128(kseq_rows, b + 2 * kStep, c_end, lane, key_of, fallback, ra);
      score_staged(b);
      stage_row_block128(s_blk, rb, lane);
      load_row_block128(kseq_rows, b + 3 * kStep, c_end, lane, key_of, fallback, rb);
      score_staged(b + kStep);
    }
    if (it < nit) {
      stage_row_block128(s_blk, ra, lane);
      score_staged(base0 + it * kStep);
    }
    if (it + 1 < nit) {
      stage_row_block128(s_blk, rb, lane);
      score_staged(base0 + (it + 1) * kStep);
    }
  } else {
    for (; it + 2 < nit; it += 2) {
      const int b = base0 + it * kStep;
      emit(ta, b);
      load_key_tiles<D, KT>(kseq, b + 2 * kStep, c_end, col, key_of, fallback, ta);
      emit(tb, b + kStep);
      load_key_tiles<D, KT>(kseq, b + 3 * kStep, c_end, col, key_of, fallback, tb);
    }
    if (it < nit) emit(ta, base0 + it * kStep);
    if (it + 1 < nit) emit(tb, base0 + (it + 1) * kStep);
  }
  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + t * 4096;
    for (int i = threadIdx.x; i < 2048; i += 256) {
      const uint32_t v = lh[i];
      if (v & 0xffffu) atomicAdd(&gh[hist_word(2 * i)], v & 0xffffu);
      if (v >> 16) atomicAdd(&gh[hist_word(2 * i + 1)], v >> 16);
    }
  }
}

// Launch, stamping the timing events at the kernel's own start and end when
// the scoring kernels are being timed.
template <typename K, typename... Args>
hipError_t launch_timed(int kid, K kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  hipEvent_t e0, e1;
  if (timing_take(kid, st, e0, e1))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  return hipGetLastError();
}

template <int D, int RT, bool GATHER>
hipError_t launch_decode(ScoreArgs a, int64_t max_len, hipStream_t st) {
  if (a.chunk <= 0) {
    // about 512 workgroups (two per CU), at least 512 keys (two iterations) each: a
    // workgroup of one iteration spends most of its time before its first keys arrive
    // (gathered candidate rows: at least 256 keys, their loads are not streamed)
    int64_t c = GATHER ? 256 : 512;
    while (c < 16384 && c * 512 < max_len * a.T) c *= 2;
    a.chunk = (int)c;
  }
  dim3 grid((unsigned)((max_len + a.chunk - 1) / a.chunk), (unsigned)a.T);
  const int kid = GATHER ? KID_GATHER_SCORE : KID_SCORE;
  if (a.hist) return launch_timed(kid, score_decode_kernel<D, RT, GATHER, true>, grid, dim3(256), st, a);
  return launch_timed(kid, score_decode_kernel<D, RT, GATHER, false>, grid, dim3(256), st, a);
}

template <int D>
hipError_t launch_decode_d(const ScoreArgs& a, bool gather, int64_t max_len, hipStream_t st) {
  const int rt = (a.hh + 15) / 16;
  if (gather) {
    switch (rt) {
      case 1: return launch_decode<D, 1, true>(a, max_len, st);
      case 2: return launch_decode<D, 2, true>(a, max_len, st);
      case 3: return launch_decode<D, 3, true>(a, max_len, st);
      default: return launch_decode<D, 4, true>(a, max_len, st);
    }
  }
  switch (rt) {
    case 1: return launch_decode<D, 1, false>(a, max_len, st);
    case 2: return launch_decode<D, 2, false>(a, max_len, st);
    case 3: return launch_decode<D, 3, false>(a, max_len, st);
    default: return launch_decode<D, 4, false>(a, max_len, st);
  }
}

template <int D, int NHP, int RT, int KB>
hipError_t launch_prefill_cfg(ScoreArgs a, int64_t max_len, hipStream_t st, bool few = false) {
  constexpr int QT = 4 * (16 * RT) / NHP;
  if ((uint64_t)QT * (uint64_t)a.out_stride * 4u >= (1ull << 32) - 16) return hipErrorInvalidValue;   // view offsets
  if (a.chunk <= 0 && few) {
    // few tiles over long prefixes: key chunks for about 512 workgroups, at least
    // 256 keys (four blocks) each
    const int64_t ntiles = (a.T + QT - 1) / QT;
    int64_t c = 256;
    while (c < 2048 && ntiles * ((max_len + c - 1) / c) > 512) c *= 2;
    a.chunk = (int)c;
  }
  if (a.chunk <= 0) a.chunk = 2048;
  const dim3 grid((unsigned)((a.T + QT - 1) / QT), (unsigned)((max_len + a.chunk - 1) / a.chunk));
  return launch_timed(KID_SCORE, score_prefill_kernel<D, NHP, RT, KB>, grid, dim3(256), st, a);
}

// Row tiles per wave and keys per LDS block, sized so that the A fragments
// (RT * D / 8 registers), the accumulators and row weights (8 * RT), one key
// tile's B fragments and the staged next block fit 256 registers (two waves per
// SIMD): up to d = 64 eight tiles (six for 48 rows per query); at d = 128 six
// for 8 rows per query, otherwise four (three for 48, six being too many); at
// d = 256 two (3 for 48, 4 for 64 rows) with 32-key blocks.
template <int D>
hipError_t launch_prefill(const ScoreArgs& a, int nhp, int64_t max_len, hipStream_t st) {
  constexpr bool W = D == 256;
  constexpr bool M = D == 128;
  constexpr int KB = W ? 32 : 64;
  switch (nhp) {
    case 4: return launch_prefill_cfg<D, 4, W ? 2 : (M ? 4 : 8), KB>(a, max_len, st);
    case 8: return launch_prefill_cfg<D, 8, W ? 2 : (M ? 6 : 8), KB>(a, max_len, st);
    case 16: return launch_prefill_cfg<D, 16, W ? 2 : (M ? 4 : 8), KB>(a, max_len, st);
    case 32: return launch_prefill_cfg<D, 32, W ? 2 : (M ? 4 : 8), KB>(a, max_len, st);
    case 48: return launch_prefill_cfg<D, 48, W ? 3 : (M ? 3 : 6), KB>(a, max_len, st);
    case 64: return launch_prefill_cfg<D, 64, W ? 4 : (M ? 4 : 8), KB>(a, max_len, st);
  }
  return hipErrorInvalidValue;
}

// Few queries per sequence (a decode step that scores several consecutive
// positions of each sequence): one query per wave, four per workgroup, so that a
// tile usually covers a single sequence, which then streams its keys once for
// all of its queries. Up to 16 routed heads take one row tile (padding rows
// cost matrix-core time only, which this memory-bound case has to spare).
template <int D>
hipError_t launch_prefill_few(const ScoreArgs& a, int nhp, int64_t max_len, hipStream_t st) {
  constexpr int KB = D == 256 ? 32 : 64;
  switch (nhp) {
    case 4:
    case 8:
    case 16: return launch_prefill_cfg<D, 16, 1, KB>(a, max_len, st, true);
    case 32: return launch_prefill_cfg<D, 32, 2, KB>(a, max_len, st, true);
    case 48: return launch_prefill_cfg<D, 48, 3, KB>(a, max_len, st, true);
    case 64: return launch_prefill_cfg<D, 64, 4, KB>(a, max_len, st, true);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int score_rows_per_query(int hh) {
  if (hh <= 4) return 4;
  if (hh <= 8) return 8;
  return 16 * ((hh + 15) / 16);
}

hipError_t launch_score(const ScoreArgs& a, int d, bool gather, bool wide, int64_t max_len, hipStream_t st,
                        bool few) {
  if (a.T == 0) return hipSuccess;
  if (!gather && few) {
    const int nhp = score_rows_per_query(a.hh);
    switch (d) {
      case 32: return launch_prefill_few<32>(a, nhp, max_len, st);
      case 64: return launch_prefill_few<64>(a, nhp, max_len, st);
      case 128: return launch_prefill_few<128>(a, nhp, max_len, st);
      case 256: return launch_prefill_few<256>(a, nhp, max_len, st);
    }
    return hipErrorInvalidValue;
  }
  if (gather || !wide) {
    switch (d) {
      case 32: return launch_decode_d<32>(a, gather, max_len, st);
      case 64: return launch_decode_d<64>(a, gather, max_len, st);
      case 128: return launch_decode_d<128>(a, gather, max_len, st);
      case 256: return launch_decode_d<256>(a, gather, max_len, st);
    }
    return hipErrorInvalidValue;
  }
  const int nhp = score_rows_per_query(a.hh);
  switch (d) {
    case 32: return launch_prefill<32>(a, nhp, max_len, st);
    case 64: return launch_prefill<64>(a, nhp, max_len, st);
    case 128: return launch_prefill<128>(a, nhp, max_len, st);
    case 256: return launch_prefill<256>(a, nhp, max_len, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace misa
