// Device building blocks of token scoring and head selection, shared by the
// scoring kernels and the fused decode pipeline so that every path computes
// bit-identical scores and routed head sets.
#pragma once

#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {

// 16-key column tiles of B fragments: lane (grp, col) holds key col of each tile,
// k-slots 8 * grp .. + 8 of every 32-dim step.
template <int D, int KT>
struct KeyTiles {
  u32x4 b[KT][D / 32];
  bool valid[KT];
};

// key_of(s) -> key row index of position s in [.., c_end), or -1 (an invalid
// column). Every lane loads unconditionally: an invalid column reads row
// `fallback` (which the caller guarantees to exist) and is only marked invalid.
// An MFMA output column depends on its own key column alone, and invalid columns
// are replaced by -inf, so their data never reaches a score. (A per-lane
// conditional load makes the compiler wait for each tile before the next is
// requested, which serializes the prefetch.)
template <int D, int KT, typename KeyOf>
__device__ __forceinline__ void load_key_tiles(const uint16_t* kseq_lane, int base, int c_end, int col, KeyOf key_of,
                                               int fallback, KeyTiles<D, KT>& out) {
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int s = base + kt * 16 + col;
    const int key = s < c_end ? key_of(s) : -1;
    out.valid[kt] = key >= 0;
    const uint16_t* kp = kseq_lane + (int64_t)(key < 0 ? fallback : key) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) out.b[kt][ks] = *reinterpret_cast<const u32x4*>(kp + ks * 32);
  }
}

// 64-key row blocks of the d = 128 decode stream. Lane l loads 16-byte piece
// (l & 15) of rows 4 * i + (l >> 4), i < 16, so every load instruction reads four
// whole 256-byte key rows (non-temporal: each key is read once). Positions past
// c_end and skipped candidates read row `fallback` (which exists); their scores
// are masked when the block is scored.
struct RowBlock128 {
  u32x4 v[16];
};

template <typename KeyOf>
__device__ __forceinline__ void load_row_block128(const uint16_t* kseq, int base, int c_end, int lane, KeyOf key_of,
                                                  int fallback, RowBlock128& rb) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int s = base + 4 * i + (lane >> 4);
    const int key = s < c_end ? key_of(s) : -1;
    const uint16_t* kp = kseq + (int64_t)(key < 0 ? fallback : key) * 128 + (lane & 15) * 8;
    rb.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp));
  }
}

// A staged block in LDS: piece p of block row k at slot k * 16 + (p ^ (k & 15)),
// so that the row-wise writes and the MFMA-layout reads (16 rows, one piece
// each) both spread over all banks.
__device__ __forceinline__ void stage_row_block128(u32x4* s_blk, const RowBlock128& rb, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int k = 4 * i + (lane >> 4);
    s_blk[k * 16 + ((lane & 15) ^ (k & 15))] = rb.v[i];
  }
}

// score_four_tiles on a staged block: the B fragment of tile kt, step ks is
// piece 4 * ks + grp of row 16 * kt + col, the same operands in the same order,
// so the scores are the same bit for bit. valid_bits: bit kt tells whether key
// 16 * kt + col of the block is valid.
template <int RT>
__device__ __forceinline__ float score_four_tiles_staged(const u32x4 (&afrag)[RT][4], const float (&wrow)[RT][4],
                                                         const u32x4* s_blk, int grp, int col, uint32_t valid_bits) {
  float mine = 0.f;
  bool mine_valid = false;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    u32x4 b[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) b[ks] = s_blk[(16 * kt + col) * 16 + ((4 * ks + grp) ^ col)];
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma_16x16x32(afrag[r][ks], b[ks], acc);
      part += wrow[r][0] * relu(acc[0]) + wrow[r][1] * relu(acc[1]) +
              wrow[r][2] * relu(acc[2]) + wrow[r][3] * relu(acc[3]);
    }
    part += __shfl_xor(part, 16, kWave);
    part += __shfl_xor(part, 32, kWave);
    if (grp == kt) {
      mine = part;
      mine_valid = (valid_bits >> kt) & 1u;
    }
  }
  return mine_valid ? mine + 0.f : -INFINITY;
}

// A fragments and row weights of one query: row r*16 + i holds head head_of(row)
// (-1: a zero row with weight 0).
template <int D, int RT, typename HeadOf>
__device__ __forceinline__ void load_query_rows(const uint16_t* q, const float* w, int64_t t, int H, int col, int grp,
                                                HeadOf head_of, u32x4 (&afrag)[RT][D / 32], float (&wrow)[RT][4]) {
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int head = head_of(16 * r + col);
    const uint16_t* qp = q + (t * H + (head < 0 ? 0 : head)) * D + grp * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head >= 0) v = *reinterpret_cast<const u32x4*>(qp + ks * 32);
      afrag[r][ks] = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hd = head_of(16 * r + 4 * grp + j);
      wrow[r][j] = hd < 0 ? 0.f : w[t * H + hd];
    }
  }
}

// Scores of 4 tiles (64 keys): ReLU, head weight and head sum on the MFMA
// accumulators. Lane (grp, col) returns the score of key 16 * grp + col of the
// group and whether that key was valid (invalid keys score -inf).
template <int D, int RT>
__device__ __forceinline__ float score_four_tiles(const u32x4 (&afrag)[RT][D / 32], const float (&wrow)[RT][4],
                                                  const KeyTiles<D, 4>& tiles, int grp) {
  float mine = 0.f;
  bool mine_valid = false;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) acc = mfma_16x16x32(afrag[r][ks], tiles.b[kt][ks], acc);
      part += wrow[r][0] * relu(acc[0]) + wrow[r][1] * relu(acc[1]) +
              wrow[r][2] * relu(acc[2]) + wrow[r][3] * relu(acc[3]);
    }
    part += __shfl_xor(part, 16, kWave);
    part += __shfl_xor(part, 32, kWave);
    if (grp == kt) {
      mine = part;
      mine_valid = tiles.valid[kt];
    }
  }
  return mine_valid ? mine + 0.f : -INFINITY;
}

// Score of one 16-key tile with the A fragments read from an LDS copy of the
// query's rows (row stride ldq bf16; rows beyond the heads are zero) and the row
// weights from LDS. Per key this is exactly the MFMA / epilogue sequence of
// score_four_tiles, so the scores are the same bit for bit; every lane of the
// wave returns the score of key col of the tile (-inf if invalid).
template <int D, int RT>
__device__ __forceinline__ float score_one_tile_lds(const uint16_t* s_q, int ldq, const float* s_w,
                                                    const KeyTiles<D, 1>& tile, int grp, int col) {
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* qa = s_q + (16 * r + col) * ldq + grp * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      acc = mfma_16x16x32(*reinterpret_cast<const u32x4*>(qa + ks * 32), tile.b[0][ks], acc);
    const float* wr = s_w + 16 * r + 4 * grp;
    part += wr[0] * relu(acc[0]) + wr[1] * relu(acc[1]) + wr[2] * relu(acc[2]) +
            wr[3] * relu(acc[3]);
  }
  part += __shfl_xor(part, 16, kWave);
  part += __shfl_xor(part, 32, kWave);
  return tile.valid[0] ? part + 0.f : -INFINITY;
}

// Head ranking of the router (one wave; lane g < H holds head g's complete-block
// aggregate A and partial-block dot x). rho_g = w_g * (n_tail * A_g + max(x_g, 0))
// (n_tail = 0: rho_g = w_g * A_g); ties go to the lower head id. Returns whether
// this lane's head is routed and its position among the routed heads (ascending
// id), and the importance r_g = rho_g / n_tail.
__device__ __forceinline__ bool route_rank(int H, int h, int lane, float w, float A, float x, int n_tail, int& pos,
                                           float& r) {
  const bool active = lane < H;
  float rho;
  if (n_tail > 0) {
    const float xt = relu(x);
    rho = w * ((float)n_tail * A + xt);
    r = w * (A + xt / (float)n_tail);
  } else {
    rho = w * A;
    r = rho;
  }
  rho += 0.f;   // -0 -> +0
  r += 0.f;
  // rank = heads ahead of this one: larger rho, or equal rho and a lower id.
  // As one 64-bit key (order-preserving bits of rho, then 63 - id) that is a
  // single unsigned compare per head; j is uniform, so each head's key bits
  // are read with v_readlane (no LDS round trip), fully unrolled for H = 64
  const uint32_t rb = __float_as_uint(rho);
  const uint32_t kh = (rb & 0x80000000u) ? ~rb : (rb | 0x80000000u);
  const uint64_t mine = ((uint64_t)kh << 32) | (uint32_t)(63 - lane);
  auto ahead = [&](int j) {
    const uint32_t oh = (uint32_t)__builtin_amdgcn_readlane((int)kh, j);
    return (((uint64_t)oh << 32) | (uint32_t)(63 - j)) > mine ? 1 : 0;
  };
  int rank = 0;
  if (H == 64) {
#pragma unroll
    for (int j = 0; j < 64; ++j) rank += ahead(j);
  } else {
    for (int j = 0; j < H; ++j) rank += ahead(j);
  }
  const bool sel = active && rank < h;
  const uint64_t m = __ballot(sel);
  pos = __popcll(m & ((1ull << lane) - 1ull));
  return sel;
}

// Complete-block aggregate of head `lane` from the router's chunk partials,
// summed in chunk order. The first kPartialBatch partials are requested
// together (one memory round trip for the usual chunk counts); the sum is the
// same sequential chunk-order sum whatever the batching.
constexpr int kPartialBatch = 16;

struct PartialBatch {
  float v[kPartialBatch];
};

// Requests the first kPartialBatch partials of head `lane` (clamped, in-bounds
// addresses; entries past nchunk are ignored by finish_partials).
__device__ __forceinline__ void load_partials(const float* partial, int64_t t, int nchunk, int H, int lane,
                                              PartialBatch& pb) {
  const float* pp = partial + t * nchunk * H + (lane < H ? lane : H - 1);
#pragma unroll
  for (int j = 0; j < kPartialBatch; ++j) pb.v[j] = pp[(int64_t)(j < nchunk ? j : 0) * H];
}

__device__ __forceinline__ float finish_partials(const float* partial, int64_t t, int nchunk, int H, int lane,
                                                 const PartialBatch& pb) {
  float A = 0.f;
  if (lane < H) {
#pragma unroll
    for (int j = 0; j < kPartialBatch; ++j)
      if (j < nchunk) A += pb.v[j];
    const float* pp = partial + t * nchunk * H + lane;
    for (int c = kPartialBatch; c < nchunk; ++c) A += pp[(int64_t)c * H];
  }
  return A;
}

__device__ __forceinline__ float sum_partials(const float* partial, int64_t t, int nchunk, int H, int lane) {
  PartialBatch pb;
  load_partials(partial, t, nchunk, H, lane, pb);
  return finish_partials(partial, t, nchunk, H, lane, pb);
}

}  // namespace misa
