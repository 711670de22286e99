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
// Work split: route_partial_kernel (grid = block chunks x queries) accumulates
// sum_j max(q_g . Kbar_j, 0) for every head over its chunk of pooled blocks (one
// lane per (head, block) pair, q_g held in registers, pooled-key rows read
// through the cache). With one chunk per query (prefill) the same workgroup then
// finalises; otherwise route_final_kernel sums the chunk partials in chunk order
// (deterministic), adds the partial-block term and selects the heads.
#include "misa_common.hpp"
#include "misa_internal.hpp"

namespace misa {
namespace {

__device__ __forceinline__ void query_prefix(const RouteArgs& a, int64_t t, int& seq, int& p) {
  seq = a.q_seq[t];
  p = a.q_len[t];
  if (seq < 0 || seq >= a.nseq) {
    seq = -1;
    p = 0;
  }
  p = p < 0 ? 0 : (p > a.Lmax ? (int)a.Lmax : p);
}

// Sum of the keys of the partial last block, per dimension, into LDS (threads < D).
template <int D>
__device__ __forceinline__ void tail_sum(const RouteArgs& a, int seq, int start, int n_tail, float* stail) {
  const int tid = threadIdx.x;
  if (tid < D) {
    float s = 0.f;
    if (n_tail > 0) {
      const uint16_t* kp = a.k + ((int64_t)seq * a.Lmax + start) * D + tid;
      for (int i = 0; i < n_tail; ++i) s += __uint_as_float((uint32_t)kp[(int64_t)i * D] << 16);
    }
    stail[tid] = s;
  }
}

// Rank heads by rho (ties: lower id) and write the routed set; runs in wave 0,
// lane g < H holds head g's complete-block aggregate A and partial-block dot x.
__device__ __forceinline__ void route_select(const RouteArgs& a, int64_t t, int lane, float A, float x,
                                             int n_tail) {
  const bool active = lane < a.H;
  const float w = active ? a.w[t * a.H + lane] : 0.f;
  float rho, r;
  if (n_tail > 0) {
    const float xt = fmaxf(x, 0.f);
    rho = w * ((float)n_tail * A + xt);
    r = w * (A + xt / (float)n_tail);
  } else {
    rho = w * A;
    r = rho;
  }
  rho += 0.f;   // -0 -> +0
  r += 0.f;
  int rank = 0;
  for (int j = 0; j < a.H; ++j) {
    const float o = __shfl(rho, j, kWave);
    rank += (o > rho || (o == rho && j < lane)) ? 1 : 0;
  }
  const bool sel = active && rank < a.h;
  const uint64_t m = __ballot(sel);
  if (sel) {
    const int pos = __popcll(m & ((1ull << lane) - 1ull));
    a.heads[t * a.h + pos] = lane;
  }
  if (active && a.router_key) a.router_key[t * a.H + lane] = r;
}

template <int D, int HP>
__global__ __launch_bounds__(256) void route_partial_kernel(RouteArgs a) {
  constexpr int BPW = 64 / HP;     // blocks per wave step
  constexpr bool PACK = D > 128;   // keep q as packed bf16 pairs when fp32 would not fit
  __shared__ float red[4][64];
  __shared__ float stail[D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane % HP, bs = lane / HP;
  const int64_t t = blockIdx.y;
  const int c = blockIdx.x;
  int seq, p;
  query_prefix(a, t, seq, p);
  const int nfull = p / a.B;
  const int64_t nblk = a.Lmax / a.B;

  constexpr int NQ = PACK ? D / 2 : D;
  float qf[PACK ? 1 : D];
  uint32_t qp[PACK ? D / 2 : 1];
  {
    const bool hv = g < a.H && seq >= 0;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.q + (t * a.H + (hv ? g : 0)) * D);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hv) v = src[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (PACK) {
          qp[4 * i + e] = v[e];
        } else {
          qf[8 * i + 2 * e] = bf16_lo(v[e]);
          qf[8 * i + 2 * e + 1] = bf16_hi(v[e]);
        }
      }
    }
  }
  (void)NQ;
  auto qv = [&](int i) -> float {
    if constexpr (PACK) return (i & 1) ? bf16_hi(qp[i >> 1]) : bf16_lo(qp[i >> 1]);
    else return qf[i];
  };

  float acc = 0.f;
  const int j0 = c * a.chunk_blocks, j1 = min(j0 + a.chunk_blocks, nfull);
  for (int j = j0 + wave * BPW + bs; j < j1; j += 4 * BPW) {
    const floatx4* kb = reinterpret_cast<const floatx4*>(a.kbar + ((int64_t)seq * nblk + j) * D);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const floatx4 v = kb[i];
      dot = fmaf(qv(4 * i), v[0], dot);
      dot = fmaf(qv(4 * i + 1), v[1], dot);
      dot = fmaf(qv(4 * i + 2), v[2], dot);
      dot = fmaf(qv(4 * i + 3), v[3], dot);
    }
    acc += fmaxf(dot, 0.f);
  }
#pragma unroll
  for (int off = HP; off < 64; off <<= 1) acc += __shfl_xor(acc, off, kWave);
  red[wave][lane] = acc;
  __syncthreads();
  if (a.nchunk > 1) {
    if (threadIdx.x < a.H) {
      const int tid = threadIdx.x;
      a.partial[(t * a.nchunk + c) * a.H + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    }
    return;
  }
  // single chunk: finalise here (q_g is still in wave 0's registers, lane g < H)
  const int n_tail = p - nfull * a.B;
  tail_sum<D>(a, seq, nfull * a.B, n_tail, stail);
  __syncthreads();
  if (wave == 0) {
    const float A = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    float x = 0.f;
    if (n_tail > 0) {
#pragma unroll
      for (int i = 0; i < D; ++i) x = fmaf(qv(i), stail[i], x);
    }
    route_select(a, t, lane, A, x, n_tail);
  }
}

template <int D>
__global__ __launch_bounds__(256) void route_final_kernel(RouteArgs a) {
  __shared__ float stail[D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  int seq, p;
  query_prefix(a, t, seq, p);
  const int nfull = p / a.B;
  const int n_tail = p - nfull * a.B;
  tail_sum<D>(a, seq, nfull * a.B, n_tail, stail);
  __syncthreads();
  if (wave != 0) return;
  float A = 0.f, x = 0.f;
  if (lane < a.H) {
    const float* pp = a.partial + t * a.nchunk * a.H + lane;
    for (int c = 0; c < a.nchunk; ++c) A += pp[(int64_t)c * a.H];
    if (n_tail > 0 && seq >= 0) {
      const uint32_t* qrow = reinterpret_cast<const uint32_t*>(a.q + (t * a.H + lane) * D);
      for (int i = 0; i < D / 2; ++i) {
        const uint32_t v = qrow[i];
        x = fmaf(bf16_lo(v), stail[2 * i], x);
        x = fmaf(bf16_hi(v), stail[2 * i + 1], x);
      }
    }
  }
  route_select(a, t, lane, A, x, n_tail);
}

template <int D>
hipError_t launch_route_d(const RouteArgs& a, hipStream_t st) {
  dim3 grid(a.nchunk, (unsigned)a.T);
  const int hp = a.H <= 8 ? 8 : (a.H <= 16 ? 16 : (a.H <= 32 ? 32 : 64));
  switch (hp) {
    case 8: hipLaunchKernelGGL((route_partial_kernel<D, 8>), grid, dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL((route_partial_kernel<D, 16>), grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((route_partial_kernel<D, 32>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((route_partial_kernel<D, 64>), grid, dim3(256), 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nchunk == 1) return e;
  hipLaunchKernelGGL((route_final_kernel<D>), dim3((unsigned)a.T), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Chunking of the pooled blocks: enough workgroups to cover the chip when
// there are few queries, one chunk per query when there are many.
size_t route_partial_floats(int64_t T, int H, int64_t Lmax, int B, int* nchunk, int* chunk_blocks) {
  const int64_t mmax = (Lmax + B - 1) / B;
  int64_t cb = 16;
  while (cb < mmax && cb * 2048 < mmax * T) cb *= 2;
  if (cb > mmax) cb = mmax < 1 ? 1 : mmax;
  const int64_t nc = (mmax + cb - 1) / cb;
  *nchunk = (int)(nc < 1 ? 1 : nc);
  *chunk_blocks = (int)cb;
  return *nchunk > 1 ? (size_t)T * (size_t)(*nchunk) * (size_t)H : 0;
}

hipError_t launch_route(const RouteArgs& a, int d, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  switch (d) {
    case 32: return launch_route_d<32>(a, st);
    case 64: return launch_route_d<64>(a, st);
    case 128: return launch_route_d<128>(a, st);
    case 256: return launch_route_d<256>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace misa
