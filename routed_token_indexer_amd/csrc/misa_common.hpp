// Shared device helpers of the MISA indexer library (gfx950 / CDNA4).
//
// Only this library uses them; the CPU oracle shares nothing with it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// D = A(16x32) * B(32x16) + C on the matrix cores, bf16 in, fp32 accumulate.
// Lane i supplies A row (i % 16) and B column (i % 16), 8 consecutive k-slots
// starting at 8 * (i / 16); it receives D column (i % 16), rows 4 * (i / 16) + 0..3.
__device__ __forceinline__ floatx4 mfma_16x16x32(const u32x4& a, const u32x4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Set bits of the wave mask m in the lanes below the calling lane (v_mbcnt).
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// max(x, 0) as one integer instruction on the bits: a float with the sign bit
// set (negative, -0) is a negative int and becomes +0, any other is kept as is.
// (A float max or median needs the compiler to quiet a possible signalling NaN
// from the MFMA first: two instructions.) Used by every scoring path so that
// all of them produce the same bits.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Raw buffer view of [p, p + bytes) (gfx9 descriptor word 3). The hardware
// range check drops stores at byte offsets >= bytes and returns 0 for such
// loads, so a ragged tail needs no branch around the access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// 32-bit load at byte offset voff + soff (soff uniform); 0 past the view.
__device__ __forceinline__ uint32_t buffer_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ void buffer_store_f32(float v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)byte_off, 0, 0);
}

// Order-preserving map of a float score onto uint32: a > b  <=>  key(a) > key(b).
// -0.0 and +0.0 map to the same key (scores compare as reals).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Hand-offs between workgroups of one launch. Stores and loads of device
// (agent) scope carry the sc1 bit: a store is written through to the memory
// side, where every XCD's loads with sc1 read it, instead of staying in the
// writer's L2; read-modify-write atomics of agent scope are performed at the
// memory side. A workgroup hands data over by storing it, waiting until its
// stores have completed (wait_stores) and only then counting its arrival with
// an atomic; a workgroup that has seen the count complete reads the data with
// agent-scope loads issued after that observation.
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint32_t atomic_add_coherent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this thread's stores and atomics have completed (the sc1 stores
// above: reached the memory side). The asm's memory clobber also keeps the
// compiler from moving memory operations across it.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The 4096-bin histograms that many workgroups add into with atomics keep bin
// b at word hist_word(b): consecutive bins fall in different 128-byte lines
// (bin b in line b % 128), so the adds of the many workgroups to the few busy
// bins of a row spread over many lines instead of queueing on one or two.
__device__ __forceinline__ int hist_word(int b) { return ((b & 127) << 5) | (b >> 7); }
__device__ __forceinline__ int hist_bin(int word) { return ((word & 31) << 7) | (word >> 5); }

// Visible prefix of query t clamped to [0, Lmax]; -1 for an invalid sequence id.
__device__ __forceinline__ int query_prefix_len(const int32_t* q_seq, const int32_t* q_len, int64_t nseq,
                                                int64_t Lmax, int64_t t) {
  const int seq = q_seq[t];
  if (seq < 0 || seq >= nseq) return -1;
  const int p = q_len[t];
  return p < 0 ? 0 : (p > Lmax ? (int)Lmax : p);
}

}  // namespace misa
