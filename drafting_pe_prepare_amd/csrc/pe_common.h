// Device-side helpers shared by the libpe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bfloat16 is stored as its 16-bit pattern (the high half of an IEEE float32).
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
// float32 -> bfloat16, round to nearest, ties to even: gfx950's
// v_cvt_pk_bf16_f32 (one instruction converts a pair).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Storage access for the two element types the library handles.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float cvt(float v) { return v; }
};
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ float cvt(float v) { return bf2f(f2bf(v)); }
};

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%16][8(l/16)..+8]
// and B[8(l/16)..+8][l%16]; it receives C[4(l/16)+i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%32][8(l/32)..+8]
// and B[8(l/32)..+8][l%32]; register i of the result holds
// C[8(i/4) + 4(l/32) + i%4][l%32].
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// Streaming 16-byte load for data read once (weights): non-temporal hint.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
#if defined(PE_W_PLAIN)
  return *reinterpret_cast<const uint4*>(p);
#else
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
#endif
}
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Order-preserving 32-bit image of a float: larger float -> larger unsigned.
__device__ __forceinline__ uint32_t float_order(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Argmax key: value in the high word, (0xFFFFFFFF - index) in the low word, so
// the largest key holds the largest value and, among equal values, the lowest index.
__device__ __forceinline__ uint64_t argmax_key(float v, int idx) {
  return (uint64_t(float_order(v)) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(idx));
}
__device__ __forceinline__ int argmax_key_index(uint64_t k) {
  return int(0xFFFFFFFFu - uint32_t(k & 0xFFFFFFFFull));
}

// Maximum of v over the 16 lanes of its row (lanes 16q .. 16q+15), in every
// lane of the row: four DPP row permutes (swap pairs, swap pairs of pairs,
// mirror each half-row, mirror the row), each combined with a max.  DPP moves
// are VALU operands: no LDS round trip and no wait.  Every lane of the row
// must be active.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false)));  // row_mirror
  return v;
}
// Largest argmax key over the 16 lanes of a row: the largest value word, then
// the largest index word among the lanes that hold that value (the 64-bit
// maximum, as two 32-bit row maxima).
__device__ __forceinline__ uint64_t row16_max_key(uint64_t k) {
  const uint32_t hi = row16_max_u32(uint32_t(k >> 32));
  const uint32_t lo = row16_max_u32(uint32_t(k >> 32) == hi ? uint32_t(k) : 0u);
  return (uint64_t(hi) << 32) | lo;
}

// Philox4x32-10 ("Parallel random numbers: as easy as 1, 2, 3", Salmon,
// Moraes, Dror, Shaw, SC 2011): the four output words for counter
// (c0, c1, 0, stream) under the 64-bit key `seed`.  Ten rounds of two 32x32
// multiplies (high and low halves), XOR with the other words and the round
// key, and a word permutation; the key advances by the two Weyl constants.
struct Words4 { uint32_t w[4]; };
__device__ __forceinline__ Words4 philox4(uint32_t c0, uint32_t c1, uint32_t stream, uint64_t seed) {
  uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = stream;
  uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t hi0 = __umulhi(0xD2511F53u, x0), lo0 = 0xD2511F53u * x0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, x2), lo1 = 0xCD9E8D57u * x2;
    const uint32_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
    x0 = y0; x1 = lo1; x2 = y2; x3 = lo0;
  }
  return Words4{{x0, x1, x2, x3}};
}
// Random-number streams of stochastic drafting and verification.  Per-token
// noise: token v of a row takes word v % 4 of block (v / 4, row).
enum RngStream : uint32_t { RNG_DRAFT = 0, RNG_ACCEPT = 1, RNG_RESIDUAL = 2 };
// U in (0, 1) from an output word: (x / 512 + 1/2) / 2^23, exact in fp32.
__device__ __forceinline__ float word_uniform(uint32_t x) {
  return (float(x >> 9) + 0.5f) * 1.1920928955078125e-7f;
}
// Gumbel noise -log(-log U); -log U as -log1p(U - 1) (U - 1 is exact).
__device__ __forceinline__ float gumbel_noise(float u) { return -logf(-log1pf(u - 1.0f)); }

// s_waitcnt vmcnt(N) only: at most N vector-memory operations of this wave in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// lgkmcnt(0) only: every LDS read issued so far has returned
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// One LDS-DMA instruction: every lane moves 16 bytes from `src` to LDS byte
// lds + 16 lane (lds wave-uniform).  Written as inline asm on purpose: the
// compiler tracks the LDS writes of its own global_load_lds and, unable to
// tell the stage being read from the stages in flight, waits for every DMA
// before each LDS read (vmcnt(0) at the top of each k-tile, which drains the
// ring).  Hidden from it, the DMAs are ordered by the calling kernel's own
// vmcnt waits (and barriers) only, and the "memory" clobber keeps the
// compiler from moving LDS reads across a DMA.  The asm writes no register
// (the data goes to LDS), so no output register can be reused while the load
// is in flight; it sets m0 and says so.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return uint32_t(uintptr_t((__attribute__((address_space(3))) const unsigned char*)p));
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sums of split-K partials: acc[v] = sum over k = 0 .. KS-1 of the float4 at
// p + k * stride + off[v], added in split order (k ascending, from zero), so
// the sums do not depend on how the loads are batched.  The loads of up to
// eight splits (all NV vectors of each) are issued before the first add: one
// memory round trip per eight splits, where a load-add loop waits once per
// split.
template <int NV>
__device__ __forceinline__ void sum_splits(const float* p, long long stride, int KS, const long long (&off)[NV],
                                           float4 (&acc)[NV]) {
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < KS; k0 += 8) {
    float4 a[8][NV];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      if (k0 + kk < KS)
#pragma unroll
        for (int v = 0; v < NV; ++v) a[kk][v] = *reinterpret_cast<const float4*>(p + (k0 + kk) * stride + off[v]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      if (k0 + kk < KS)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc[v].x += a[kk][v].x;
          acc[v].y += a[kk][v].y;
          acc[v].z += a[kk][v].z;
          acc[v].w += a[kk][v].w;
        }
  }
}

}  // namespace pe
