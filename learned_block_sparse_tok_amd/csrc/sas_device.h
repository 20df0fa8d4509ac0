// Device-side helpers shared by the libsas kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

constexpr int kHeadDim = 128;
constexpr int kGateDim = 128;
constexpr int kBlock = 64;
constexpr int kMaxGroup = 16;
#define SAS_MAX_BLOCKS_DEV 16384
constexpr float kLog2e = 1.4426950408889634f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}
// The same packing by the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, b16x2));
}

// 16-byte global load (the address must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of
// the row receives the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)); // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)); // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)); // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)); // row_ror:1
  return x;
}

// A lane's value from another lane of its 16-lane row (DPP): kRor4 / kRor8
// rotate the row by 4 / 8 lanes, kXor2 / kXor1 swap lanes j and j^2 / j^1.
constexpr int kRor4 = 0x124, kRor8 = 0x128, kXor2 = 0x4E, kXor1 = 0xB1;
template <int kCtrl>
__device__ __forceinline__ float row_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// One step of a transposing row sum over n value pairs (v[c], v[c + n]): a
// lane keeps the half its bit picks and adds the same half from its partner.
template <int kCtrl, int n>
__device__ __forceinline__ void row16_keep_half(bool bit, float *v) {
#pragma unroll
  for (int c = 0; c < n; ++c) {
    const float keep = bit ? v[c + n] : v[c], send = bit ? v[c] : v[c + n];
    v[c] = keep + row_dpp<kCtrl>(send);
  }
}

// Transposing sum over the 16 lanes of a DPP row: lane o gets the sum over
// the row's lanes of their value for row index o.  The caller stores row r at
// v[row16_slot(r)]; the first step may pair lanes by a rotation because every
// lane still holds all 16 rows, the next three use exact partners (lane bits
// 3, 1, 0).  15 exchanges instead of 16 separate 4-step row sums.
__device__ __forceinline__ int row16_slot(int r) { return ((r >> 2) & 1) * 8 + ((r >> 3) & 1) * 4 + (r & 3); }
__device__ __forceinline__ float row16_transpose_sum(float (&v)[16]) {
  const int o = threadIdx.x & 15;
  row16_keep_half<kRor4, 8>(o & 4, v);  // row bit 2
  row16_keep_half<kRor8, 4>(o & 8, v);  // row bit 3
  row16_keep_half<kXor2, 2>(o & 2, v);  // row bit 1
  row16_keep_half<kXor1, 1>(o & 1, v);  // row bit 0
  return v[0];
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// One global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// i's bytes land at LDS byte lds + 16 i (lds is wave-uniform).  Written out
// (rather than through the builtin) so that the compiler, which does not
// track these LDS writes, inserts no vmcnt(0) before every later LDS read;
// the instruction sequence is the one the compiler emits for the builtin (M0
// write, one wait state).  The compiler does not count these loads either:
// completion is awaited explicitly with wait_vm, and every compiler-visible
// load must be complete before the first copy is issued (a later wait the
// compiler computes for such a load would not account for the copies).
// The asm clobbers M0, which the compiler reserves: that is sound only while
// no compiler-generated code in the kernel keeps a value in M0, and while no
// other vector-memory instruction falls between the first copy and the
// drain.  tests/test_prefill_asm.py checks both on the built assembly, so
// the compiler's warning about the reserved register is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with only the vector-memory counter: at most n loads outstanding
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// LDS byte address of a __shared__ object
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)p;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads, so gathers issued earlier stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Order-preserving map fp32 -> uint32 for a descending Top-K: NaN ranks as
// -inf and -0 as +0, so equal keys mean equal scores.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) s = -__builtin_inff();
  if (s == 0.0f) s = 0.0f;
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// cos and sin of pos * inv_freq for RoPE.  The angle can reach ~1e5 rad, so
// it is formed and reduced to [-pi, pi] in fp64 (error ~1e-11 rad); the
// reduced angle's sine and cosine are then taken in fp32.
__device__ __forceinline__ void rope_cos_sin(double pos, double inv_freq, float &c, float &s) {
  const double kTwoPi = 6.283185307179586;
  const double ang = pos * inv_freq;
  const double r = ang - rint(ang * (1.0 / kTwoPi)) * kTwoPi;
  sincosf((float)r, &s, &c);
}

}  // namespace sas
