// Internal helpers shared by the HIP kernels of libdllm (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 values are carried as raw uint16_t bit patterns.
struct bf16 { uint16_t bits; };

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even, NaN stays NaN: gfx950's v_cvt_pk_bf16_f32 (the
// compiler pairs neighbouring conversions into one instruction).  Checked on the device
// against the integer form (add 0x7fff plus the lowest kept bit, truncate) over every
// fp32 bit pattern: identical for all non-NaN inputs.
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Element access for the two storage types (float, or bf16 bits in uint16_t).
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: A lane l holds row l%16, k = 8(l/16)..+8; B lane l holds
// column l%16, the same k; C lane l holds column l%16, rows 4(l/16)..+4.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Wave-wide reductions (64 lanes) with a fixed combination order.
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Lane permutes on the DPP path (a VALU operand modifier, no LDS crossbar).  Controls:
// 0xB1 = quad_perm [1,0,3,2] (lane ^ 1), 0x4E = quad_perm [2,3,0,1] (lane ^ 2),
// 0x141 = row_half_mirror (lane 7 - i within 8), 0x140 = row_mirror (15 - i within 16).
// All four are full permutations inside a 16-lane row, so every source lane is valid.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Reduce within aligned groups of G = 2, 4, 8 or 16 consecutive lanes: afterwards every
// lane of a group holds op over the group.  op must be commutative (max, min, +), so
// partner lanes compute bit-identical values.
template <int G, typename V, typename Op>
__device__ __forceinline__ V group_reduce(V v, Op op) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group size");
  v = op(v, dpp<0xB1>(v));
  if constexpr (G >= 4) v = op(v, dpp<0x4E>(v));
  if constexpr (G >= 8) v = op(v, dpp<0x141>(v));
  if constexpr (G >= 16) v = op(v, dpp<0x140>(v));
  return v;
}

// Combine each lane with its partner lane ^ 16 or lane ^ 32 (gfx950 v_permlane16_swap /
// v_permlane32_swap of a register with itself).  The swap returns, in every lane, the
// pair's two values in lane order, so a commutative op gives both partners the same
// bits, as an xor shuffle would, without the LDS crossbar.
template <typename Op>
__device__ __forceinline__ float xor16_combine(float x, Op op) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ float xor32_combine(float x, Op op) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fmax_op(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float add_op(float a, float b) { return a + b; }

// Whole-wave reduction: 16-lane rows on the DPP path, then the four row results read
// into scalar registers and combined in a fixed order ((r0, r1), (r2, r3)).  Every lane
// receives the same value.
__device__ __forceinline__ float wave_max_dpp(float v) {
  auto mx = [](float a, float b) { return fmaxf(a, b); };
  v = group_reduce<16>(v, mx);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = group_reduce<16>(v, [](float a, float b) { return a + b; });
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ int wave_min_dpp(int v) {
  v = group_reduce<16>(v, [](int a, int b) { return min(a, b); });
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Cross-workgroup hand-off of split partial results without cache-wide maintenance.
// Partials are written with device-coherent stores (relaxed agent-scope atomics: the
// store carries sc1 and is acknowledged once it is visible to every XCD) and read back
// with device-coherent loads.  A device-scope release/acquire fence would instead write
// back and invalidate the whole L2 of the issuing XCD on every arrival.
// The same stores also carry outputs that only the next kernel reads, from other XCDs:
// written through, they leave no dirty lines for the end-of-kernel write-back (used
// where that measured faster, see the callers).
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// four bf16 values as one 8-byte device-coherent store (p 8-byte aligned)
__device__ __forceinline__ void st_dev(uint16_t* p, u16x4 v) {
  uint64_t bits;
  __builtin_memcpy(&bits, &v, sizeof bits);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// "Last block" detection for fixed-order split reductions.  Every workgroup of a group
// calls it once after publishing its partials with st_dev; exactly one (the last to
// arrive) gets true and may then read all partials with ld_dev.  The wait makes each
// thread's coherent stores complete before the barrier, hence before the arrival
// counter moves.  The counter is reset by the last workgroup, so it is clean for the
// next launch.
__device__ __forceinline__ bool arrive_last(int* counter, int expected, int* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = (prev == expected - 1);
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag != 0;
}

}  // namespace dllm
