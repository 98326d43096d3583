// Device-side helpers shared by the gfx950 attention kernels: vector types,
// matrix-core wrappers, cross-lane reductions and type conversions.
//
// Matrix-core operand layouts used throughout (wave64, verified on gfx950):
//   32x32x16 (bf16/f16): lane l holds A[l%32][8*(l/32)+j] and B[8*(l/32)+j][l%32]
//                        (j = 0..7); result register i of lane l is
//                        C[8*(i/4) + 4*(l/32) + i%4][l%32].
//   32x32x2 (f32):       lane l holds A[l%32][l/32] and B[l/32][l%32]; same C.
//   16x16x32 (bf16/f16): lane l holds A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16];
//                        result register i of lane l is C[4*(l/16)+i][l%16].
//   16x16x16 (bf16/f16): lane l holds A[l%16][4*(l/16)+j], B[4*(l/16)+j][l%16]
//                        (j = 0..3); same C as 16x16x32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the two halves of a wave (lane l and lane l^32). Both
// lanes of a pair combine the operands in the same order, so they end up
// with bitwise identical values.
// max of two floats that are never signalling NaNs (no quieting step).
__device__ __forceinline__ float max_quiet(float a, float b) {
  float r;
  __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_quiet(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Reductions between 16-lane rows r and r^1 (lane l and lane l^16).
__device__ __forceinline__ float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS reads at a 32-bit LDS byte address. Writing the address as a per-lane
// base plus a constant lets the compiler fold the constant into the
// instruction's offset field.
template <typename T>
__device__ __forceinline__ T lds_read16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(static_cast<uintptr_t>(addr));
}
// Transposed read of a 4x4 block of 16-bit values (ds_read_b64_tr_b16).
__device__ __forceinline__ i16x4 lds_read_tr8(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4*>(static_cast<uintptr_t>(addr)));
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's 16 bytes land at lds + 16 * i; `lds` must be wave-uniform. POLICY
// is the instruction's cache-policy operand (2 = non-temporal). The explicit
// address-space casts keep the host compilation pass well-formed.
template <int POLICY>
__device__ __forceinline__ void load_lds16_policy(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0,
                                   POLICY);
}

// The same copy issued from inline assembly, for kernels that track these
// loads themselves (explicit vmcnt waits and barriers). The compiler does not
// see the LDS write, so it adds no conservative wait for all outstanding
// vector-memory loads in front of later LDS reads, and the caller must order
// every read of `lds` (an LDS byte address) after the copy with s_waitcnt
// vmcnt + a barrier. M0 (the LDS destination register of the copy) is saved
// and restored around it.
__device__ __forceinline__ void load_lds16_async(const void* g, uint32_t lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(a)
      : "memory");
}

// The same copy from a wave-uniform base address plus a per-lane 32-bit byte
// offset (the instruction's scalar-base form), to the LDS byte address
// `lds` (wave-uniform). Stepping a tile then changes only scalar registers.
__device__ __forceinline__ void load_lds16_sbase(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// Buffer resource over `bytes` bytes from `base` for untyped loads (no
// stride, no swizzle, 32-bit data format): a load whose offset lies at or
// beyond `bytes` touches no memory and returns zeros. All fields are
// wave-uniform. `base` is a device address below 2^48 (the API rejects
// others), so its upper word fits the 16-bit address field and leaves the
// stride and swizzle fields zero.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

// Direct buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 with
// lds): lane i reads the resource at byte offset voff (zeros when out of
// range) and its 16 bytes land at LDS byte address lds + 16 * i (`lds`
// wave-uniform). As for load_lds16_async, the caller orders later reads of
// that LDS range with s_waitcnt vmcnt + a barrier; the compiler sets M0 (the
// LDS destination register) from the operand.
__device__ __forceinline__ void load_lds16_buf(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "{m0}"(l)
                   : "memory");
}

// Element types. Storage is handled as raw 16-bit words; arithmetic types
// are the compiler's __bf16 / _Float16.
struct BF16 {
  using scalar = __bf16;
  using vec8 = bf16x8;
  static __device__ __forceinline__ f32x16 mma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16k16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // Round-to-nearest-even of 4 floats, as the raw 16-bit words of an operand.
  static __device__ __forceinline__ i16x4 pack4(float a, float b, float c, float d) {
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
    const v4 r = {static_cast<__bf16>(a), static_cast<__bf16>(b), static_cast<__bf16>(c),
                  static_cast<__bf16>(d)};
    return __builtin_bit_cast(i16x4, r);
  }
  static __device__ __forceinline__ float to_f32(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
  }
  // acc + v[2e] + v[2e+1] (one dot2 against (1, 1); the products are exact).
  static __device__ __forceinline__ float sum2(vec8 v, int e, float acc) {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    const v2 p = {v[2 * e], v[2 * e + 1]};
    const v2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
};
struct F16 {
  using scalar = _Float16;
  using vec8 = f16x8;
  static __device__ __forceinline__ f32x16 mma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16k16(i16x4 a, i16x4 b, f32x4 c) {
    typedef _Float16 v4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4, a),
                                                  __builtin_bit_cast(v4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ i16x4 pack4(float a, float b, float c, float d) {
    typedef _Float16 v4 __attribute__((ext_vector_type(4)));
    const v4 r = {static_cast<_Float16>(a), static_cast<_Float16>(b), static_cast<_Float16>(c),
                  static_cast<_Float16>(d)};
    return __builtin_bit_cast(i16x4, r);
  }
  static __device__ __forceinline__ float to_f32(uint16_t u) {
    return static_cast<float>(__builtin_bit_cast(_Float16, u));
  }
  static __device__ __forceinline__ float sum2(vec8 v, int e, float acc) {
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    const v2 p = {v[2 * e], v[2 * e + 1]};
    const v2 one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
    return __builtin_amdgcn_fdot2(p, one, acc, false);
  }
};

// Round-to-nearest-even conversion of 8 floats into one matrix-core operand.
template <typename E>
__device__ __forceinline__ typename E::vec8 pack8(float a0, float a1, float a2, float a3,
                                                  float a4, float a5, float a6, float a7) {
  typename E::vec8 r;
  r[0] = static_cast<typename E::scalar>(a0);
  r[1] = static_cast<typename E::scalar>(a1);
  r[2] = static_cast<typename E::scalar>(a2);
  r[3] = static_cast<typename E::scalar>(a3);
  r[4] = static_cast<typename E::scalar>(a4);
  r[5] = static_cast<typename E::scalar>(a5);
  r[6] = static_cast<typename E::scalar>(a6);
  r[7] = static_cast<typename E::scalar>(a7);
  return r;
}

// The value is rounded to fp32 before any narrowing store: without this the
// compiler may fuse the last multiply into a mixed-precision op that rounds
// once, straight to fp16, and the fp16 output would no longer be exactly the
// round-to-nearest-even of the fp32 output of the same computation.
__device__ __forceinline__ float as_f32(float x) {
  __asm__("" : "+v"(x));
  return x;
}

// Output stores of 4 consecutive floats in the output element type.
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  v4 r;
  r[0] = static_cast<__bf16>(as_f32(a)); r[1] = static_cast<__bf16>(as_f32(b));
  r[2] = static_cast<__bf16>(as_f32(c)); r[3] = static_cast<__bf16>(as_f32(d));
  *reinterpret_cast<v4*>(p) = r;
}
__device__ __forceinline__ void store4(_Float16* p, float a, float b, float c, float d) {
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  v4 r;
  r[0] = static_cast<_Float16>(as_f32(a)); r[1] = static_cast<_Float16>(as_f32(b));
  r[2] = static_cast<_Float16>(as_f32(c)); r[3] = static_cast<_Float16>(as_f32(d));
  *reinterpret_cast<v4*>(p) = r;
}
__device__ __forceinline__ void store1(float* p, float a) { *p = a; }
__device__ __forceinline__ void store1(__bf16* p, float a) { *p = static_cast<__bf16>(as_f32(a)); }
__device__ __forceinline__ void store1(_Float16* p, float a) {
  *p = static_cast<_Float16>(as_f32(a));
}

// Workgroup id remap so that consecutive logical ids run on the same XCD.
// The dispatcher hands workgroup p to XCD p % kXcds; here logical id L is
// given to physical id p such that each XCD receives one contiguous range of
// logical ids (their K/V then share that XCD's L2).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int p, int total) {
  const int q = total / kXcds, r = total % kXcds;
  const int x = p % kXcds, k = p / kXcds;
  const int base = (x < r) ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return base + k;
}

// Workgroup id -> (group, unit) for work made of `groups` independent groups
// (e.g. (sequence, KV head) pairs) of `units` workgroups each. XCD x (which
// the dispatcher feeds the physical ids x, x + kXcds, ...) takes the groups
// x, x + kXcds, x + 2 kXcds, ... one after the other, all units of a group in
// order: a group's units share that XCD's L2, and groups of very different
// cost (long and short sequences of a ragged batch) spread over all XCDs.
// The grid has kXcds * ceil(groups / kXcds) * units workgroups; ids past the
// last group return group = -1.
__device__ __forceinline__ void xcd_group_unit(int p, int groups, int units, int* group,
                                               int* unit) {
  const int x = p % kXcds, k = p / kXcds;
  const int g = x + kXcds * (k / units);
  *unit = k % units;
  *group = g < groups ? g : -1;
}

}  // namespace fa
