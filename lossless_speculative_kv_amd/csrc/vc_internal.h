// Internal helpers shared by the gfx950 kernels of libvc (not part of the ABI).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vc.h"

namespace vc {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------- MFMA ----
// v_mfma_f32_16x16x32_{f16,bf16}. Lane l holds A row (l % 16) and B column
// (l % 16), each with 8 contraction slots selected by l / 16 (the same slot
// mapping for A and B); the result lane l holds column l % 16, rows
// 4 * (l / 16) + r, r = 0..3.
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16) return mfma_bf16(a, b, c);
  else return mfma_f16(a, b, c);
}

// ------------------------------------------------------- conversions ----
// Round-to-nearest-even packs (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 v;
  v.x = (_Float16)lo;
  v.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
template <bool BF16>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  if constexpr (BF16) return pack_bf16(lo, hi);
  else return pack_f16(lo, hi);
}
// Reinterpret a 32-bit word as two fp16 values and back. The word is taken by
// value on purpose: this hipcc (clang 22) reads element 0 when
// __builtin_bit_cast is applied directly to an ext-vector subscript such as
// v[r] inside an unrolled loop, so vector elements must pass through a
// scalar first.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).x; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).y; }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
}
// fp32 -> bf16 bits, nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------ cross-lane ops ----
// DPP quad permutations: xor 1 ([1,0,3,2]) and xor 2 ([2,3,0,1]).
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
// Sum / max over the four lanes {l, l^16, l^32, l^48}; every lane gets the
// bitwise-identical result (the swap pairs operands in lane-independent order).
__device__ __forceinline__ float sum_q(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_q(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Rotations within a row of 16 lanes (DPP row_ror:4 / row_ror:8).
__device__ __forceinline__ float dpp_ror4(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_ror8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
// Max over the 16 lanes of a row; every lane of the row gets the same value.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_xor1(x));
  x = fmaxf(x, dpp_xor2(x));
  x = fmaxf(x, dpp_ror4(x));
  return fmaxf(x, dpp_ror8(x));
}
// Sum over the 16 lanes of a row (the order of the last two additions
// depends on the lane's quad, so lanes may differ in the last bit).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_xor1(x);
  x += dpp_xor2(x);
  x += dpp_ror4(x);
  return x + dpp_ror8(x);
}
// Sum over the NG adjacent lanes of a column group (NG in {1, 2, 4}).
template <int NG>
__device__ __forceinline__ float sum_group(float x) {
  if constexpr (NG >= 2) x = x + dpp_xor1(x);
  if constexpr (NG >= 4) x = x + dpp_xor2(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// --------------------------------------------------------- wave pacing ----
// Waves with equal static shares that share a SIMD do not progress equally:
// the SIMD's issue arbiter prefers the older wave at equal priority, so the
// younger ones finish long after. Each wave publishes the step it has
// reached in an LDS array of ints at lds_base (8 for up to eight waves, else
// 16; zeroed before the first call) and runs at priority 1 while it is
// behind the workgroup's leading wave, else at 0. Only the timing changes, never the work a wave
// does. The exchange is one asm block that waits for its own LDS accesses
// (as plain LDS accesses the compiler would order them after every pending
// direct-to-LDS load), and the priority is chosen inside asm (branches the
// compiler sees would split a pipelined loop body).
template <int NW>
__device__ __forceinline__ void pace_waves(uint32_t lds_base, int wave, int step) {
  static_assert(NW >= 1 && NW <= 16, "sixteen progress slots");
  u32x4 p0, p1, p2, p3;
  if constexpr (NW <= 8) {
    asm volatile(
        "ds_write_b32 %2, %3\n\t"
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p0), "=&v"(p1)
        : "v"(lds_base + 4 * wave), "v"(step), "v"(lds_base));
  } else {
    asm volatile(
        "ds_write_b32 %4, %5\n\t"
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %6 offset:16\n\t"
        "ds_read_b128 %2, %6 offset:32\n\t"
        "ds_read_b128 %3, %6 offset:48\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p0), "=&v"(p1), "=&v"(p2), "=&v"(p3)
        : "v"(lds_base + 4 * wave), "v"(step), "v"(lds_base));
  }
  int lead = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const u32x4& q = w < 4 ? p0 : w < 8 ? p1 : w < 12 ? p2 : p3;
    lead = max(lead, (int)q[w & 3]);
  }
  const int lag = __builtin_amdgcn_readfirstlane(lead - step);
  asm volatile(
      "s_cmp_gt_i32 %0, 0\n\t"
      "s_cbranch_scc0 1f\n\t"
      "s_setprio 1\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "s_setprio 0\n"
      "2:"
      :
      : "s"(lag)
      : "scc");
}
// LDS byte address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)p;
}

// ------------------------------------------------------------ loads ----
// Cache policy of the direct-to-LDS loads that stream the KV cache (records,
// rows, tiles): non-temporal (the gfx950 `nt` bit), so the lines are not kept
// in L2 or the memory-side cache. Measured on MI355X: plain reads of 2 GiB
// stream at 6.2 TB/s, non-temporal ones at 6.8 TB/s, and the draft KIVI
// kernel went from 47.6 to 42.4 us. Plain global loads get the same policy
// through __builtin_nontemporal_load. The vocabulary weights keep the default
// policy: read again at every draft step, part of them stays in the
// memory-side cache (non-temporal weight loads made the draft-step product
// 10% slower).
constexpr int kStreamPolicy = 2;

template <typename T>
__device__ __forceinline__ T ldg(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

// ---------------------------------------------------- host-side errors ----
void set_error(const char* fmt, ...);
vc_status fail(vc_status code, const char* fmt, ...);
vc_status check_launch(const char* what);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Events the caller asked the next call on this thread to record (see
// vc_time_next_call); take_timing() hands them over once and clears them.
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
  int scope = VC_TIME_CALL;
};
Timing take_timing();

// Launch, with the dispatch itself recording start / stop events when given.
template <typename F, typename... A>
void launch_ev(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, hipEvent_t start, hipEvent_t stop,
               A... args) {
  if (start != nullptr || stop != nullptr) hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, start, stop, 0u, args...);
  else hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

}  // namespace vc
