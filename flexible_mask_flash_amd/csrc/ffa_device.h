// Device helpers shared by the forward and backward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "ffa_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

#define FFA_LDS __attribute__((address_space(3)))
// plan records are read-only for the kernels: reading them through the constant
// address space lets the compiler use scalar loads
#define FFA_CONST __attribute__((address_space(4)))

namespace ffa {
namespace dev {

// buffer resource word 3 for raw (untyped) dword loads on gfx9-class parts
constexpr int kBufferFlags = 0x00020000;
// s_waitcnt immediates (gfx9 encoding: vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// LDS reads are issued through inline asm with an explicit address register and
// a compile-time offset; the results are waited for with lds_wait<N>() (at most N
// LDS reads of this wave still outstanding) and pinned behind that wait with
// fence().  Going around the compiler here keeps it from draining the in-flight
// K/V prefetch (it cannot prove the reads and the DMA writes are disjoint) and
// lets several reads be in flight while MFMAs run.
template <int OFF>
__device__ __forceinline__ f32x4_t lds_read_b128(uint32_t addr) {
  f32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4 of
// the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12 of the group.
// Pointing lane j at row (key0 + j/4), columns (c0 + 4*(j%4) .. +3) therefore
// hands lane i the column c0 + i of rows key0 .. key0+3.
template <int OFF>
__device__ __forceinline__ s16x4_t lds_read_tr16(uint32_t addr) {
  s16x4_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

template <int N>
__device__ __forceinline__ void lds_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
template <typename T>
__device__ __forceinline__ void fence(T& x) {
  asm volatile("" : "+v"(x));
}

// Workgroup barrier without a memory fence (the waits are explicit), but a
// compiler barrier for memory operations on both sides.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float partner_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(f32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

// Element type of q, k, v, out and the gradients: bfloat16 or IEEE half.  The
// kernels are templated on it; the two differ only in the MFMA opcode and in the
// conversions (and, in the forward, in how large a probability may grow before
// the exact rescale: fp16 tops out at 65504).
template <typename T>
struct ElemT;
template <>
struct ElemT<__bf16> {
  typedef bf16x8_t v8;
  typedef bf16x4_t v4;
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static constexpr float kMaxP = 18446744073709551616.0f;  // 2^64
};
template <>
struct ElemT<_Float16> {
  typedef f16x8_t v8;
  typedef f16x4_t v4;
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static constexpr float kMaxP = 32768.0f;  // 2^15
};
template <typename T>
__device__ __forceinline__ typename ElemT<T>::v8 as_v8(f32x4_t x) {
  return __builtin_bit_cast(typename ElemT<T>::v8, x);
}
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Tile iterator over an item's runs (wave-uniform): the tile's first key and the
// mask parameters of its run.
struct TileIt {
  int ri, ti, k0, nt, nf, khi, eb, nl, lb;
  __device__ __forceinline__ int kstart() const { return k0 + ti * ffa::kBlockN; }
  // tiles [nl, nl + nf) of a run are visible to every row; the others need the mask
  __device__ __forceinline__ bool edge() const { return (unsigned)(ti - nl) >= (unsigned)nf; }
};
__device__ __forceinline__ void tile_first(TileIt& t, const FFA_CONST int32_t* rp) {
  t.ri = 0; t.ti = 0;
  t.k0 = rp[0]; t.nt = rp[1]; t.nf = rp[2]; t.khi = rp[3]; t.eb = rp[4]; t.nl = rp[5]; t.lb = rp[6];
}
__device__ __forceinline__ void tile_next(TileIt& t, const FFA_CONST int32_t* rp, int n_runs) {
  if (++t.ti >= t.nt && t.ri + 1 < n_runs) {
    ++t.ri;
    t.ti = 0;
    const FFA_CONST int32_t* r = rp + t.ri * ffa::kRec;
    t.k0 = r[0]; t.nt = r[1]; t.nf = r[2]; t.khi = r[3]; t.eb = r[4]; t.nl = r[5]; t.lb = r[6];
  }
}

// Host: calls f(std::integral_constant<int, D>{}) for the head dim d (16, 32, 64 or
// 128; the planner has validated it).
template <typename F>
inline void dispatch_dtype(int dtype, F&& f) {
  if (dtype == FFA_DTYPE_F16) f(_Float16{});
  else f(__bf16{});
}
template <typename F>
inline void dispatch_head_dim(int d, F&& f) {
  if (d == 128) f(std::integral_constant<int, 128>{});
  else if (d == 64) f(std::integral_constant<int, 64>{});
  else if (d == 32) f(std::integral_constant<int, 32>{});
  else f(std::integral_constant<int, 16>{});
}

}  // namespace dev
}  // namespace ffa
