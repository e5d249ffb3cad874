// device_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_{bf16,f16},
// one 64-lane wavefront, half = lane / 32, r = lane % 32):
//   A (32 x 16): lane holds A[m = r][k = half*8 .. half*8+7]       (16 bytes)
//   B (16 x 32): lane holds B[k = half*8 .. half*8+7][n = r]       (16 bytes)
//   C (32 x 32): lane holds C[m = (i/4)*8 + half*4 + i%4][n = r], i = 0..15
// A C tile can therefore feed the next product as a B operand without any
// data movement when its rows become the reduction index: the eight values
// i = 8s .. 8s+7 of a lane cover rows 16s + {half*4 + 0..3, 8 + half*4 + 0..3},
// i.e. a fixed permutation of 16 consecutive reduction indices.  Operands
// read from LDS along that index are stored in the same permuted order
// (perm16 below), so every product is a plain 16-byte read per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage-type traits: the 32x32x16 matrix-core product and the
// round-to-nearest-even packing of two fp32 values.
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  static __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
  // c += a * b with the accumulator in AGPRs (see acc_fence); NOP waits the
  // two cycles a matrix instruction needs after vector code wrote b.
  template <bool NOP>
  static __device__ __forceinline__ void mma_acc(f32x16_t& c, u32x4_t a, u32x4_t b) {
    if (NOP)
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    else
      asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  // acc + lo + hi of a packed pair, exactly as stored (v_dot2 with ones).
  static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed),
                                           __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
  }
};

template <>
struct Elem<_Float16> {
  static __device__ __forceinline__ f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
  template <bool NOP>
  static __device__ __forceinline__ void mma_acc(f32x16_t& c, u32x4_t a, u32x4_t b) {
    if (NOP)
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    else
      asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, packed),
                                  __builtin_bit_cast(f16x2_t, 0x3C003C00u), acc, false);
  }
};

// Accumulators held in AGPRs by the inline-asm matrix instructions of
// mma_acc: the compiler does not see those instructions, so before vector
// code reads or rewrites such accumulators this fence waits out the matrix
// pipeline (an 8-pass 32x32 product needs well under 24 wait states) and
// ties every accumulator to it, so that no such access is scheduled earlier.
template <int N>
__device__ __forceinline__ void acc_fence(f32x16_t (&acc)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int b = 0; b < N; ++b) asm volatile("" : "+a"(acc[b]));
}

// Position of reduction index j inside its group of 16 in a permuted LDS
// row: swaps bits 2 and 3 (see the file comment).
__device__ __forceinline__ int perm16(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ u32x4_t ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st_global8(void* p, u32x2_t v) {
  *reinterpret_cast<u32x2_t*>(p) = v;
}
__device__ __forceinline__ u32x4_t ld_lds16(const char* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st_lds16(char* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ void st_lds8(char* p, u32x2_t v) { *reinterpret_cast<u32x2_t*>(p) = v; }

// Value held by the other half of the wavefront (lane ^ 32), combined with
// this lane's value by max / sum; symmetric in the two operands, so the
// result is the same in both halves.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v *= s elementwise, in place.  Written with a tied operand so that a
// rarely-taken rescale keeps the accumulator in the registers it already
// occupies (otherwise the common path pays a copy of every register to merge
// the two versions).
__device__ __forceinline__ void scale_in_place(f32x16_t& v, float s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = v[i];
    asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(s));
    v[i] = x;
  }
}

// Buffer resources over one head's rows: loads past `bytes` return zeros and
// stores past it are dropped by the hardware, which is how ragged tails and
// padding rows are handled without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
__device__ __forceinline__ void buf_store8(u32x2_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r,
                                        static_cast<int>(voff), 0, 0);
}
__device__ __forceinline__ void buf_store16(u32x4_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(voff), 0, 0);
}
__device__ __forceinline__ void buf_store4(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(voff), 0, 0);
}

// Direct HBM-to-LDS load of 16 bytes per lane: lane i of the wavefront writes
// lds + 16*i (the LDS address is wavefront-uniform); past `bytes` of the
// buffer the hardware writes zeros.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                               uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16,
                                           static_cast<int>(voff), static_cast<int>(soff), 0, 0);
}

// Waits until every vector-memory operation this wavefront issued (including
// direct-to-LDS loads) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits until at most N of this wavefront's vector-memory operations are
// still outstanding (they complete in issue order), i.e. everything but the N
// most recently issued has completed.  s_waitcnt encodes vmcnt in bits 3:0
// and 15:14; expcnt (bits 6:4) and lgkmcnt (bits 11:8) are left at "any".
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lanes 4t .. 4t+3 point at the four 4-element pieces of row t of a 4 x 16
// block of 16-bit elements; lane j of the group receives column j, i.e. the
// four elements (row 0..3, column j).
__device__ __forceinline__ u32x2_t ld_lds_tr8(const char* p) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (__attribute__((address_space(3))) s16x4_t*)(p)));
}

// Transpose helper: from four 32-bit words holding element pairs (e, e+1) of
// four rows r0..r3, build two words per element: (r0, r1) and (r2, r3).
// byte selectors for v_perm_b32 (bytes 0..3 of the second operand, 4..7 of
// the first): low halves and high halves of two words.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // a.lo | b.lo << 16
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.hi | b.hi << 16
}

// Writes the transpose of a 4-row x 8-column block of 16-bit elements into a
// column-major LDS tile whose columns are rows of `pitch` bytes: rows[r] holds
// row r's 8 elements; column c of the block goes to LDS row (c0 + c), at the
// 8-byte slot `slot_off(c0 + c)` returned by the caller's layout functor.
template <typename SlotOff>
__device__ __forceinline__ void write_transposed_4x8(char* base, const u32x4_t rows[4], int c0,
                                                     SlotOff slot_off) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x0 = rows[0][w], x1 = rows[1][w], x2 = rows[2][w], x3 = rows[3][w];
    u32x2_t even = {lo_halves(x0, x1), lo_halves(x2, x3)};
    u32x2_t odd = {hi_halves(x0, x1), hi_halves(x2, x3)};
    st_lds8(base + slot_off(c0 + 2 * w), even);
    st_lds8(base + slot_off(c0 + 2 * w + 1), odd);
  }
}

}  // namespace attn
