// device_common.h -- gfx950 building blocks shared by the prefill and decode
// kernels: vector types, bf16 MFMA wrappers, the LDS transpose read, the
// cross-half lane exchange and the declared conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace invattn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kNegInf = -__builtin_inff();

// Word 3 of a raw buffer resource (gfx9 family): 32-bit data format, no
// swizzle, no index stride.  Loads past num_records return zeros.
constexpr int kBufferFlags = 0x00020000;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Operand layout (lane l): A row l%32, k 8*(l/32)+s; B column l%32, same k.
// Result: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4, i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Operand layout (lane l): A row l%16, k 8*(l/16)+s; B column l%16, same k.
// Result: lane l holds column l%16, rows 4*(l/16) + i, i = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// D(16x16, fp32) += A(16x16, bf16) * B(16x16, bf16).
// Operand layout (lane l): A row l%16, k 4*(l/16)+s; B column l%16, same k.
// Result: lane l holds column l%16, rows 4*(l/16) + i, i = 0..3.
__device__ __forceinline__ f32x4 mfma16k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                  __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// 16-byte load from global memory as 8 bf16.
__device__ __forceinline__ bf16x8 ld_global_x8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// 16-byte load from LDS.
__device__ __forceinline__ bf16x8 ld_lds_x8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4a+c receives element c of the 4-element rows addressed by lanes
// a, a+4, a+8, a+12 of the group (as result elements 0..3).
__device__ __forceinline__ bf16x4 ld_lds_tr(const bf16* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
  return __builtin_bit_cast(bf16x4, t);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Values of lanes l and l^32 as (low-half lane's value, high-half lane's
// value), identical in both lanes.
struct HalfPair {
  float lo, hi;
};
__device__ __forceinline__ HalfPair half_pair(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return HalfPair{__builtin_bit_cast(float, (uint32_t)r[0]),
                  __builtin_bit_cast(float, (uint32_t)r[1])};
}

// Values of lanes l and l^16 as (even 16-lane row's value, odd row's value),
// identical in both lanes.
__device__ __forceinline__ HalfPair row_pair(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return HalfPair{__builtin_bit_cast(float, (uint32_t)r[0]),
                  __builtin_bit_cast(float, (uint32_t)r[1])};
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes
// complete, then s_barrier.  Unlike __syncthreads() (a release/acquire fence
// at workgroup scope), it leaves direct HBM -> LDS loads in flight: the
// caller waits for the ones the next step reads (wait_vmcnt) before it.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// acc *= a for a 16x16 accumulator held in AGPRs (one wave per SIMD): each
// element moves to a VGPR, is multiplied, and moves back.  The elements are
// taken apart and put back so the vector itself never needs an address.
__device__ __forceinline__ void scale_acc4(f32x4& acc, float a) {
  float e[4] = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t;
    __asm__ volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(e[i]), "=&v"(t)
        : "v"(a));
  }
  acc = f32x4{e[0], e[1], e[2], e[3]};
}

// acc (=|+=) A * B on v_mfma_f32_16x16x32_bf16 with the accumulator in
// VGPRs.  With one wave per SIMD the compiler puts every builtin MFMA
// accumulator in AGPRs, and on gfx950 a read of an AGPR (v_accvgpr_read)
// while MFMAs are in flight stalls for about ten cycles, so accumulators
// that VALU code reads (attention scores) are formed here instead.  Hazards
// are the caller's: A and B are not rewritten during the MFMA's first
// passes (they come from LDS reads waited for before, or stay fixed), acc is
// only chained through these MFMAs, and the caller waits (mfma_drain) before
// VALU code reads it.
__device__ __forceinline__ void mfma16_vacc_first(f32x4& acc, bf16x8 a, bf16x8 b) {
  __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_vacc(f32x4& acc, bf16x8 a, bf16x8 b) {
  __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// acc (=|+=) A * B on v_mfma_f32_16x16x32_bf16 with the accumulator pinned
// to AGPRs (one wave per SIMD keeps large accumulators there).  Written as
// volatile inline asm so the register allocator never moves accumulators
// through VGPRs and LDS reads keep their source order around the MFMAs (the
// caller places operand reads ahead by hand).  Hazard distances are the
// caller's: no VALU write of a or b in the two cycles before, no VALU read
// of acc within 18 cycles after.
__device__ __forceinline__ void mfma16_agpr_first(f32x4& acc, bf16x8 a, bf16x8 b) {
  __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_agpr(f32x4& acc, bf16x8 a, bf16x8 b) {
  __asm__ volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last accumulator MFMA and VALU reads of it.
__device__ __forceinline__ void mfma_drain() {
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
}

// A zero accumulator created in AGPRs (a 16x16x32 MFMA of zero operands with
// an inline-constant zero addend), so a loop-carried accumulator is AGPR from
// its first definition on.
__device__ __forceinline__ f32x4 agpr_zero4() {
  f32x4 r;
  const bf16x8 z = {};
  // The nop keeps the zero operand's VALU writes three wait states away.
  __asm__("s_nop 2\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(r) : "v"(z));
  return r;
}

// Wait until every vector-memory load of this wave (including direct
// HBM -> LDS loads) has completed.
__device__ __forceinline__ void wait_vmem() {
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// acc *= a.  With one wave per SIMD the accumulators live in AGPRs; the
// scaling is written on AGPR operands so they stay there (each element moves
// to a VGPR, is multiplied, and moves back).
template <int OCC>
__device__ __forceinline__ void scale_acc(f32x16& acc, float a) {
  if constexpr (OCC == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float t;
      __asm__ volatile(
          "v_accvgpr_read_b32 %1, %0\n\t"
          "v_mul_f32 %1, %1, %2\n\t"
          "v_accvgpr_write_b32 %0, %1"
          : "+a"(acc[i]), "=&v"(t)
          : "v"(a));
    }
  } else {
    acc *= a;
  }
}

// Wait until at most `n` vector-memory loads of this wave are outstanding
// (the newest ones); N is the pipeline depth minus two (0 = wait for all).
template <int N>
__device__ __forceinline__ void wait_vmem_keep(int n) {
  if constexpr (N == 0) {
    wait_vmem();
  } else {
    // vmcnt(n) with n = loads issued per tile times the tiles allowed in
    // flight; the encodings are immediates, so pick from a small table.
    switch (n * N) {
      case 1: __asm__ volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
      case 2: __asm__ volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
      case 4: __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
      case 8: __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
      case 16: __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
      case 32: __asm__ volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
      default: wait_vmem(); break;
    }
  }
}

// Declared cast: fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Find the span holding packed token `tok` in a sorted, disjoint list of
// [start, end) pairs.  Returns true and the bounds if found.
__device__ __forceinline__ bool find_span(const int32_t* __restrict__ spans, int n, int tok,
                                          int& s, int& e) {
  int lo = 0, hi = n;  // first span with start > tok
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (spans[2 * mid] <= tok) lo = mid + 1; else hi = mid;
  }
  if (lo == 0) return false;
  int a = spans[2 * (lo - 1)], b = spans[2 * (lo - 1) + 1];
  if (tok < b) { s = a; e = b; return true; }
  return false;
}

}  // namespace invattn
