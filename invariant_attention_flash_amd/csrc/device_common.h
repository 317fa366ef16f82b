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
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kNegInf = -__builtin_inff();

// Word 3 of a raw buffer resource (gfx9 family): 32-bit data format, no
// swizzle, no index stride.  Loads past num_records return zeros.
constexpr int kBufferFlags = 0x00020000;

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

// Wait until every vector-memory load of this wave (including direct
// HBM -> LDS loads) has completed.
__device__ __forceinline__ void wait_vmem() {
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Read a loaded register here, so that the compiler's own wait insertion
// (to which the waits above are opaque) waits for its load at this point.
// Placed before a loop, it keeps a register loaded before the loop and first
// read inside it from getting a wait in the loop body: such a wait runs every
// iteration and, since the hardware counter does not tell loads apart, also
// waits for the loads the loop has in flight by then.
template <class T>
__device__ __forceinline__ void arrived(const T& x) {
  __asm__ volatile("" ::"v"(x));
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

// x / l rounded as the IEEE fp32 division rounds it, given y = RN(1/l):
// q0 = RN(x*y) is within one ulp of x/l, the residual x - q0*l is exact as
// an FMA, and RN(q0 + residual*y) is then the correctly rounded quotient
// (Markstein's correction step with a correctly rounded reciprocal).  This
// holds while nothing underflows: for l in [1, 2^40) and a quotient of
// magnitude at least kRecipDivMin.  Callers check the result against that
// bound and divide directly when it fails (or is NaN).
constexpr float kRecipDivMin = 0x1p-100f;
__device__ __forceinline__ float div_by_recip(float x, float l, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, l, x);
  return __builtin_fmaf(r, y, q0);
}

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

// The spans of a sorted, disjoint list of [start, end) pairs that meet the
// packed tokens [a, b): indices [first, last), with first the first span
// ending after a and last the first starting at or after b.  A token t in
// [a, b) lies in span i (start_i <= t < end_i) for at most one i, in
// [first, last): the span find_span returns for t.  a and b are
// wave-uniform, and the list is read with scalar loads (spans_at), so a
// search costs scalar-cache round trips rather than vector-memory ones.
__device__ __forceinline__ int span_word(const int32_t* __restrict__ spans, int i) {
  using ConstI32 = const __attribute__((address_space(4))) int32_t;
  return ((ConstI32*)spans)[i];
}
__device__ __forceinline__ void spans_meeting(const int32_t* __restrict__ spans, int n, int a,
                                              int b, int& first, int& last) {
  a = __builtin_amdgcn_readfirstlane(a);
  b = __builtin_amdgcn_readfirstlane(b);
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (span_word(spans, 2 * mid + 1) <= a) lo = mid + 1; else hi = mid;
  }
  first = lo;
  while (lo < n && span_word(spans, 2 * lo) < b) ++lo;
  last = lo;
}

}  // namespace invattn
