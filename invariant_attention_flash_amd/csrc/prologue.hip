// prologue.hip -- the attention prologue of a layer, on Q and K in place:
// RMSNorm of every (token, head) vector over the head dim, then rotary
// position embedding (RoPE) on its first R dims.
//
// Sources: the layer prologue names a Q/K RMSNorm for head dims 256 and 512,
// a RoPE on the sliding layers and a proportional ("p") RoPE on the global
// layers ("RFC: Gemma-4-31B-it train/rollout consistency", section 6, items 4
// and 6); the norm keeps every multiply in fp32 with one cast at the store,
// and scales by (weight offset + weight) ("Gated RMSNorm CUDA kernel for the
// GDN block", Summary; without its gate).  The pages give no epsilon, offset,
// rotary width, frequency base or pairing: they are arguments, and the
// pairing is (i, i + R/2).
//
// Declared arithmetic, per (token, head) vector x of D bf16 values:
//   ss = sum of x_d^2 in fp32: each lane adds its D/64 elements in ascending
//        order, then lanes combine by the exchange tree xor 32, 16, 8, 4, 2,
//        1 (each step adds two lanes' sums; every lane ends with the same bits)
//   r  = 1 / sqrt(ss / D + eps)          (IEEE fp32 division and square root)
//   y_d = (x_d * r) * (offset + w_d)     (no norm when the weight is NULL)
//   for i < R/2, the angle a_i = pos * 2^(-2i/F * log2 theta) is formed in
//   fp64 and reduced in fp64 by the nearest multiple k of pi/2 (pi/2 held as
//   two doubles); c_i and s_i are the fp32 cosine and sine of the reduced
//   angle (|r| <= pi/4, rounded to fp32), placed by the quadrant k mod 4; then
//   out_i = y_i c_i - y_{i+R/2} s_i,  out_{i+R/2} = y_i s_i + y_{i+R/2} c_i
//   (fp32, each product rounded), dims R .. D-1 pass through; bf16 RNE store.
// A vector's bytes depend only on itself, its position and the arguments:
// nothing in it depends on the batch, the packing or the launch.
//
// Work map: one workgroup of four waves per token; the table of (c_i, s_i)
// is formed once per token in LDS, and each wave takes every fourth head
// vector of the token (Q heads, then K heads), one or two at a time, lane l
// holding elements [l*D/64, (l+1)*D/64).  HBM-bound: every vector is read
// and written once.
#include "device_common.h"
#include "kernels.h"

namespace invattn {

namespace {

constexpr int kPrologueThreads = 256;
// Head vectors a wave loads before it computes: 2 at head dims up to 256, 1
// at 512 (more registers per vector cost more occupancy than the extra loads
// in flight gain; batches of 4 and 8 were slower at both).
template <int D>
constexpr int prologue_batch() { return D >= 512 ? 1 : 2; }

template <int E>
struct Chunk;
template <>
struct Chunk<1> {
  using T = uint16_t;
};
template <>
struct Chunk<4> {
  using T = uint2;
};
template <>
struct Chunk<8> {
  using T = uint4;
};

template <int E>
__device__ __forceinline__ void unpack(const typename Chunk<E>::T& c, float (&x)[E]) {
  const bf16* b = reinterpret_cast<const bf16*>(&c);
#pragma unroll
  for (int j = 0; j < E; ++j) x[j] = (float)b[j];
}

template <int E>
__device__ __forceinline__ typename Chunk<E>::T pack(const float (&x)[E]) {
  typename Chunk<E>::T c;
  bf16* b = reinterpret_cast<bf16*>(&c);
#pragma unroll
  for (int j = 0; j < E; ++j) b[j] = to_bf16(x[j]);
  return c;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kPrologueThreads) void qk_prologue_kernel(
    bf16* __restrict__ q, bf16* __restrict__ k, const int32_t* __restrict__ positions, int hq,
    int hkv, const float* __restrict__ qw, const float* __restrict__ kw, float eps, float offset,
    int half, int freq_dims, double theta) {
  constexpr int E = D / 64;  // elements per lane
  constexpr int kPrologueBatch = prologue_batch<D>();
  using CT = typename Chunk<E>::T;
  __shared__ float2 cs[D / 2];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double pos = (double)positions[t];
  const double l2t = log2(theta);
  for (int i = tid; i < half; i += kPrologueThreads) {
    const double ang = pos * exp2(-2.0 * i / freq_dims * l2t);
    // reduce by pi/2 in fp64 (2/pi, and pi/2 as a leading double plus the
    // rest), then the fp32 functions on |r| <= pi/4
    const double kq = rint(ang * 0.63661977236758134308);
    const float r =
        (float)(__builtin_fma(-kq, 1.5707963267948966192, ang) - kq * 6.123233995736766e-17);
    const float sr = sinf(r), cr = cosf(r);
    const int qd = (int)((long long)kq & 3);
    const float cv = qd == 0 ? cr : qd == 1 ? -sr : qd == 2 ? -cr : sr;
    const float sv = qd == 0 ? sr : qd == 1 ? cr : qd == 2 ? -sr : -cr;
    cs[i] = make_float2(cv, sv);
  }
  __syncthreads();

  // This lane's elements and their rotation partner lane (the host requires
  // R/2 to be a multiple of E, so a lane's elements lie in one half).
  const int e0 = E * lane;
  const bool first = e0 < half;
  const bool turned = e0 < 2 * half;
  const int partner = first ? lane + half / E : (turned ? lane - half / E : lane);
  float c[E], s[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = turned ? (first ? e0 + j : e0 + j - half) : 0;  // always inside the table
    const float2 v = turned ? cs[i] : make_float2(1.f, 0.f);
    c[j] = v.x;
    s[j] = v.y;
  }

  const int nh = hq + hkv;
  for (int h0 = wave; h0 < nh; h0 += 4 * kPrologueBatch) {
    CT* rows[kPrologueBatch];
    CT raw[kPrologueBatch];
#pragma unroll
    for (int u = 0; u < kPrologueBatch; ++u) {
      const int h = h0 + 4 * u;
      const int hh = h < nh ? h : h0;  // past the last vector: reload the first (never stored)
      bf16* row = hh < hq ? q + ((size_t)t * hq + hh) * D : k + ((size_t)t * hkv + (hh - hq)) * D;
      rows[u] = reinterpret_cast<CT*>(row) + lane;
      raw[u] = *rows[u];
    }
#pragma unroll
    for (int u = 0; u < kPrologueBatch; ++u) {
      const int h = h0 + 4 * u;
      if (h >= nh) break;  // wave-uniform
      float x[E];
      unpack<E>(raw[u], x);
      const float* w = h < hq ? qw : kw;
      if (w != nullptr) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < E; ++j) ss = ss + x[j] * x[j];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) ss = ss + __shfl_xor(ss, m, 64);
        const float r = 1.0f / __builtin_sqrtf(ss / (float)D + eps);
#pragma unroll
        for (int j = 0; j < E; ++j) x[j] = (x[j] * r) * (offset + w[e0 + j]);
      }
      if (half > 0) {
        float p[E];
#pragma unroll
        for (int j = 0; j < E; ++j) p[j] = __shfl(x[j], partner, 64);
        if (turned) {
#pragma unroll
          for (int j = 0; j < E; ++j)
            x[j] = first ? x[j] * c[j] - p[j] * s[j] : p[j] * s[j] + x[j] * c[j];
        }
      }
      *rows[u] = pack<E>(x);
    }
  }
}

hipError_t launch_qk_prologue(const PrologueArgs& a, hipStream_t stream, const char** kernel) {
  const dim3 grid((unsigned)a.tokens), block(kPrologueThreads);
  const int half = a.rotary_dims / 2;
#define X(D)                                                                                  \
  if (a.d == D) {                                                                             \
    *kernel = "qk_prologue_kernel<" #D ">";                                                   \
    hipLaunchKernelGGL(qk_prologue_kernel<D>, grid, block, 0, stream, (bf16*)a.q, (bf16*)a.k, \
                       a.positions, a.hq, a.hkv, a.q_weight, a.k_weight, a.eps, a.offset, half, \
                       a.freq_dims, a.theta);                                                 \
    return hipGetLastError();                                                                 \
  }
  X(64) X(256) X(512)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
