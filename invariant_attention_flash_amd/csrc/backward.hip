// backward.hip -- deterministic attention backward (dq, dk, dv) for packed
// variable-length prefill, with every sum in a fixed order and no atomics.
//
// Sources: the train/rollout consistency goal covers the training step
// ("RFC: Gemma-4-31B-it train/rollout consistency", section 1 and section 4
// item 1: every reduction has a declared fp32 accumulator and a fixed order;
// item 3: no split-K, Stream-K or cross-workgroup atomics); the gradient is
// the chain rule on the forward's definition (same masks, spans and GQA map
// as prefill.hip).
//
// Arithmetic (fp32 FMAs throughout; c = fl32(scale * log2 e), and the
// forward's natural-log LSE enters as lse2 = fl32(lse * log2 e)):
//   delta_i = sum_d dout[i,d] * o[i,d]         (o: the forward's bf16 output)
//   s_ij    = sum_d q[i,d] * k[j,d]             dp_ij = sum_d dout[i,d] * v[j,d]
//   p_ij    = exp2(fma(s_ij, c, -lse2_i))       (0 where the mask excludes j)
//   ds_ij   = p_ij * (dp_ij - delta_i)
//   dq_i    = scale * sum_j ds_ij k_j           (keys ascending)
//   dk_j    = scale * sum_i sum_h ds_ij q_i     (rows ascending, then the
//   dv_j    =         sum_i sum_h p_ij dout_i    group's query heads ascending)
// Each dot product runs over the head dim in 32-element parts (fma chain,
// ascending), the parts added by a fixed butterfly.  A thread owns 32
// head-dim elements of one row (dq kernel) or one key (dk/dv kernel); the
// D/32 threads of a row or key are adjacent lanes.  Every output element is
// written once, by one thread, so the result does not depend on the batch,
// the packing or the launch geometry.
#include "device_common.h"
#include "kernels.h"

namespace invattn {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kPart = 32;  // head-dim elements per thread

template <int D>
struct BwdCfg {
  static constexpr int P = D / kPart;               // threads per row / key
  static constexpr int kRows = kBwdThreads / P;     // rows (keys) per workgroup
  // LDS staging: 64 KB of fp32 per chunk.
  static constexpr int kKeyChunk = 65536 / (D * 4 * 2);  // keys per chunk (K and V)
  static_assert(D % kPart == 0 && P <= 64 && (P & (P - 1)) == 0, "part map");
};

// Sum over the P adjacent lanes of a row (butterfly: every lane ends with
// the same value, the additions in the same order).
template <int P>
__device__ __forceinline__ float part_sum(float x) {
#pragma unroll
  for (int m = P / 2; m >= 1; m >>= 1) x = x + __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ void load_part(const bf16* __restrict__ src, float* dst) {
#pragma unroll
  for (int c = 0; c < kPart; c += 8) {
    const bf16x8 x = ld_global_x8(src + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[c + e] = (float)x[e];
  }
}

__device__ __forceinline__ float dot_part(const float* a, const float* b) {
  float s = a[0] * b[0];
#pragma unroll
  for (int c = 1; c < kPart; ++c) s = __builtin_fmaf(a[c], b[c], s);
  return s;
}

__device__ __forceinline__ bool admits(int i, int j, int window, int ss, int se) {
  const bool causal = j <= i && (window < 0 || i - j < window);
  return causal || (j >= ss && j < se);
}

// dq of a tile of rows of one query head, and delta of those rows.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads)))
void bwd_dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                   const bf16* __restrict__ v, const bf16* __restrict__ o,
                   const float* __restrict__ lse, const bf16* __restrict__ dout,
                   float* __restrict__ dq, float* __restrict__ delta,
                   const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ spans,
                   int num_spans, int hq, int hkv, int window, float scale, float c2) {
  using C = BwdCfg<D>;
  constexpr int P = C::P, KC = C::kKeyChunk;
  __shared__ __attribute__((aligned(16))) float kv[2][KC][D];
  const int b = blockIdx.z, h = blockIdx.y, g = h / (hq / hkv);
  const int seq0 = cu_seqlens[b], L = cu_seqlens[b + 1] - seq0;
  const int r0 = blockIdx.x * C::kRows;
  if (r0 >= L) return;
  const int r1 = min(r0 + C::kRows, L);
  const int tid = threadIdx.x, part = tid % P;
  const int i = r0 + tid / P;
  const bool live = i < r1;
  const int ic = live ? i : r0;  // rows past the tile load row r0 and store nothing
  const size_t qo = ((size_t)(seq0 + ic) * hq + h) * D + part * kPart;

  float qv[kPart], dov[kPart], acc[kPart];
  load_part(q + qo, qv);
  load_part(dout + qo, dov);
  float del;
  {
    float ov[kPart];
    load_part(o + qo, ov);
    del = part_sum<P>(dot_part(dov, ov));
  }
  if (live && part == 0) delta[(size_t)(seq0 + i) * hq + h] = del;
  const float lse2 = lse[(size_t)(seq0 + ic) * hq + h] * 1.4426950408889634f;
#pragma unroll
  for (int c = 0; c < kPart; ++c) acc[c] = 0.f;

  int ss = 0, se = 0, s0, e0;
  if (num_spans > 0 && find_span(spans, num_spans, seq0 + ic, s0, e0)) {
    ss = s0 - seq0;
    se = e0 - seq0;
  }
  // Keys of the tile's rows: the window below its first row, the span of its
  // first row, its last row, the span of its last row.
  int lo = window > 0 ? max(0, r0 - window + 1) : 0;
  int hi = r1;
  if (num_spans > 0) {
    if (find_span(spans, num_spans, seq0 + r0, s0, e0)) lo = min(lo, max(s0 - seq0, 0));
    if (find_span(spans, num_spans, seq0 + r1 - 1, s0, e0)) hi = max(hi, min(e0 - seq0, L));
  }
  for (int j0 = lo; j0 < hi; j0 += KC) {
    const int n = min(KC, hi - j0);
    __syncthreads();
    for (int e = tid * 8; e < n * D; e += kBwdThreads * 8) {
      const int jj = e / D, c = e % D;
      const size_t ko = ((size_t)(seq0 + j0 + jj) * hkv + g) * D + c;
      const bf16x8 xk = ld_global_x8(k + ko), xv = ld_global_x8(v + ko);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        kv[0][jj][c + u] = (float)xk[u];
        kv[1][jj][c + u] = (float)xv[u];
      }
    }
    __syncthreads();
    for (int jj = 0; jj < n; ++jj) {
      const float* kr = &kv[0][jj][part * kPart];
      const float* vr = &kv[1][jj][part * kPart];
      float kp[kPart], vp[kPart];
#pragma unroll
      for (int c = 0; c < kPart; ++c) {
        kp[c] = kr[c];
        vp[c] = vr[c];
      }
      const float s = part_sum<P>(dot_part(qv, kp));
      const float dp = part_sum<P>(dot_part(dov, vp));
      const int j = j0 + jj;
      const float p = admits(ic, j, window, ss, se) ? fast_exp2(__builtin_fmaf(s, c2, -lse2)) : 0.f;
      const float ds = p * (dp - del);
#pragma unroll
      for (int c = 0; c < kPart; ++c) acc[c] = __builtin_fmaf(ds, kp[c], acc[c]);
    }
  }
  if (!live) return;
  float* out = dq + qo;
#pragma unroll
  for (int c = 0; c < kPart; c += 4) {
    float4 w;
    w.x = acc[c] * scale;
    w.y = acc[c + 1] * scale;
    w.z = acc[c + 2] * scale;
    w.w = acc[c + 3] * scale;
    *reinterpret_cast<float4*>(out + c) = w;
  }
}

// dk and dv of a tile of keys of one KV head.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads)))
void bwd_dkv_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ v, const float* __restrict__ lse,
                    const bf16* __restrict__ dout, const float* __restrict__ delta,
                    float* __restrict__ dk, float* __restrict__ dv,
                    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ spans,
                    int num_spans, int hq, int hkv, int window, float scale, float c2) {
  using C = BwdCfg<D>;
  constexpr int P = C::P;
  constexpr int kStage = 65536 / (D * 4 * 2);  // (row, head) pairs staged per chunk
  __shared__ __attribute__((aligned(16))) float qd[2][kStage][D];
  __shared__ float rl[kStage][2];     // lse2, delta
  __shared__ int rs[kStage][3];       // row, span start, span end
  const int b = blockIdx.z, g = blockIdx.y, G = hq / hkv;
  const int seq0 = cu_seqlens[b], L = cu_seqlens[b + 1] - seq0;
  const int j0 = blockIdx.x * C::kRows;
  if (j0 >= L) return;
  const int j1 = min(j0 + C::kRows, L);
  const int tid = threadIdx.x, part = tid % P;
  const int j = j0 + tid / P;
  const bool live = j < j1;
  const int jc = live ? j : j0;
  const size_t ko = ((size_t)(seq0 + jc) * hkv + g) * D + part * kPart;
  float kp[kPart], vp[kPart], ak[kPart], av[kPart];
  load_part(k + ko, kp);
  load_part(v + ko, vp);
#pragma unroll
  for (int c = 0; c < kPart; ++c) {
    ak[c] = 0.f;
    av[c] = 0.f;
  }
  // Rows that admit a key of the tile: from its first key (or the span of
  // its first key) to the window above its last key (or the span of its
  // last key).
  int s0, e0;
  int lo = j0;
  int hi = window > 0 ? min(L, j1 - 1 + window) : L;
  if (num_spans > 0) {
    if (find_span(spans, num_spans, seq0 + j0, s0, e0)) lo = min(lo, max(s0 - seq0, 0));
    if (find_span(spans, num_spans, seq0 + j1 - 1, s0, e0)) hi = max(hi, min(e0 - seq0, L));
  }
  // (row, head) pairs in order: rows ascending, the group's heads ascending.
  const long long n_pairs = (long long)(hi - lo) * G;
  for (long long w0 = 0; w0 < n_pairs; w0 += kStage) {
    const int n = (int)min((long long)kStage, n_pairs - w0);
    __syncthreads();
    for (int e = tid * 8; e < n * D; e += kBwdThreads * 8) {
      const int ww = e / D, c = e % D;
      const long long w = w0 + ww;
      const int i = lo + (int)(w / G), h = g * G + (int)(w % G);
      const size_t qo = ((size_t)(seq0 + i) * hq + h) * D + c;
      const bf16x8 xq = ld_global_x8(q + qo), xd = ld_global_x8(dout + qo);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        qd[0][ww][c + u] = (float)xq[u];
        qd[1][ww][c + u] = (float)xd[u];
      }
    }
    for (int ww = tid; ww < n; ww += kBwdThreads) {
      const long long w = w0 + ww;
      const int i = lo + (int)(w / G), h = g * G + (int)(w % G);
      const size_t ro = (size_t)(seq0 + i) * hq + h;
      rl[ww][0] = lse[ro] * 1.4426950408889634f;
      rl[ww][1] = delta[ro];
      int ss = 0, se = 0;
      if (num_spans > 0 && find_span(spans, num_spans, seq0 + i, s0, e0)) {
        ss = s0 - seq0;
        se = e0 - seq0;
      }
      rs[ww][0] = i;
      rs[ww][1] = ss;
      rs[ww][2] = se;
    }
    __syncthreads();
    for (int ww = 0; ww < n; ++ww) {
      const float* qr = &qd[0][ww][part * kPart];
      const float* dr = &qd[1][ww][part * kPart];
      float qv[kPart], dov[kPart];
#pragma unroll
      for (int c = 0; c < kPart; ++c) {
        qv[c] = qr[c];
        dov[c] = dr[c];
      }
      const float s = part_sum<P>(dot_part(qv, kp));
      const float dp = part_sum<P>(dot_part(dov, vp));
      const float p = admits(rs[ww][0], jc, window, rs[ww][1], rs[ww][2])
                          ? fast_exp2(__builtin_fmaf(s, c2, -rl[ww][0]))
                          : 0.f;
      const float ds = p * (dp - rl[ww][1]);
#pragma unroll
      for (int c = 0; c < kPart; ++c) {
        ak[c] = __builtin_fmaf(ds, qv[c], ak[c]);
        av[c] = __builtin_fmaf(p, dov[c], av[c]);
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int c = 0; c < kPart; c += 4) {
    float4 w;
    w.x = ak[c] * scale;
    w.y = ak[c + 1] * scale;
    w.z = ak[c + 2] * scale;
    w.w = ak[c + 3] * scale;
    *reinterpret_cast<float4*>(dk + ko + c) = w;
    *reinterpret_cast<float4*>(dv + ko + c) = make_float4(av[c], av[c + 1], av[c + 2], av[c + 3]);
  }
}

template <int D>
hipError_t launch_bwd_d(const BackwardArgs& a, hipStream_t stream) {
  using C = BwdCfg<D>;
  const unsigned tiles = (unsigned)((a.max_seqlen + C::kRows - 1) / C::kRows);
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(tiles, a.hq, a.batch), dim3(kBwdThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.o,
                     a.lse, (const bf16*)a.dout, a.dq, a.delta, a.cu_seqlens, a.spans,
                     a.num_spans, a.hq, a.hkv, a.window, a.scale, a.c2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3(tiles, a.hkv, a.batch), dim3(kBwdThreads), 0,
                     stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.lse,
                     (const bf16*)a.dout, (const float*)a.delta, a.dk, a.dv, a.cu_seqlens,
                     a.spans, a.num_spans, a.hq, a.hkv, a.window, a.scale, a.c2);
  return hipGetLastError();
}

}  // namespace

int backward_rows_per_tile(int d) {
  switch (d) {
    case 64: return BwdCfg<64>::kRows;
    case 256: return BwdCfg<256>::kRows;
    case 512: return BwdCfg<512>::kRows;
    default: return 0;
  }
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_bwd_d<64>(a, stream);
    case 256: return launch_bwd_d<256>(a, stream);
    case 512: return launch_bwd_d<512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace invattn
