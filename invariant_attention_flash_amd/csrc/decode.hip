// decode.hip -- single-token attention against a paged KV cache, read in
// place through the block table, with a fixed split and a fixed merge.
//
// Sources: strict decode reads the paged KV cache directly with a fixed
// schedule ("Vime ROCm Attention operator ablation", "Prerequisites" and
// "Runtime artifacts and validation"); a split-KV is allowed only when the
// split and the merge tree are fixed ("RFC: Gemma-4-31B-it train/rollout
// consistency", section 4, item 3); hybrid_kv_cache_contract (section 6).
//
// Split.  Keys are cut into chunks of kDecodeChunk positions aligned to
// position 0.  The chunk size is a constant, so a sequence's chunks -- and
// the bytes of its output -- do not depend on the batch it is decoded in.
//
// Chunk kernel: one workgroup per (chunk, KV head, sequence).  It walks the
// chunk in 32-key sub-tiles, ascending.  K and V of a sub-tile go to LDS
// (keys outside [kv_lo, L) are zero and their block-table entries are never
// read).  Every wave computes the same S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
// the G query heads of the group padded to 16 columns) and so the same
// online-softmax state; each wave owns a quarter of the head dim for
// O^T += V^T P^T.  The record (acc[D], m, l) of the chunk goes to the
// workspace.
//
// Merge kernel: one workgroup per (query head, sequence) folds the chunk
// records in ascending chunk order (m' = max(m, m_c); acc = acc*2^(m-m') +
// acc_c*2^(m_c-m'); l likewise), then o = bf16_rne(acc / l).
#include "device_common.h"
#include "kernels.h"

namespace invattn {

template <int D_, int G_>
struct DecodeCfg {
  static constexpr int D = D_, G = G_;
  static constexpr int kThreads = 256;
  static constexpr int kSub = kDecodeSub;
  static constexpr int kStrideK = D + 8;
  static constexpr int kStrideV = D + 8;
  static constexpr int kLdsElems = kSub * (kStrideK + kStrideV);
  static constexpr int kSteps = D / 32;        // 16x16x32 k-steps over d
  static constexpr int kDPerWave = D / 4;
  static constexpr int kDBlk = kDPerWave / 16;  // 16-wide output blocks per wave
  static constexpr int kChunkPerRow = D / 8;
  static constexpr int kChunksPerThread = kSub * D / 8 / kThreads;
  static constexpr int kRec = decode_record_floats(D);
  static_assert(G <= 16, "group fits one MFMA column block");
  static_assert(kSub * D / 8 % kThreads == 0, "sub-tile load split");
};

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void decode_chunk_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                         const bf16* __restrict__ vc, const int32_t* __restrict__ bt,
                         int max_blocks, const int32_t* __restrict__ seq_lens, int max_seq_len,
                         int num_blocks, int hq, int hkv, int window, float c2,
                         float* __restrict__ ws, int n_chunks) {
  constexpr int D = C::D, G = C::G;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::kLdsElems];
  bf16* Ks = smem;
  bf16* Vs = smem + C::kSub * C::kStrideK;

  const int b = blockIdx.z, g = blockIdx.y, c = blockIdx.x;
  int L = seq_lens[b];
  L = min(L, min(max_seq_len, max_blocks * 16));
  if (L <= 0) return;
  const int kv_lo = window > 0 ? max(0, L - window) : 0;
  const int c0 = c * kDecodeChunk;
  const int c1 = min(c0 + kDecodeChunk, L);
  const int a0 = max(c0, kv_lo);
  if (a0 >= c1) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const bool qv = col < G;
  const int head = g * G + (qv ? col : 0);

  // Q^T operand: column col = query head g*G+col, k = d = 32*s + 8*grp + e.
  bf16x8 qr[C::kSteps];
  {
    const bf16* qrow = q + ((size_t)b * hq + head) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      bf16x8 x = ld_global_x8(qrow + 32 * s);
      qr[s] = qv ? x : bf16x8{};
    }
  }

  f32x4 oacc[C::kDBlk];
#pragma unroll
  for (int db = 0; db < C::kDBlk; ++db) oacc[db] = f32x4{};
  float m = kNegInf, l = 0.f;

  const int32_t* table = bt + (size_t)b * max_blocks;
  const size_t slot_stride = (size_t)hkv * D;
  const int st0 = a0 / C::kSub, st1 = (c1 + C::kSub - 1) / C::kSub;
  for (int st = st0; st < st1; ++st) {
    const int k0 = st * C::kSub;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int cc = tid + i * C::kThreads;
      const int row = cc / C::kChunkPerRow;
      const int cx = (cc % C::kChunkPerRow) * 8;
      const int key = k0 + row;
      u32x4 kx = u32x4{}, vx = u32x4{};
      if (key >= kv_lo && key < L) {
        const int blk = table[key >> 4];
        if (blk >= 0 && blk < num_blocks) {
          const size_t off = ((size_t)blk * 16 + (key & 15)) * slot_stride + (size_t)g * D + cx;
          kx = *reinterpret_cast<const u32x4*>(kc + off);
          vx = *reinterpret_cast<const u32x4*>(vc + off);
        }
      }
      *reinterpret_cast<u32x4*>(Ks + row * C::kStrideK + cx) = kx;
      *reinterpret_cast<u32x4*>(Vs + row * C::kStrideV + cx) = vx;
    }
    __syncthreads();

    // S^T for keys k0 + [0,16) (s0) and k0 + [16,32) (s1).
    f32x4 s0 = f32x4{}, s1 = f32x4{};
    const bf16* krow = Ks + col * C::kStrideK + 8 * grp;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      s0 = mfma16(ld_lds_x8(krow + 32 * s), qr[s], s0);
      s1 = mfma16(ld_lds_x8(krow + 16 * C::kStrideK + 32 * s), qr[s], s1);
    }
    float x[8];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = k0 + (i < 4 ? 0 : 16) + 4 * grp + (i & 3);
      const float sv = (i < 4 ? s0[i] : s1[i - 4]) * c2;
      const bool ok = qv && j >= kv_lo && j < L;
      x[i] = ok ? sv : kNegInf;
      tmax = fmaxf(tmax, x[i]);
    }
    // Reduce over the four lane groups holding the same query (xor 16, 32).
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m - m_new);
    const float msub = (m_new == kNegInf) ? 0.f : m_new;
    float psum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = fast_exp2(x[i] - msub);
      psum += p;
      pb[i] = to_bf16(p);
    }
    psum = psum + __shfl_xor(psum, 16);
    psum = psum + __shfl_xor(psum, 32);
    l = l * alpha + psum;
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::kDBlk; ++db) oacc[db] *= alpha;
    }
    // O^T += V^T P^T for this wave's quarter of the head dim.  Operand slot
    // e covers key (e < 4 ? 0 : 16) + 4*grp + e%4 on both sides.
    const bf16* vrow = Vs + (4 * grp + (col >> 2)) * C::kStrideV + wave * C::kDPerWave +
                       4 * (col & 3);
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db) {
      const bf16x4 lo4 = ld_lds_tr(vrow + 16 * db);
      const bf16x4 hi4 = ld_lds_tr(vrow + 16 * C::kStrideV + 16 * db);
      oacc[db] = mfma16(cat8(lo4, hi4), pb, oacc[db]);
    }
  }

  if (qv) {
    float* rec = ws + (((size_t)b * hq + head) * n_chunks + c) * C::kRec;
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db)
      *reinterpret_cast<f32x4*>(rec + wave * C::kDPerWave + 16 * db + 4 * grp) = oacc[db];
    if (wave == 0 && grp == 0) {
      rec[D] = m;
      rec[D + 1] = l;
    }
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void decode_merge_kernel(const float* __restrict__ ws, const int32_t* __restrict__ seq_lens,
                         int max_seq_len, int max_blocks, int hq, int window, int n_chunks,
                         bf16* __restrict__ o) {
  constexpr int kPer = D / 64;
  constexpr int kRec = decode_record_floats(D);
  const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  bf16* orow = o + ((size_t)b * hq + head) * D + tid * kPer;
  int L = seq_lens[b];
  L = min(L, min(max_seq_len, max_blocks * 16));
  if (L <= 0) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) orow[e] = to_bf16(0.f);
    return;
  }
  const int kv_lo = window > 0 ? max(0, L - window) : 0;
  const int c_lo = kv_lo / kDecodeChunk, c_hi = (L - 1) / kDecodeChunk;
  const float* base = ws + ((size_t)b * hq + head) * n_chunks * kRec;
  float m = kNegInf, l = 0.f, acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  for (int c = c_lo; c <= c_hi; ++c) {
    const float* rec = base + (size_t)c * kRec;
    const float mc = rec[D], lc = rec[D + 1];
    const float m_new = fmaxf(m, mc);
    const float a = fast_exp2(m - m_new);
    const float bc = fast_exp2(mc - m_new);
    l = l * a + lc * bc;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] = acc[e] * a + rec[tid * kPer + e] * bc;
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) orow[e] = to_bf16(acc[e] / l);
}

template <int D, int G>
static hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  using C = DecodeCfg<D, G>;
  dim3 grid(a.n_chunks, a.hkv, a.batch);
  hipLaunchKernelGGL(decode_chunk_kernel<C>, grid, dim3(C::kThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache,
                     a.block_table, a.max_blocks, a.seq_lens, a.max_seq_len, a.num_blocks, a.hq,
                     a.hkv, a.window, a.c2, a.workspace, a.n_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(a.hq, a.batch), dim3(64), 0, stream,
                     (const float*)a.workspace, a.seq_lens, a.max_seq_len, a.max_blocks, a.hq,
                     a.window, a.n_chunks, (bf16*)a.o);
  return hipGetLastError();
}

#define INVATTN_DECODE_TABLE(X) \
  X(64, 1) X(64, 2) X(64, 4) X(64, 8)     \
  X(256, 1) X(256, 2) X(256, 4) X(256, 8) \
  X(512, 1) X(512, 2) X(512, 4) X(512, 8)

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.hq / a.hkv;
#define X(D, G) \
  if (a.d == D && group == G) return launch_one<D, G>(a, stream);
  INVATTN_DECODE_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
