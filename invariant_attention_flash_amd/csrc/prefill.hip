// prefill.hip -- batch-invariant attention forward over packed
// variable-length sequences (sliding-window and global layers, GQA,
// bidirectional spans), bf16 MFMA on gfx950.
//
// Sources: sliding and global attention cores are separate layer types with
// their own head geometry and masks ("RFC: Gemma-4-31B-it train/rollout
// consistency", section 3 "Architecture map", section 6
// sliding_attention_core / global_attention_core); the numerical contract of
// section 4 (fixed fp32 accumulators, an order independent of batch, packing,
// launch geometry and occupancy, no split-KV, no fast-math, declared casts);
// bidirectional soft-token spans (section 1, Phase B; contiguous soft-token
// runs in "Gemma-4-E4B-it multimodal baseline").
//
// Work map.  A workgroup owns `positions` consecutive positions of ONE
// sequence (aligned to the sequence start, never to the packed buffer) for
// the G query heads of one KV head: 128 query rows, 32 per wave, ordered
// position-major (row r = position*G + head).  A row therefore always lands
// in the same wave, lane and MFMA slot, and visits the same KV tiles in the
// same ascending order, whatever else is in the batch.
//
// Per KV tile (BN keys, ascending):
//   S^T = K Q^T  on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q in
//                registers), so each lane holds one query's scores;
//   scale by c = fl32(scale*log2 e), mask by select (-inf);
//   online softmax in fp32: tile max and row sums reduce first inside the
//                lane in register order, then across the lane pair (l, l^32);
//   P -> bf16 (RNE), O^T += V^T P^T on the same MFMA, with V^T read from a
//                row-major LDS tile by the LDS transpose read.
// Fully masked tiles are exact no-ops (alpha = 1, p = 0), so a wave skips
// the tiles outside its own key range and skips the O rescale when every
// alpha of the wave is 1; both skips depend only on the sequence.
#include "device_common.h"
#include "kernels.h"

namespace invattn {

template <int D_, int G_, int BN_>
struct PrefillCfg {
  static constexpr int D = D_, G = G_, BN = BN_;
  static constexpr int kThreads = 256;
  static constexpr int kRows = 128;
  static constexpr int kPositions = kRows / G;
  static constexpr int kPosPerWave = 32 / G;
  static constexpr int kStrideK = D + 8;  // LDS row stride (elements)
  static constexpr int kStrideV = D + 8;
  static constexpr int kLdsElems = BN * (kStrideK + kStrideV);
  static constexpr int kSteps = D / 16;  // MFMA k-steps over the head dim
  static constexpr int kSBlk = BN / 32;  // 32-key score blocks per tile
  static constexpr int kDBlk = D / 32;   // 32-wide output blocks
  static constexpr int kKK = BN / 16;    // 16-key PV k-steps per tile
  static constexpr int kChunkPerRow = D / 8;
  static constexpr int kChunksPerThread = BN * D / 8 / kThreads;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(BN * D / 8 % kThreads == 0, "tile load split");
};

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void prefill_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ v, bf16* __restrict__ o,
                    float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                    const int32_t* __restrict__ spans, int num_spans, int hq, int hkv,
                    int window, float c2) {
  constexpr int D = C::D, G = C::G, BN = C::BN;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::kLdsElems];
  bf16* Ks = smem;
  bf16* Vs = smem + BN * C::kStrideK;

  const int b = blockIdx.z, g = blockIdx.y;
  const int t = gridDim.x - 1 - blockIdx.x;  // longest causal tiles first
  const int seq0 = cu_seqlens[b];
  const int L = cu_seqlens[b + 1] - seq0;
  const int p0 = t * C::kPositions;
  if (p0 >= L) return;
  const int p1 = min(p0 + C::kPositions, L);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const bool windowed = window > 0;

  // This lane's query row.
  const int r = 32 * wave + n;
  const int qpos = p0 + r / G;
  const int qhead = g * G + (r % G);
  const bool qvalid = qpos < L;

  int ss, se;
  // Key range of the workgroup: the window below its first row, the span
  // holding its first row, its last row, the span holding its last row.
  int lo = windowed ? max(0, p0 - window + 1) : 0;
  int hi = p1;
  if (num_spans > 0) {
    if (find_span(spans, num_spans, seq0 + p0, ss, se)) lo = min(lo, max(ss - seq0, 0));
    if (find_span(spans, num_spans, seq0 + p1 - 1, ss, se)) hi = max(hi, min(se - seq0, L));
  }
  // Key range of this wave's rows (used only to skip no-op tiles).
  const int pw0 = p0 + wave * C::kPosPerWave;
  const int pw1 = min(pw0 + C::kPosPerWave, L);
  const bool wave_has_rows = pw0 < L;
  const bool wave_full = pw0 + C::kPosPerWave <= L;
  int lo_w = 0, hi_w = 0;
  if (wave_has_rows) {
    lo_w = windowed ? max(0, pw0 - window + 1) : 0;
    hi_w = pw1;
    if (num_spans > 0) {
      if (find_span(spans, num_spans, seq0 + pw0, ss, se)) lo_w = min(lo_w, max(ss - seq0, 0));
      if (find_span(spans, num_spans, seq0 + pw1 - 1, ss, se)) hi_w = max(hi_w, min(se - seq0, L));
    }
  }
  // This row's own span, sequence-relative (empty when none).
  int my_ss = 0, my_se = 0;
  if (num_spans > 0 && qvalid && find_span(spans, num_spans, seq0 + qpos, ss, se)) {
    my_ss = ss - seq0;
    my_se = min(se - seq0, L);
  }

  // Q^T operand: lane holds q[row][16*s + 8*hh .. +7] for every k-step s.
  bf16x8 qr[C::kSteps];
  {
    const bf16* qrow = q + ((size_t)(seq0 + (qvalid ? qpos : 0)) * hq + qhead) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      bf16x8 x = ld_global_x8(qrow + 16 * s);
      qr[s] = qvalid ? x : bf16x8{};
    }
  }

  f32x16 oacc[C::kDBlk];
#pragma unroll
  for (int db = 0; db < C::kDBlk; ++db) oacc[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  const size_t row_stride = (size_t)hkv * D;
  const bf16* kbase = k + ((size_t)seq0 * hkv + g) * D;
  const bf16* vbase = v + ((size_t)seq0 * hkv + g) * D;
  const int qg = lane >> 4, lg = lane & 15;

  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    // K and V tiles -> LDS, row-major; keys past the sequence end are zero.
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int c = tid + i * C::kThreads;
      const int row = c / C::kChunkPerRow;
      const int col = (c % C::kChunkPerRow) * 8;
      const int key = k0 + row;
      u32x4 kx = u32x4{}, vx = u32x4{};
      if (key < L) {
        kx = *reinterpret_cast<const u32x4*>(kbase + key * row_stride + col);
        vx = *reinterpret_cast<const u32x4*>(vbase + key * row_stride + col);
      }
      *reinterpret_cast<u32x4*>(Ks + row * C::kStrideK + col) = kx;
      *reinterpret_cast<u32x4*>(Vs + row * C::kStrideV + col) = vx;
    }
    __syncthreads();
    if (!wave_has_rows || k0 >= hi_w || k0 + BN <= lo_w) continue;

    // S^T = K Q^T: score block `blk` holds keys k0 + 32*blk + [0, 32).
    f32x16 sacc[C::kSBlk];
#pragma unroll
    for (int blk = 0; blk < C::kSBlk; ++blk) {
      sacc[blk] = f32x16{};
      const bf16* krow = Ks + (32 * blk + n) * C::kStrideK + 8 * hh;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s)
        sacc[blk] = mfma32(ld_lds_x8(krow + 16 * s), qr[s], sacc[blk]);
    }

    // Scale, mask by select, tile max.
    const bool need_mask =
        !(wave_full && k0 + BN - 1 <= pw0 && (!windowed || pw1 - 1 - k0 < window));
    float tmax = kNegInf;
#pragma unroll
    for (int blk = 0; blk < C::kSBlk; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = sacc[blk][i] * c2;
        if (need_mask) {
          const int j = k0 + 32 * blk + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool ok = qvalid && ((j <= qpos && (!windowed || qpos - j < window)) ||
                                     (j >= my_ss && j < my_se));
          x = ok ? x : kNegInf;
        }
        sacc[blk][i] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    HalfPair hp = half_pair(tmax);
    tmax = fmaxf(hp.lo, hp.hi);
    const float m_new = fmaxf(m, tmax);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m - m_new);
    const float msub = (m_new == kNegInf) ? 0.f : m_new;

    // p = exp2(s - m), row sum in register order, P -> bf16 operands.
    float psum = 0.f;
    bf16x8 pb[C::kKK];
#pragma unroll
    for (int blk = 0; blk < C::kSBlk; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(sacc[blk][i] - msub);
        psum += p;
        pb[2 * blk + (i >> 3)][i & 7] = to_bf16(p);
      }
    }
    hp = half_pair(psum);
    psum = hp.lo + hp.hi;
    l = l * alpha + psum;
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::kDBlk; ++db) oacc[db] *= alpha;
    }

    // O^T += V^T P^T.  PV k-step kk covers keys 16*kk + 8*(e/4) + 4*hh + e%4
    // in operand slot e; the transpose read gathers exactly those rows.
#pragma unroll
    for (int kk = 0; kk < C::kKK; ++kk) {
      const bf16* vrow = Vs + (16 * kk + 4 * (qg >> 1) + (lg >> 2)) * C::kStrideV +
                         16 * (qg & 1) + 4 * (lg & 3);
#pragma unroll
      for (int db = 0; db < C::kDBlk; ++db) {
        const bf16x4 lo4 = ld_lds_tr(vrow + 32 * db);
        const bf16x4 hi4 = ld_lds_tr(vrow + 8 * C::kStrideV + 32 * db);
        oacc[db] = mfma32(cat8(lo4, hi4), pb[kk], oacc[db]);
      }
    }
  }

  // Epilogue: o = acc / l (IEEE fp32 division), bf16 RNE, store.
  if (qvalid) {
    bf16* orow = o + ((size_t)(seq0 + qpos) * hq + qhead) * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = to_bf16(oacc[db][4 * gi + e] / l);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * gi) = w;
      }
    }
    if (lse != nullptr && hh == 0)
      lse[(size_t)(seq0 + qpos) * hq + qhead] = (m + fast_log2(l)) * 0.693147180559945309f;
  }
}

template <int D, int G, int BN>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  using C = PrefillCfg<D, G, BN>;
  const int tiles = (a.max_seqlen + C::kPositions - 1) / C::kPositions;
  dim3 grid(tiles, a.hkv, a.batch);
  hipLaunchKernelGGL(prefill_kernel<C>, grid, dim3(C::kThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse,
                     a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2);
  return hipGetLastError();
}

// One kernel instance per (head_dim, group); BN is fixed per instance.
#define INVATTN_PREFILL_TABLE(X) \
  X(64, 1, 64) X(64, 2, 64) X(64, 4, 64) X(64, 8, 64)      \
  X(256, 1, 32) X(256, 2, 32) X(256, 4, 32) X(256, 8, 32)  \
  X(512, 1, 32) X(512, 2, 32) X(512, 4, 32) X(512, 8, 32)

bool prefill_schedule(int d, int group, PrefillSchedule* s) {
#define X(D, G, BN)                                         \
  if (d == D && group == G) {                               \
    *s = PrefillSchedule{128, 128 / G, BN, 256};            \
    return true;                                            \
  }
  INVATTN_PREFILL_TABLE(X)
#undef X
  return false;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.hq / a.hkv;
#define X(D, G, BN) \
  if (a.d == D && group == G) return launch_one<D, G, BN>(a, stream);
  INVATTN_PREFILL_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
