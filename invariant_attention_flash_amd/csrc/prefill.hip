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
//   K and V tiles stream HBM -> LDS with direct loads (global_load_lds,
//   16 B per lane), double-buffered so the next tile lands while this one is
//   computed; rows are stored unpadded with an XOR swizzle of their 16-byte
//   chunks (conflict-free MFMA operand reads).  Keys past the sequence end
//   read the sequence's last row and are masked (p = 0).
//   S^T = K Q^T  on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q in
//                registers), so each lane holds one query's scores;
//   scale by c = fl32(scale*log2 e), mask by select (-inf);
//   online softmax in fp32 with a per-row reference max m: m moves (and the
//                running sum and accumulator are rescaled by 2^(m_old-m_new))
//                only when the tile max exceeds m by more than kRescale, so
//                p = 2^(s*c - m) <= 2^kRescale; the tile max and the row sum
//                reduce inside the lane in register order, then across the
//                lane pair (l, l^32);
//   P -> bf16 (RNE), O^T += V^T P^T on the same MFMA, with V^T read from the
//                row-major LDS tile by the LDS transpose read.
// Every decision (skip a tile, move m, rescale) is a function of the row's
// own sequence, so the bytes of a row never depend on the rest of the batch.
#include "device_common.h"
#include "kernels.h"


namespace invattn {

// Reference-max hysteresis (log2 units): m moves only when a tile max
// exceeds it by more than this.  A fixed constant of the arithmetic.
constexpr float kRescale = 8.0f;



template <int D_, int G_, int BN_, int OCC_, int DSPLIT_>
struct PrefillCfg {
  static constexpr int D = D_, G = G_, BN = BN_, OCC = OCC_, DSPLIT = DSPLIT_;
  static constexpr int kRowBlocks = 4;                 // 32-row blocks per workgroup
  static constexpr int kWaves = kRowBlocks * DSPLIT;   // DSPLIT waves share a row block
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 32 * kRowBlocks;
  static constexpr int kPositions = kRows / G;
  static constexpr int kPosPerBlock = 32 / G;
  static constexpr int DW = D / DSPLIT;   // head-dim slice of one wave
  static constexpr int kChunks = D / 8;   // 16-byte chunks per row
  static constexpr int kTile = BN * D;    // elements per K (or V) tile
  static constexpr int kKVElems = 2 * 2 * kTile;  // two buffers of K and V
  // Partial-score exchange between the waves of a row block: fp32, one
  // 16-float record per lane per wave.
  static constexpr int kXchgFloats = DSPLIT > 1 ? kWaves * 64 * 16 * (BN / 32) : 0;
  static constexpr int kLoads = BN * kChunks / 64 / kWaves;  // direct loads per wave per tensor
  static constexpr int kSteps = DW / 16;  // MFMA k-steps over this wave's head-dim slice
  static constexpr int kSBlk = BN / 32;   // 32-key score blocks per tile
  static constexpr int kDBlk = DW / 32;   // 32-wide output blocks of this wave
  static constexpr int kKK = BN / 16;     // 16-key PV k-steps per tile
  static constexpr int kSwK = kChunks >= 16 ? 15 : kChunks - 1;
  static constexpr int kSwV = kChunks >= 16 ? 14 : kChunks - 2;
  static_assert(BN % 32 == 0 && DW % 32 == 0, "tile shape");
  static_assert(BN * kChunks % (64 * kWaves) == 0, "tile load split");
  static_assert(DSPLIT == 1 || DW / 8 >= 32, "head-dim slices start on a swizzle boundary");
  static_assert(kKVElems * 2 + kXchgFloats * 4 <= 163840, "LDS budget");
};

// Swizzled element offset of logical 16-byte chunk `lc` of LDS row `row`.
template <class C>
__device__ __forceinline__ int k_off(int row, int lc) {
  return row * C::D + ((lc ^ (row & C::kSwK)) << 3);
}
template <class C>
__device__ __forceinline__ int v_off(int row, int lc) {
  return row * C::D + ((lc ^ ((row << 1) & C::kSwV)) << 3);
}

// Direct HBM -> LDS loads of one K and one V tile (keys k0 .. k0+BN-1) into
// buffer `buf`.  Lane offsets (elements, 32-bit; one sequence's K or V stays
// below 4 GiB) are row*stride + swizzled chunk; keys past the sequence end
// clamp to its last row (offset last_row).
template <class C>
__device__ __forceinline__ void issue_tile(bf16* smem, int buf, int k0, uint32_t rs,
                                           uint32_t last_row, const uint32_t* ld_row,
                                           const uint32_t* ld_ck, const uint32_t* ld_cv,
                                           const bf16* kbase, const bf16* vbase, int wave) {
  bf16* ks = smem + buf * 2 * C::kTile;
  bf16* vs = ks + C::kTile;
  const uint32_t base = (uint32_t)k0 * rs;
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    const int cbase = (wave * C::kLoads + i) * 64;
    const uint32_t off = min(base + ld_row[i], last_row);
    __builtin_amdgcn_global_load_lds(kbase + (off + ld_ck[i]), LDS_PTR(void, ks + cbase * 8), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vbase + (off + ld_cv[i]), LDS_PTR(void, vs + cbase * 8), 16, 0, 0);
  }
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::kThreads, C::kThreads),
                          amdgpu_waves_per_eu(C::OCC, C::OCC)))
void prefill_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ v, bf16* __restrict__ o,
                    float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                    const int32_t* __restrict__ spans, int num_spans, int hq, int hkv,
                    int window, float c2) {
  constexpr int D = C::D, G = C::G, BN = C::BN, DW = C::DW;
  __shared__ __attribute__((aligned(1024))) bf16 smem[C::kKVElems + 2 * C::kXchgFloats];
  float* xchg = reinterpret_cast<float*>(smem + C::kKVElems);

  const int b = blockIdx.z, g = blockIdx.y;
  const int t = gridDim.x - 1 - blockIdx.x;  // longest causal tiles first
  const int seq0 = cu_seqlens[b];
  const int L = cu_seqlens[b + 1] - seq0;
  const int p0 = t * C::kPositions;
  if (p0 >= L) return;
  const int p1 = min(p0 + C::kPositions, L);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int rb = wave / C::DSPLIT;   // row block of this wave
  const int dh = wave % C::DSPLIT;   // head-dim slice of this wave
  const int n = lane & 31, hh = lane >> 5;
  const bool windowed = window > 0;
  const int wlim = windowed ? window : 0x7fffffff;

  // This lane's query row.
  const int r = 32 * rb + n;
  const int qpos = p0 + r / G;
  const int qhead = g * G + (r % G);
  const bool qvalid = qpos < L;
  const int qpos_m = qvalid ? qpos : -1;  // an invalid row admits no key

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
  const int pw0 = p0 + rb * C::kPosPerBlock;
  const int pw1 = min(pw0 + C::kPosPerBlock, L);
  const bool wave_has_rows = pw0 < L;
  const bool wave_full = pw0 + C::kPosPerBlock <= L;
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

  const size_t row_stride = (size_t)hkv * D;
  const bf16* kbase = k + ((size_t)seq0 * hkv + g) * D;
  const bf16* vbase = v + ((size_t)seq0 * hkv + g) * D;

  // Direct HBM -> LDS loads of one K and one V tile into buffer `buf`.
  // Lane offsets (elements, 32-bit; one sequence's K or V stays below 4 GiB)
  // are row*stride + swizzled chunk; keys past the sequence end clamp to its
  // last row.
  const uint32_t rs = (uint32_t)row_stride;
  const uint32_t last_row = (uint32_t)(L - 1) * rs;
  uint32_t ld_row[C::kLoads], ld_ck[C::kLoads], ld_cv[C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    const int pch = (wave * C::kLoads + i) * 64 + lane;
    const int row = pch / C::kChunks;
    const int pc = pch % C::kChunks;
    ld_row[i] = (uint32_t)row * rs;
    ld_ck[i] = (uint32_t)((pc ^ (row & C::kSwK)) << 3);
    ld_cv[i] = (uint32_t)((pc ^ ((row << 1) & C::kSwV)) << 3);
  }
  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;
  issue_tile<C>(smem, 0, kt0 * BN, rs, last_row, ld_row, ld_ck, ld_cv, kbase, vbase, wave);

  // Q^T operand: lane holds q[row][16*s + 8*hh .. +7] for every k-step s.
  bf16x8 qr[C::kSteps];
  {
    const bf16* qrow =
        q + ((size_t)(seq0 + (qvalid ? qpos : 0)) * hq + qhead) * D + dh * DW + 8 * hh;
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

  // Per-lane LDS offsets that do not change across tiles.  K: this lane's
  // row is n (+32*blk), logical chunk 2*s + hh, physical chunk
  // (2*s + hh) ^ (n & kSwK) = 2*s ^ kx.  V: the transpose read of this lane
  // starts at row vrow0 (+16*kk, +8), logical chunk 4*db + vc1, physical
  // chunk (4*db + vc1) ^ (2*vrow0 & kSwV) = 4*db ^ vx.
  const int kx = hh ^ (n & C::kSwK);
  const int qg = lane >> 4, lg = lane & 15;
  const int vrow0 = 4 * (qg >> 1) + (lg >> 2);
  const int vx = (2 * (qg & 1) + ((lg & 3) >> 1)) ^ ((vrow0 << 1) & C::kSwV);
  const int vsub = (lg & 1) * 4;

  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * BN;
    const int buf = (kt - kt0) & 1;
    // Tile kt landed once every wave has waited for its own direct loads;
    // after the barrier nobody reads buffer buf^1 any more.
    wait_vmem();
    __syncthreads();
    if (kt + 1 < kt1)
      issue_tile<C>(smem, buf ^ 1, k0 + BN, rs, last_row, ld_row, ld_ck, ld_cv, kbase, vbase, wave);
    const bool active = wave_has_rows && k0 < hi_w && k0 + BN > lo_w;
    const bool need_mask =
        !(wave_full && k0 + BN - 1 <= pw0 && (!windowed || pw1 - 1 - k0 < window));
    const bf16* ks = smem + buf * 2 * C::kTile;
    const bf16* vs = ks + C::kTile;
    {
      // S^T = K Q^T over this wave's head-dim slice: score block `blk` holds
      // keys k0 + 32*blk + [0, 32).
      f32x16 sacc[C::kSBlk];
      if (active) {
#pragma unroll
        for (int blk = 0; blk < C::kSBlk; ++blk) {
          sacc[blk] = f32x16{};
          const bf16* krow = ks + (32 * blk + n) * D + dh * DW;
#pragma unroll
          for (int s = 0; s < C::kSteps; ++s)
            sacc[blk] = mfma32(ld_lds_x8(krow + (((2 * s) ^ kx) << 3)), qr[s], sacc[blk]);
        }
        {
          constexpr int kN = C::kSBlk * C::kSteps, kAhead = 4;
          __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
          for (int i = 0; i < kN - kAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
        }
        if constexpr (C::DSPLIT > 1) {
#pragma unroll
          for (int blk = 0; blk < C::kSBlk; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              xchg[((wave * C::kSBlk + blk) * 16 + i) * 64 + lane] = sacc[blk][i];
        }
      }
      if constexpr (C::DSPLIT > 1) {
        // Full scores = slice 0 + slice 1, added in that order by both waves.
        __syncthreads();
        if (active) {
#pragma unroll
          for (int blk = 0; blk < C::kSBlk; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float other = xchg[(((wave ^ 1) * C::kSBlk + blk) * 16 + i) * 64 + lane];
              sacc[blk][i] = dh == 0 ? sacc[blk][i] + other : other + sacc[blk][i];
            }
        }
      }
      if (!active) continue;

      // Scale, mask by select, tile max.  Interior tiles skip the selects
      // (they would keep every score).
      float tmax = kNegInf;
      if (need_mask) {
#pragma unroll
        for (int blk = 0; blk < C::kSBlk; ++blk) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = k0 + 32 * blk + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool ok =
                ((j <= qpos_m) & (qpos_m - j < wlim)) | ((j >= my_ss) & (j < my_se));
            const float x = ok ? sacc[blk][i] * c2 : kNegInf;
            sacc[blk][i] = x;
            tmax = fmaxf(tmax, x);
          }
        }
      } else {
#pragma unroll
        for (int blk = 0; blk < C::kSBlk; ++blk) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = sacc[blk][i] * c2;
            sacc[blk][i] = x;
            tmax = fmaxf(tmax, x);
          }
        }
      }
      HalfPair hp = half_pair(tmax);
      tmax = fmaxf(hp.lo, hp.hi);
      // Move the reference max only on a jump of more than kRescale.
      const bool move = tmax > m + kRescale || (m == kNegInf && tmax != kNegInf);
      const float m_new = move ? tmax : m;
      const float alpha = move ? fast_exp2(m - m_new) : 1.f;
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
        for (int db = 0; db < C::kDBlk; ++db) scale_acc<C::OCC>(oacc[db], alpha);
      }

      // O^T += V^T P^T.  PV k-step kk covers keys 16*kk + 8*(e/4) + 4*hh + e%4
      // in operand slot e; the transpose read gathers exactly those rows.
#pragma unroll
      for (int kk = 0; kk < C::kKK; ++kk) {
        const bf16* vrow = vs + (16 * kk + vrow0) * D + dh * DW + vsub;
#pragma unroll
        for (int db = 0; db < C::kDBlk; ++db) {
          const int col = ((4 * db) ^ vx) << 3;
          const bf16x4 lo4 = ld_lds_tr(vrow + col);
          const bf16x4 hi4 = ld_lds_tr(vrow + 8 * D + col);
          oacc[db] = mfma32(cat8(lo4, hi4), pb[kk], oacc[db]);
        }
      }
      {
        constexpr int kN = C::kKK * C::kDBlk, kAhead = 3;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 1);
#pragma unroll
        for (int i = 0; i < kN - kAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 1);
      }
    }
  }

  // Epilogue: o = acc / l (IEEE fp32 division), bf16 RNE, store.
  if (qvalid) {
    bf16* orow = o + ((size_t)(seq0 + qpos) * hq + qhead) * D + dh * DW + 4 * hh;
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
    if (lse != nullptr && hh == 0 && dh == 0)
      lse[(size_t)(seq0 + qpos) * hq + qhead] = (m + fast_log2(l)) * 0.693147180559945309f;
  }
}

template <int D, int G, int BN, int OCC, int DSPLIT>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  using C = PrefillCfg<D, G, BN, OCC, DSPLIT>;
  const int tiles = (a.max_seqlen + C::kPositions - 1) / C::kPositions;
  dim3 grid(tiles, a.hkv, a.batch);
  hipLaunchKernelGGL(prefill_kernel<C>, grid, dim3(C::kThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse,
                     a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2);
  return hipGetLastError();
}

// One kernel instance per (head_dim, group): keys per tile, waves per SIMD
// and the head-dim split are fixed per instance.
#define INVATTN_PREFILL_TABLE(X)                                                          \
  X(64, 1, 64, 2, 1) X(64, 2, 64, 2, 1) X(64, 4, 64, 2, 1) X(64, 8, 64, 2, 1)             \
  X(256, 1, 32, 2, 1) X(256, 2, 32, 2, 1) X(256, 4, 32, 2, 1) X(256, 8, 32, 2, 1)         \
  X(512, 1, 32, 2, 2) X(512, 2, 32, 2, 2) X(512, 4, 32, 2, 2) X(512, 8, 32, 2, 2)

bool prefill_schedule(int d, int group, PrefillSchedule* s) {
#define X(D, G, BN, OCC, DSPLIT)                                        \
  if (d == D && group == G) {                                           \
    using C = PrefillCfg<D, G, BN, OCC, DSPLIT>;                        \
    *s = PrefillSchedule{C::kRows, C::kPositions, BN, C::kThreads};     \
    return true;                                                        \
  }
  INVATTN_PREFILL_TABLE(X)
#undef X
  return false;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.hq / a.hkv;
#define X(D, G, BN, OCC, DSPLIT) \
  if (a.d == D && group == G) return launch_one<D, G, BN, OCC, DSPLIT>(a, stream);
  INVATTN_PREFILL_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
