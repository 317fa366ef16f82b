// prefill_wide.hip -- the prefill kernel for head dim 512: 32x32x16 bf16
// MFMAs, each wave pair splitting the head dim (partial scores exchanged
// through LDS).  Same contract and masks as prefill.hip.
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
// the G query heads of one KV head.  Its query rows are ordered
// position-major (row r = position*G + head) and cut into 32-row blocks; a
// wave owns RBW row blocks (and, when DSPLIT = 2, one half of the head dim,
// its partner wave the other half).  A row therefore always lands in the same
// wave, lane and MFMA slot, and visits the same KV tiles in the same ascending
// order, whatever else is in the batch.
//
// Per KV tile (BN keys, ascending):
//   K and V tiles stream HBM -> LDS with direct loads (buffer loads with the
//   LDS bit, 16 B per lane) into a ring of NST stage buffers, so later tiles
//   land while this one is computed; rows are stored unpadded with an XOR
//   swizzle of their 16-byte chunks (conflict-free MFMA operand reads).  Keys
//   past the sequence end land as zeros and are masked (p = 0).
//   S^T = K Q^T  on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, read once
//                and used by every row block of the wave; B = Q in
//                registers), so each lane holds one query's scores; with
//                DSPLIT = 2 each wave of a pair forms the partial sum over its
//                half of the head dim and the pair adds them through LDS in a
//                fixed order (half 0 + half 1);
//   mask by select (-inf) on boundary tiles;
//   online softmax in fp32 with a per-row reference max m (scaled units):
//                m moves (and the running sum and accumulator are rescaled by
//                2^(m_old-m_new)) only when the tile max exceeds m by more than
//                kRescale, so p = 2^(fma(s, c, -m)) <= 2^kRescale, with
//                c = fl32(scale*log2 e); the tile max and the row sum reduce
//                inside the lane in register order, then across the lane pair
//                (l, l^32);
//   P -> bf16 (RNE), O^T += V^T P^T on the same MFMA, with V^T read from the
//                row-major LDS tile by the LDS transpose read (once, used by
//                every row block of the wave).
// Fully masked tiles are exact no-ops for a row (p = 0, alpha = 1), and every
// decision (mask, move m, rescale) is a function of the row's own sequence,
// so the bytes of a row never depend on the rest of the batch.
#include "device_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace invattn {
#ifndef PF_AHEAD_QK
#define PF_AHEAD_QK 3
#endif
#ifndef PF_AHEAD_PV
#define PF_AHEAD_PV 3
#endif

template <int D_, int G_, int BN_, int DSPLIT_, int RBW_, int WAVES_, int NST_, int OCC_>
struct PrefillCfg {
  static constexpr bool kPaged = false;  // contiguous keys (PagedOf<> sets it)
  static constexpr int D = D_, G = G_, BN = BN_, DSPLIT = DSPLIT_, RBW = RBW_, OCC = OCC_;
  static constexpr int kWaves = WAVES_;
  static constexpr int kStages = NST_;                 // K/V tile buffers in flight
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWaveGroups = kWaves / DSPLIT;  // waves sharing row blocks
  static constexpr int kRowBlocks = kWaveGroups * RBW; // 32-row blocks per workgroup
  static constexpr int kRows = 32 * kRowBlocks;
  static constexpr int kPositions = kRows / G;
  static constexpr int kPosPerWave = 32 * RBW / G;
  static constexpr int DW = D / DSPLIT;   // head-dim slice of one wave
  static constexpr int kChunks = D / 8;   // 16-byte chunks per row
  static constexpr int kTile = BN * D;    // elements per K (or V) tile
  static constexpr int kSteps = DW / 16;  // MFMA k-steps over this wave's head-dim slice
  static constexpr int kSBlk = BN / 32;   // 32-key score blocks per tile
  static constexpr int kDBlk = DW / 32;   // 32-wide output blocks of this wave
  static constexpr int kKK = BN / 16;     // 16-key PV k-steps per tile
  // Partial-score exchange of a wave pair: fp32, 16 floats per lane per
  // score block per row block.
  static constexpr int kXchgFloats = DSPLIT > 1 ? kWaves * RBW * kSBlk * 16 * 64 : 0;
  static constexpr int kLoads = BN * kChunks / 64 / kWaves;  // direct loads per wave per tensor
  static constexpr int kSwK = kChunks >= 16 ? 15 : kChunks - 1;
  static constexpr int kSwV = kChunks >= 16 ? 14 : kChunks - 2;
  static_assert(BN % 32 == 0 && DW % 32 == 0, "tile shape");
  static_assert(kWaves % DSPLIT == 0 && 32 % G == 0, "wave map");
  static_assert(BN * kChunks % (64 * kWaves) == 0, "tile load split");
  static_assert(DSPLIT == 1 || DW / 8 >= 32, "head-dim slices start on a swizzle boundary");
  static_assert(kStages == 2 || kStages == 3, "double or triple buffering");
  static_assert(kStages * 2 * kTile * 2 + kXchgFloats * 4 <= 163840, "LDS budget");
};

// Direct HBM -> LDS loads of one K and one V tile (keys k0 .. k0+BN-1) into
// the stage buffer `kv` (K tile, then V tile), through buffer resources that
// span exactly the sequence's rows of this KV head: keys past the sequence
// end land as zeros (and are masked).
template <class C, class KT>
__device__ __forceinline__ void issue_tile(bf16* kv, int kt, const KT& src, int wave,
                                           int lane) {
  u32x4 krs, vrs;
  int k0;
  src.get(kt, true, wave, krs, vrs, k0);
  const uint32_t rs_bytes = src.rs_bytes;
  const uint32_t kl = lds_addr(kv), vl = lds_addr(kv + C::kTile);
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(kl, krs, k0, i, rs_bytes, wave, lane);
    dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(vl, vrs, k0, i, rs_bytes, wave, lane);
  }
}

// Per-lane constants of the tile computation.
template <class C>
struct Lane {
  int lane, wave, n, hh, dh;
  int kx;                 // K operand: physical chunk of k-step s is 2*s ^ kx
  int vrow0, vx, vsub;    // V transpose read: row, chunk xor, in-chunk offset
  int wlim;               // window (or a huge value for global layers)
  float c2;               // fl32(scale * log2 e)
  int qpos_m[C::RBW];     // row position (-1 for rows past the sequence end)
  int my_ss[C::RBW], my_se[C::RBW];  // the row's own span (empty when none)
};

// One KV tile (keys k0 .. k0+BN-1) for the rows of this wave: scores,
// online softmax, P.V.  ks/vs: the stage buffer holding the tile.
template <class C>
__device__ __forceinline__ void compute_tile(const bf16* __restrict__ ks,
                                             const bf16* __restrict__ vs, float* xchg, int k0,
                                             bool need_mask, const Lane<C>& ln,
                                             const bf16x8 (*qr)[C::kSteps],
                                             f32x16 (*oacc)[C::kDBlk], float* m, float* l) {
  constexpr int D = C::D, DW = C::DW, RBW = C::RBW;
  const int lane = ln.lane, wave = ln.wave, hh = ln.hh, dh = ln.dh;
  // S^T = K Q^T over this wave's head-dim slice: score block `blk` holds keys
  // k0 + 32*blk + [0, 32); each K operand read serves every row block.
  f32x16 sacc[RBW][C::kSBlk];
#pragma unroll
  for (int blk = 0; blk < C::kSBlk; ++blk) {
#pragma unroll
    for (int r = 0; r < RBW; ++r) sacc[r][blk] = f32x16{};
    const bf16* krow = ks + (32 * blk + ln.n) * D + dh * DW;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      const bf16x8 kop = ld_lds_x8(krow + (((2 * s) ^ ln.kx) << 3));
#pragma unroll
      for (int r = 0; r < RBW; ++r) sacc[r][blk] = mfma32(kop, qr[r][s], sacc[r][blk]);
    }
  }
  {
    constexpr int kN = C::kSBlk * C::kSteps, kAhead = PF_AHEAD_QK;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < kN - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, RBW, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RBW * kAhead, 0);
  }
  if constexpr (C::DSPLIT > 1) {
    // Full scores = slice 0 + slice 1, added in that order by both waves.
    constexpr int kRec = RBW * C::kSBlk * 16;
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
      for (int blk = 0; blk < C::kSBlk; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xchg[(wave * kRec + (r * C::kSBlk + blk) * 16 + i) * 64 + lane] = sacc[r][blk][i];
    lds_barrier();
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
      for (int blk = 0; blk < C::kSBlk; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float other = xchg[((wave ^ 1) * kRec + (r * C::kSBlk + blk) * 16 + i) * 64 + lane];
          sacc[r][blk][i] = dh == 0 ? sacc[r][blk][i] + other : other + sacc[r][blk][i];
        }
  }

  // Mask by select (raw scores) on boundary tiles.
  if (need_mask) {
#pragma unroll
    for (int r = 0; r < RBW; ++r)
#pragma unroll
      for (int blk = 0; blk < C::kSBlk; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = k0 + 32 * blk + 8 * (i >> 2) + 4 * hh + (i & 3);
          const int qp = ln.qpos_m[r];
          const bool ok = ((j <= qp) & (qp - j < ln.wlim)) | ((j >= ln.my_ss[r]) & (j < ln.my_se[r]));
          sacc[r][blk][i] = ok ? sacc[r][blk][i] : kNegInf;
        }
  }

  bf16x8 pb[RBW][C::kKK];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    // Tile max of the raw scores; the scaled max is fl(max * c) (rounding is
    // monotone, so it equals the max of the scaled scores).
    float tmax = kNegInf;
#pragma unroll
    for (int blk = 0; blk < C::kSBlk; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[r][blk][i]);
    HalfPair hp = half_pair(tmax);
    tmax = fmaxf(hp.lo, hp.hi) * ln.c2;
    // Move the reference max only on a jump of more than kRescale.
    const bool move = tmax > m[r] + kRescale || (m[r] == kNegInf && tmax != kNegInf);
    const float m_new = move ? tmax : m[r];
    const float alpha = move ? fast_exp2(m[r] - m_new) : 1.f;
    const float msub = (m_new == kNegInf) ? 0.f : m_new;
    // p = exp2(fma(s, c, -m)), row sum in register order, P -> bf16 operands.
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < C::kSBlk; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sacc[r][blk][i], ln.c2, -msub));
        psum += p;
        pb[r][2 * blk + (i >> 3)][i & 7] = to_bf16(p);
      }
    }
    hp = half_pair(psum);
    psum = hp.lo + hp.hi;
    l[r] = l[r] * alpha + psum;
    m[r] = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::kDBlk; ++db) scale_acc<C::OCC>(oacc[r][db], alpha);
    }
  }

  // O^T += V^T P^T.  PV k-step kk covers keys 16*kk + 8*(e/4) + 4*hh + e%4 in
  // operand slot e; the transpose read gathers exactly those rows.
#pragma unroll
  for (int kk = 0; kk < C::kKK; ++kk) {
    const bf16* vrow = vs + (16 * kk + ln.vrow0) * D + dh * DW + ln.vsub;
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db) {
      const int col = ((4 * db) ^ ln.vx) << 3;
      const bf16x8 vop = cat8(ld_lds_tr(vrow + col), ld_lds_tr(vrow + 8 * D + col));
#pragma unroll
      for (int r = 0; r < RBW; ++r) oacc[r][db] = mfma32(vop, pb[r][kk], oacc[r][db]);
    }
  }
  {
    constexpr int kN = C::kKK * C::kDBlk, kAhead = PF_AHEAD_PV;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 1);
#pragma unroll
    for (int i = 0; i < kN - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, RBW, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RBW * kAhead, 1);
  }
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::kThreads, C::kThreads),
                          amdgpu_waves_per_eu(C::OCC, C::OCC)))
void prefill_wide_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ v, bf16* __restrict__ o,
                    float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                    const int32_t* __restrict__ spans, int num_spans, int hq, int hkv,
                    int window, float c2, PagedKv pk) {
  constexpr int D = C::D, G = C::G, BN = C::BN, DW = C::DW, RBW = C::RBW;
  // One LDS object per pipeline stage (K tile then V tile), so the compiler
  // can tell that direct loads into one stage never alias reads of another.
  __shared__ __attribute__((aligned(1024))) bf16 kv0[2 * C::kTile];
  __shared__ __attribute__((aligned(1024))) bf16 kv1[2 * C::kTile];
  __shared__ __attribute__((aligned(1024))) bf16 kv2[C::kStages > 2 ? 2 * C::kTile : 8];
  __shared__ __attribute__((aligned(16))) float xchg[C::kXchgFloats > 0 ? C::kXchgFloats : 4];

  // Tile t covers positions [t*P, (t+1)*P), counted from the first tile
  // holding a query row of the sequence; longest causal tiles first.
  const int b = blockIdx.z, g = blockIdx.y;
  constexpr bool PAGED = C::kPaged;
  const SeqGeo sg = seq_geo<PAGED>(cu_seqlens, pk, b);
  const int L = sg.L;
  const int seq0 = sg.qbase;  // packed row of position 0 (q / o / lse, spans)
  const int t = sg.qlo / C::kPositions + (int)(gridDim.x - 1 - blockIdx.x);
  const int p0 = t * C::kPositions;
  if (p0 >= sg.qhi) return;
  const int p1 = min(p0 + C::kPositions, sg.qhi);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wg = wave / C::DSPLIT;  // wave group (shares row blocks)
  const int dh = wave % C::DSPLIT;  // head-dim slice of this wave
  const int n = lane & 31, hh = lane >> 5;
  const bool windowed = window > 0;

  int ss, se;
  // Key range of the workgroup: the window below its first row, the span
  // holding its first row, its last row, the span holding its last row.
  int lo = windowed ? max(0, p0 - window + 1) : 0;
  int hi = p1;
  if (num_spans > 0) {
    if (find_span(spans, num_spans, seq0 + p0, ss, se)) lo = min(lo, max(ss - seq0, 0));
    if (find_span(spans, num_spans, seq0 + p1 - 1, ss, se)) hi = max(hi, min(se - seq0, L));
  }
  // Positions of this wave's rows (masks are needed on tiles that are not
  // fully allowed for every one of them).
  const int pw0 = p0 + wg * C::kPosPerWave;
  const int pw1 = min(pw0 + C::kPosPerWave, sg.qhi);
  const bool wave_full = pw0 >= sg.qlo && pw0 + C::kPosPerWave <= sg.qhi;

  Lane<C> ln;
  ln.lane = lane;
  ln.wave = wave;
  ln.n = n;
  ln.hh = hh;
  ln.dh = dh;
  ln.kx = hh ^ (n & C::kSwK);
  {
    // V transpose read of this lane: row vrow0 (+16*kk, +8), logical chunk
    // 4*db + c1, physical chunk (4*db + c1) ^ (2*vrow0 & kSwV) = 4*db ^ vx.
    const int qg = lane >> 4, lg = lane & 15;
    ln.vrow0 = 4 * (qg >> 1) + (lg >> 2);
    ln.vx = (2 * (qg & 1) + ((lg & 3) >> 1)) ^ ((ln.vrow0 << 1) & C::kSwV);
    ln.vsub = (lg & 1) * 4;
  }
  ln.wlim = windowed ? window : 0x7fffffff;
  ln.c2 = c2;
  int qpos[RBW], qhead[RBW];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    const int row = 32 * (wg * RBW + r) + n;
    qpos[r] = p0 + row / G;
    qhead[r] = g * G + row % G;
    const bool valid = qpos[r] >= sg.qlo && qpos[r] < sg.qhi;
    ln.qpos_m[r] = valid ? qpos[r] : -1;  // an invalid row admits no key
    ln.my_ss[r] = 0;
    ln.my_se[r] = 0;
    if (num_spans > 0 && valid && find_span(spans, num_spans, seq0 + qpos[r], ss, se)) {
      ln.my_ss[r] = ss - seq0;
      ln.my_se[r] = min(se - seq0, L);
    }
  }

  // This KV head's rows of the sequence, loaded through buffer resources of
  // exactly that extent (the host rejects inputs whose rows span 2 GiB or
  // more), or its cache blocks.
  const KvTiles<PAGED> src = kv_tiles<D, PAGED>(k, v, pk, sg, b, g, hkv, window);
  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;
  issue_tile<C>(kv0, kt0, src, wave, lane);
  if (C::kStages > 2 && kt0 + 1 < kt1) issue_tile<C>(kv1, kt0 + 1, src, wave, lane);

  // Q^T operands: lane holds q[row][dh*DW + 16*s + 8*hh .. +7] for every s.
  bf16x8 qr[RBW][C::kSteps];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    const bool valid = ln.qpos_m[r] >= 0;
    const bf16* qrow =
        q + ((size_t)(seq0 + (valid ? qpos[r] : sg.qlo)) * hq + qhead[r]) * D + dh * DW + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      bf16x8 x = ld_global_x8(qrow + 16 * s);
      qr[r][s] = valid ? x : bf16x8{};
    }
  }

  f32x16 oacc[RBW][C::kDBlk];
  float m[RBW], l[RBW];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db) oacc[r][db] = f32x16{};
  }

  // One step: wait for tile kt (later tiles may stay in flight), barrier
  // (after it nobody reads the buffer of tile kt-1), prefetch tile
  // kt + kStages - 1 into `pre` (the buffer of tile kt-1), compute tile kt
  // from `cur`.  The loop is unrolled by the stage count so every buffer is a
  // distinct LDS object at every step.
  auto step = [&] __device__(const bf16* cur, bf16* pre, int kt) {
    const int k0 = kt * BN;
    if (kt + C::kStages - 2 < kt1) wait_vmem_keep<C::kStages - 2>(2 * C::kLoads);
    else wait_vmem();
    lds_barrier();
    if (kt + C::kStages - 1 < kt1)
      issue_tile<C>(pre, kt + C::kStages - 1, src, wave, lane);
    const bool need_mask =
        !(wave_full && k0 + BN - 1 <= pw0 && (!windowed || pw1 - 1 - k0 < window));
    compute_tile<C>(cur, cur + C::kTile, xchg, k0, need_mask, ln, qr, oacc, m, l);
  };
  for (int kt = kt0; kt < kt1;) {
    step(kv0, C::kStages == 2 ? kv1 : kv2, kt++);
    if (kt >= kt1) break;
    step(kv1, kv0, kt++);
    if (kt >= kt1) break;
    if constexpr (C::kStages == 3) {
      step(kv2, kv1, kt++);
      if (kt >= kt1) break;
    }
  }

  // Epilogue: o = acc / l (IEEE fp32 division), bf16 RNE, store.
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    if (ln.qpos_m[r] < 0) continue;
    bf16* orow = o + ((size_t)(seq0 + qpos[r]) * hq + qhead[r]) * D + dh * DW + 4 * hh;
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = to_bf16(oacc[r][db][4 * gi + e] / l[r]);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * gi) = w;
      }
    }
    if (lse != nullptr && hh == 0 && dh == 0)
      lse[(size_t)(seq0 + qpos[r]) * hq + qhead[r]] =
          (m[r] + fast_log2(l[r])) * 0.693147180559945309f;
  }
}

template <class C>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  const int tiles = prefill_grid_tiles(a, C::kPositions);
  dim3 grid(tiles, a.hkv, a.batch);
  const PagedKv pk{a.q_start, a.block_table, a.max_blocks, a.num_blocks, a.max_context};
  if (a.q_start != nullptr)
    hipLaunchKernelGGL(prefill_wide_kernel<PagedOf<C>>, grid, dim3(C::kThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse,
                       a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2, pk);
  else
    hipLaunchKernelGGL(prefill_wide_kernel<C>, grid, dim3(C::kThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse,
                       a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2, pk);
  return hipGetLastError();
}

// One kernel instance per (head_dim, group).  Parameters after (D, G): keys
// per tile, head-dim split, row blocks per wave, waves, stages, waves per
// SIMD.  All fixed per instance.
#ifndef PF_CFG512
#define PF_CFG512 32, 2, 1, 4, 2, 1
#endif
#define INVATTN_PREFILL_WIDE_TABLE(X)                                         \
  X(512, 1, PF_CFG512) X(512, 2, PF_CFG512) X(512, 4, PF_CFG512)              \
  X(512, 8, PF_CFG512)

bool prefill_wide_schedule(int d, int group, PrefillSchedule* s) {
#define X(D, G, ...)                                                          \
  if (d == D && group == G) {                                                 \
    using C = PrefillCfg<D, G, __VA_ARGS__>;                                  \
    *s = PrefillSchedule{C::kRows, C::kPositions, C::BN, C::kThreads};        \
    return true;                                                              \
  }
  INVATTN_PREFILL_WIDE_TABLE(X)
#undef X
  return false;
}

hipError_t launch_prefill_wide(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.hq / a.hkv;
#define X(D, G, ...) \
  if (a.d == D && group == G) return launch_one<PrefillCfg<D, G, __VA_ARGS__>>(a, stream);
  INVATTN_PREFILL_WIDE_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
