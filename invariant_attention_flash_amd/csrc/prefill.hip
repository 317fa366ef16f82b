// prefill.hip -- batch-invariant attention forward over packed
// variable-length sequences (sliding-window and global layers, GQA,
// bidirectional spans), bf16 MFMA on gfx950.  Head dim 64 runs the kernel
// below; head dims 256 and 512 run prefill_ws.hip.
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
// Work map.  A workgroup (4 waves, one per SIMD) owns `positions`
// consecutive positions of ONE sequence, aligned to the sequence start, for
// the G query heads of one KV head.  Its rows are ordered position-major
// (row = position*G + head); wave w owns rows [16*RB*w, 16*RB*(w+1)) as RB
// blocks of 16.  A row therefore always lands in the same wave, lane and
// MFMA slot and visits the same KV tiles in the same ascending order,
// whatever else is in the batch.
//
// Operand reuse.  Every K and V operand read from LDS feeds RB MFMAs (one
// per row block), so LDS traffic per MFMA falls as RB grows; RB is bounded by
// the accumulators: O (D/16 blocks of 4 fp32 per row block) and two tiles of
// scores stay in the 256 accumulation registers of the wave.
//
// Per KV tile of 32 keys (ascending), software-pipelined by one tile:
//   K and V tiles stream HBM -> LDS with direct loads (16 B per lane) into a
//   ring of NST stage buffers (distinct LDS objects), issued NST-1 tiles
//   ahead; rows are stored unpadded with an XOR swizzle of their 16-byte
//   chunks.  Keys past the sequence end load as zeros and are masked.
//   S^T(t+1) = K Q^T on v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 head-dim
//               elements from LDS, B = Q^T in registers): lane l holds keys
//               4*(l/16) + i of query row l%16, for 16-key halves kb = 0, 1;
//   meanwhile the softmax of tile t (fp32, raw scores masked by select on
//               boundary tiles):
//               reference max m (scaled units) moves only when the tile max
//               exceeds it by more than kRescale; then the running sum and
//               the accumulator are scaled by 2^(m_old - m_new);
//               p = 2^(fma(s, c, -m)), c = fl32(scale * log2 e);
//               tile max and row sum reduce in-lane in slot order (kb, i),
//               then across lanes l^32 and l^16, each step adding (lower
//               lane's value) + (upper lane's value);
//   O^T += V^T P^T on the same MFMA: P^T (bf16, round to nearest even) is
//               the lane's own 8 probabilities, k-slot 8*(l/16) + s meaning
//               key 16*(s/4) + 4*(l/16) + s%4; V^T comes from the row-major
//               LDS tile through the transpose read.
// Fully masked tiles are exact no-ops for a row (p = 0, alpha = 1), and every
// decision (mask, moving m, rescaling) is a function of the row's own
// sequence, so the bytes of a row never depend on the rest of the batch.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace invattn {

template <int D_, int G_, int RB_, int NST_>
struct Pf16Cfg {
  static constexpr bool kPaged = false;  // contiguous keys (PagedOf<> sets it)
  static constexpr int D = D_, G = G_, RB = RB_, NST = NST_;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BN = 32;                       // keys per KV tile
  static constexpr int kRowsPerWave = 16 * RB;
  static constexpr int kRows = kWaves * kRowsPerWave;
  static constexpr int kPositions = kRows / G;
  static constexpr int kPosPerWave = kRowsPerWave / G;
  static constexpr int kSt = D / 32;       // QK k-steps (32 head-dim elements)
  static constexpr int kDb = D / 16;       // PV output blocks (16 head-dim elements)
  static constexpr int kChunks = D / 8;    // 16-byte chunks per row
  static constexpr int kTile = BN * D;     // elements of one K (or V) tile
  static constexpr int kLoads = BN * kChunks / (64 * kWaves);  // per lane per tensor
  static constexpr int kSwK = kChunks >= 16 ? 15 : kChunks - 1;
  static constexpr int kSwV = kChunks >= 16 ? 14 : kChunks - 2;
  static_assert(D % 32 == 0 && kRowsPerWave % G == 0, "row map");
  static_assert(kLoads >= 1 && BN * kChunks % (64 * kWaves) == 0, "tile load split");
  static_assert(NST == 5, "stage ring: tiles t-1 .. t+3");
  static_assert(NST * 2 * kTile * 2 <= 163840, "LDS budget");
  static_assert(RB * kDb * 4 + 2 * RB * 8 <= 256, "accumulators fit the AGPR file");
};


// Load j of this lane's 2*kLoads direct loads of one tile into a stage
// buffer (even j: K rows through krs, odd j: V rows through vrs, after the
// K tile); k0: the row offset of KvTiles::get.
template <class C>
__device__ __forceinline__ void dma_load(bf16* __restrict__ kv, const u32x4& krs,
                                         const u32x4& vrs, int k0, int j, uint32_t rs_bytes,
                                         int wave, int lane) {
  if ((j & 1) == 0)
    dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(lds_addr(kv), krs, k0, j >> 1, rs_bytes, wave,
                                                 lane);
  else
    dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(lds_addr(kv + C::kTile), vrs, k0, j >> 1,
                                                 rs_bytes, wave, lane);
}

template <class C, class KT>
__device__ __forceinline__ void issue16(bf16* __restrict__ kv, const KT& src, int kt,
                                        bool live, int wave, int lane) {
  u32x4 krs, vrs;
  int k0;
  src.get(kt, live, wave, krs, vrs, k0);
#pragma unroll
  for (int j = 0; j < 2 * C::kLoads; ++j)
    dma_load<C>(kv, krs, vrs, k0, j, src.rs_bytes, wave, lane);
}

// One pipelined tile step: S^T(t+1) = K Q^T on the K tile `ks` and
// (PV) O^T += V^T P^T(t-1) on the V tile `vs`, on 16x16x32 MFMAs; the
// softmax VALU of tile t (formed by the caller in the same block) fills the
// MFMA shadow.  FIRST: the step forming the first PV product, which starts
// the accumulator (zero addend) instead of adding to it.
//   K operand (k-step st, half kb): key row 16*kb + x, logical chunk
//     4*st + gq, physical chunk (4*st + gq) ^ (x & kSwK);
//   V operand (output block db): rows 4*gq + x/4 and +16, logical chunk
//     2*db + (x%4)/2, physical chunk ^ ((2*row) & kSwV), element 4*(x%2).
template <class C, bool PV, bool FIRST, bool DMA>
__device__ __forceinline__ void mfma_phase(const bf16* __restrict__ ks,
                                           const bf16* __restrict__ vs, bf16* __restrict__ pre,
                                           const u32x4& krs, const u32x4& vrs, int nk0,
                                           uint32_t rs_bytes, int wave,
                                           int lane, uint32_t krow, uint32_t kq16, uint32_t vrow,
                                           uint32_t vc16, const bf16x8 (*q)[C::kSt],
                                           f32x4 (*s)[2], const bf16x8* pprev,
                                           f32x4 (*o)[C::kDb]) {
  constexpr int kN = 2 * C::kSt;  // K operand groups = V operand groups (= D/16)
  static_assert(kN == C::kDb, "one K group per V group");
  const char* kb0 = reinterpret_cast<const char*>(ks) + krow;
  const char* vb0 = reinterpret_cast<const char*>(vs) + vrow;
  auto kread = [&](int i) {
    return ld_lds_x8(reinterpret_cast<const bf16*>(
        kb0 + (kq16 ^ (uint32_t)((i >> 1) << 6)) + (i & 1) * 32 * C::D));
  };
  auto vread = [&](int i) {
    const bf16* p = reinterpret_cast<const bf16*>(vb0 + (vc16 ^ (uint32_t)(i << 5)));
    return cat8(ld_lds_tr(p), ld_lds_tr(p + 16 * C::D));
  };
  // LDS reads run kAhead groups ahead of their MFMAs.  The order of reads
  // and MFMAs is pinned by scheduling fences that only VALU and SALU
  // instructions may cross, so the softmax VALU fills the gaps while the
  // reads stay early.
  constexpr int kAhead = 3;
  bf16x8 kop[kAhead], vop[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    kop[i] = kread(i);
    if constexpr (PV) vop[i] = vread(i);
  }
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) s[rb][0] = s[rb][1] = f32x4{};
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const int st = i >> 1, kb = i & 1;
    const bf16x8 a = kop[i % kAhead];
    bf16x8 b;
    if constexpr (PV) b = vop[i % kAhead];
    if (i + kAhead < kN) {
      kop[i % kAhead] = kread(i + kAhead);
      if constexpr (PV) vop[i % kAhead] = vread(i + kAhead);
    }
    // The next tile's loads (into `pre`) are spread over the groups.
    if constexpr (DMA) {
      constexpr int kEvery = kN / (2 * C::kLoads);
      if (i % kEvery == 0)
        dma_load<C>(pre, krs, vrs, nk0, i / kEvery, rs_bytes, wave, lane);
    }
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) s[rb][kb] = mfma16(a, q[rb][st], s[rb][kb]);
    if constexpr (PV) {
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
        o[rb][i] = mfma16(b, pprev[rb], FIRST ? f32x4{} : o[rb][i]);
    }
    __builtin_amdgcn_sched_barrier(0x0006);
  }
}

// O^T += V^T P^T for the last tile (no scores left to form).
template <class C, bool FIRST>
__device__ __forceinline__ void pv_last(const bf16* __restrict__ vs, uint32_t vrow, uint32_t vc16,
                                        const bf16x8* pprev, f32x4 (*o)[C::kDb]) {
  const char* vb0 = reinterpret_cast<const char*>(vs) + vrow;
#pragma unroll
  for (int db = 0; db < C::kDb; ++db) {
    const bf16* p = reinterpret_cast<const bf16*>(vb0 + (vc16 ^ (uint32_t)(db << 5)));
    const bf16x8 b = cat8(ld_lds_tr(p), ld_lds_tr(p + 16 * C::D));
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
      o[rb][db] = mfma16(b, pprev[rb], FIRST ? f32x4{} : o[rb][db]);
  }
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::kThreads, C::kThreads),
                          amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ v, bf16* __restrict__ o,
                    float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                    const int32_t* __restrict__ spans, int num_spans, int hq, int hkv,
                    int window, float c2, int tiles, int nseq, PagedKv pk) {
  constexpr int D = C::D, G = C::G, RB = C::RB, BN = C::BN, NST = C::NST;
  // Stage ring: NST buffers of (K tile, V tile); tile kt lives in buffer
  // (kt - kt0) % NST.  While step kt runs, tiles kt-1 (V read), kt, kt+1 (K
  // read), kt+2 (landing) and kt+3 (issued) occupy the five buffers.
  __shared__ __attribute__((aligned(1024))) bf16 kvs[NST][2 * C::kTile];

  // Item = (tile, KV head, sequence) in run-major order (kernels.h); tiles
  // are numbered from the end of the sequence (longest causal rows first).
  int tile;
  long long grp;
  if (!run_major_item(blockIdx.x, tiles, (long long)hkv * nseq, tile, grp)) return;
  const int g = (int)(grp % hkv);
  const int b = (int)(grp / hkv);
  constexpr bool PAGED = C::kPaged;
  const SeqGeo sg = seq_geo<PAGED>(cu_seqlens, pk, b);
  const int L = sg.L;
  const int t = sg.qlo / C::kPositions + tiles - 1 - tile;
  const int p0 = t * C::kPositions;
  if (p0 >= sg.qhi) return;
  const int p1 = min(p0 + C::kPositions, sg.qhi);
  const int seq0 = sg.qbase;  // packed row of position 0 (q / o / lse, spans)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
  // Positions of this wave's rows (a tile needs masks unless it is fully
  // allowed for every one of them).
  const int pw0 = p0 + wave * C::kPosPerWave;
  const int pw1 = min(pw0 + C::kPosPerWave, sg.qhi);
  const bool wave_full = pw0 >= sg.qlo && pw0 + C::kPosPerWave <= sg.qhi;

  Lane16 ln;
  ln.x = lane & 15;
  ln.gq = lane >> 4;
  ln.krow = (uint32_t)(ln.x * D * 2);
  ln.kq16 = (uint32_t)((ln.gq ^ (ln.x & C::kSwK)) << 4);
  {
    const int y = ln.x, vr = 4 * ln.gq + (y >> 2);
    ln.vrow = (uint32_t)(vr * D * 2 + 8 * (y & 1));
    ln.vc16 = (uint32_t)((((y & 3) >> 1) ^ ((2 * vr) & C::kSwV)) << 4);
  }
  ln.wlim = windowed ? window : 0x7fffffff;
  ln.c2 = c2;

  int qpos[RB], qhead[RB], my_ss[RB], my_se[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = C::kRowsPerWave * wave + 16 * rb + ln.x;
    const int pos = p0 + row / G;
    qhead[rb] = g * G + row % G;
    const bool valid = pos >= sg.qlo && pos < sg.qhi;
    qpos[rb] = valid ? pos : -1;  // an invalid row admits no key
    my_ss[rb] = 0;
    my_se[rb] = 0;
    if (num_spans > 0 && valid && find_span(spans, num_spans, seq0 + pos, ss, se)) {
      my_ss[rb] = ss - seq0;
      my_se[rb] = min(se - seq0, L);
    }
  }

  // Q^T operands: lane holds q[row][32*st + 8*gq .. +7] for every st.  Rows
  // outside the sequence's query positions load its first query row instead;
  // every key is masked for them (qpos = -1) and they are never stored.
  bf16x8 qr[RB][C::kSt];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bf16* qrow =
        q + ((size_t)(seq0 + (qpos[rb] >= 0 ? qpos[rb] : sg.qlo)) * hq + qhead[rb]) * D +
        8 * ln.gq;
#pragma unroll
    for (int st = 0; st < C::kSt; ++st) qr[rb][st] = ld_global_x8(qrow + 32 * st);
  }

  const uint32_t rs_bytes = (uint32_t)hkv * D * 2;
  // This KV head's keys, loaded through buffer resources of exactly their
  // extent: the sequence's rows (contiguous layout; the host rejects inputs
  // whose rows span 2 GiB or more) or one cache block per half tile (paged).
  static_assert(BN == 32 && C::kWaves == 4, "KvTiles: wave w loads tile rows [8w, 8w+8)");
  const KvTiles<PAGED> src = kv_tiles<D, PAGED>(k, v, pk, sg, b, g, hkv, window);
  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;
  constexpr int kPerTile = 2 * C::kLoads;  // direct loads per lane per tile

  // Accumulators: O starts at the first PV product (zero addend).
  f32x4 oacc[RB][C::kDb];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
  }

  // Prologue: tiles kt0 .. kt0+2 in flight; wait for Q and tile kt0.
  issue16<C>(kvs[0], src, kt0, true, wave, lane);
  issue16<C>(kvs[1], src, kt0 + 1, kt0 + 1 < kt1, wave, lane);
  issue16<C>(kvs[2], src, kt0 + 2, kt0 + 2 < kt1, wave, lane);
  wait_vmcnt<2 * kPerTile>();
  lds_barrier();

  // Scores and probabilities of consecutive tiles alternate between two
  // arrays each (steps are unrolled by two), so nothing is copied.
  f32x4 sa[RB][2], sb[RB][2];
  bf16x8 pa[RB], pbb[RB];
  const u32x4 no_rs{};
  mfma_phase<C, false, false, false>(kvs[0], kvs[0], kvs[1], no_rs, no_rs, 0, rs_bytes, wave, lane,
                                     ln.krow, ln.kq16, ln.vrow, ln.vc16, qr, sa, pa, oacc);

  // Step kt: wait for tile kt+1, then S(kt+1) and PV(kt-1) on the MFMAs,
  // the loads of tile kt+3 spread among them (into the buffer of tile kt-2,
  // free once every wave is past the barrier), while the VALU takes the
  // softmax of tile kt; the
  // rare reference-max moves are handled after the MFMAs are issued.  After
  // the last tile the scores formed are never used (the K buffer holds an
  // older tile); forming them keeps the step branch-free.  MODE 0: first
  // tile (no PV yet); 1: first PV (starts O); 2: steady state.
  auto step = [&] __device__(int kt, f32x4(&sc)[RB][2], f32x4(&sn)[RB][2], bf16x8(&pc)[RB],
                             const bf16x8(&pp)[RB], auto mode) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool PV = MODE > 0, FIRST = MODE == 1;
    const int r = (kt - kt0) % NST;
    const bf16* __restrict__ kbuf = kvs[(r + 1) % NST];
    const bf16* __restrict__ vbuf = kvs[(r + NST - 1) % NST] + C::kTile;  // V tile of kt-1
    bf16* __restrict__ pre = kvs[(r + 3) % NST];
    const int k0 = kt * BN;
    // Tile kt+1 must have landed; tile kt+2 may still be in flight (every
    // step issues one tile's loads, real or zero-length).
    wait_vmcnt<kPerTile>();
    lds_barrier();
    u32x4 nkrs, nvrs;
    int nk0;
    src.get(kt + 3, kt + 3 < kt1, wave, nkrs, nvrs, nk0);
    const bool need_mask =
        !(wave_full && k0 + BN - 1 <= pw0 && (!windowed || pw1 - 1 - k0 < window));
    const uint32_t kq16 = opaque(ln.kq16), vc16 = opaque(ln.vc16);
    // Scale the accumulator blocks whose rows moved their reference max
    // (after PV(kt-1) is in: it belongs to the old reference).
    float alpha[RB];
    auto rescale = [&](uint32_t mask) {
      if constexpr (PV) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if (mask & (1u << rb)) {
#pragma unroll
            for (int db = 0; db < C::kDb; ++db) oacc[rb][db] *= alpha[rb];
          }
      }
    };
    if (need_mask) {
      const bool moved = softmax_fast<RB, true>(sc, k0, ln, qpos, my_ss, my_se, m, l, pc);
      mfma_phase<C, PV, FIRST, true>(kbuf, vbuf, pre, nkrs, nvrs, nk0, rs_bytes, wave, lane,
                                     ln.krow, kq16, ln.vrow, vc16, qr, sn, pp, oacc);
      if (moved) rescale(softmax_move<RB, true>(sc, k0, ln, qpos, my_ss, my_se, m, l, pc, alpha));
    } else {
      const bool moved = softmax_fast<RB, false>(sc, k0, ln, qpos, my_ss, my_se, m, l, pc);
      mfma_phase<C, PV, FIRST, true>(kbuf, vbuf, pre, nkrs, nvrs, nk0, rs_bytes, wave, lane,
                                     ln.krow, kq16, ln.vrow, vc16, qr, sn, pp, oacc);
      if (moved) rescale(softmax_move<RB, false>(sc, k0, ln, qpos, my_ss, my_se, m, l, pc, alpha));
    }
  };
  using Mode0 = std::integral_constant<int, 0>;
  using Mode1 = std::integral_constant<int, 1>;
  using Mode2 = std::integral_constant<int, 2>;
  step(kt0, sa, sb, pa, pbb, Mode0{});
  if (kt0 + 1 < kt1) step(kt0 + 1, sb, sa, pbb, pa, Mode1{});
  int kt = kt0 + 2;
  for (; kt + 1 < kt1; kt += 2) {
    step(kt, sa, sb, pa, pbb, Mode2{});
    step(kt + 1, sb, sa, pbb, pa, Mode2{});
  }
  if (kt < kt1) {
    step(kt, sa, sb, pa, pbb, Mode2{});
    pv_last<C, false>(kvs[(kt - kt0) % NST] + C::kTile, ln.vrow, ln.vc16, pa, oacc);
  } else if (kt1 - kt0 >= 2) {
    pv_last<C, false>(kvs[(kt - 1 - kt0) % NST] + C::kTile, ln.vrow, ln.vc16, pbb, oacc);
  } else {
    pv_last<C, true>(kvs[0] + C::kTile, ln.vrow, ln.vc16, pa, oacc);
  }

  // Epilogue: o = acc / l (the IEEE fp32 quotient, formed as in the other
  // prefill kernel: reciprocal and one correction, dividing where a live
  // quotient is below kRecipDivMin, zero or NaN), bf16 RNE, store.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float y = 1.0f / l[rb];
    float qv[C::kDb][4];
    bool small = false;
#pragma unroll
    for (int db = 0; db < C::kDb; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[db][i] = div_by_recip(oacc[rb][db][i], l[rb], y);
        small |= !(__builtin_fabsf(qv[db][i]) >= kRecipDivMin);
      }
    if (__builtin_amdgcn_ballot_w64(qpos[rb] >= 0 && small) != 0) {
#pragma unroll
      for (int db = 0; db < C::kDb; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[db][i] = oacc[rb][db][i] / l[rb];
    }
    if (qpos[rb] < 0) continue;
    bf16* orow = o + ((size_t)(seq0 + qpos[rb]) * hq + qhead[rb]) * D + 4 * ln.gq;
#pragma unroll
    for (int db = 0; db < C::kDb; ++db) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = to_bf16(qv[db][i]);
      *reinterpret_cast<bf16x4*>(orow + 16 * db) = w;
    }
    if (lse != nullptr && ln.gq == 0)
      lse[(size_t)(seq0 + qpos[rb]) * hq + qhead[rb]] =
          (m[rb] + fast_log2(l[rb])) * 0.693147180559945309f;
  }
}

template <class C>
static hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
  const int tiles = prefill_grid_tiles(a, C::kPositions);
  const long long blocks = run_major_blocks(tiles, (long long)a.hkv * a.batch);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const PagedKv pk{a.q_start, a.block_table, a.max_blocks, a.num_blocks, a.max_context};
  if (a.q_start != nullptr)
    hipLaunchKernelGGL(prefill_kernel<PagedOf<C>>, dim3((unsigned)blocks), dim3(C::kThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse,
                       a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2, tiles,
                       a.batch, pk);
  else
    hipLaunchKernelGGL(prefill_kernel<C>, dim3((unsigned)blocks), dim3(C::kThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse,
                       a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2, tiles,
                       a.batch, pk);
  return hipGetLastError();
}

// One kernel instance per group at head dim 64: four row blocks of 16 per
// wave, a ring of five stage buffers.  Head dims 256 and 512 run the
// two-kind kernel of prefill_ws.hip.
#define INVATTN_PREFILL64_TABLE(X) X(64, 1) X(64, 2) X(64, 4) X(64, 8)

bool prefill_schedule(int d, int group, PrefillSchedule* s) {
  if (prefill_ws_schedule(d, group, s)) return true;
#define X(D, G)                                                               \
  if (d == D && group == G) {                                                 \
    using C = Pf16Cfg<D, G, 4, 5>;                                            \
    *s = PrefillSchedule{C::kRows, C::kPositions, C::BN, C::kThreads,         \
                         "prefill_kernel<" #D "," #G ",4,5>"};                \
    return true;                                                              \
  }
  INVATTN_PREFILL64_TABLE(X)
#undef X
  return false;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.hq / a.hkv;
  PrefillSchedule sp;
  if (prefill_ws_schedule(a.d, group, &sp)) return launch_prefill_ws(a, stream);
#define X(D, G) \
  if (a.d == D && group == G) return launch_one<Pf16Cfg<D, G, 4, 5>>(a, stream);
  INVATTN_PREFILL64_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
