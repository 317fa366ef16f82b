// prefill_split.hip -- batch-invariant prefill for head dim 256 with the PV
// product split over head-dim columns across the waves of a workgroup.
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
// Why the split.  On gfx950 the V operand of O += P V has to reach the MFMA
// with 8 consecutive keys per lane, which the row-major V tile only gives
// through the LDS transpose read, and that read moves half the bytes of a
// 16-byte read per instruction.  When every wave forms all head-dim columns
// of its own rows, each wave transposes the whole V tile every step.  Here
// wave w forms columns [D/4 * w, D/4 * (w+1)) of ALL 128 rows of the
// workgroup instead: V traffic per wave falls to a quarter and each V operand
// feeds 8 MFMAs; the probabilities of every row are exchanged through LDS
// (plain 16-byte reads).
//
// Work map.  A workgroup (4 waves, one per SIMD) owns `positions`
// consecutive positions of ONE sequence, aligned to the sequence start, for
// the G query heads of one KV head; rows are position-major
// (row = position*G + head), cut into 8 blocks of 16.  Wave w owns row blocks
// 2w, 2w+1 for the scores and the softmax (Q in registers), and output
// columns [64w, 64w+64) of all 8 row blocks for P V.  A row therefore always
// lands in the same waves, lanes and MFMA slots and visits the same KV tiles
// in the same ascending order, whatever else is in the batch.
//
// Per KV tile of 32 keys (ascending), software-pipelined by one tile; step t:
//   S^T(t+1) = K Q^T  (v_mfma_f32_16x16x32_bf16, K operand from LDS,
//                      lane l holds keys 4*(l/16)+i of query row l%16, for
//                      16-key halves kb = 0, 1);
//   softmax of tile t (fp32; the online rule of prefill_common.h), its
//                      probabilities P(t) (bf16, RNE) to LDS, with the
//                      accumulator factors of rows whose reference max moved;
//   O^T += V^T P^T(t-1) for this wave's columns and every row block, after
//                      scaling the blocks whose rows moved in tile t-1; P^T is
//                      the writer lane's own 8 probabilities, k-slot
//                      8*(l/16) + s meaning key 16*(s/4) + 4*(l/16) + s%4, and
//                      V^T comes through the transpose read in that key order.
// K and V tiles stream HBM -> LDS with direct loads into two rings of three
// buffers: step t loads K(t+3) and V(t+1) (both needed two steps later) in
// between its MFMAs.  Keys past the sequence end load as zeros and are
// masked.  The accumulation order of every output element is the same
// sequence of MFMAs and scalings as when one wave forms all columns of its
// rows; fully masked tiles are exact no-ops for a row (p = 0, alpha = 1).
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace invattn {

template <int D_, int G_>
struct PfSplitCfg {
  static constexpr bool kPaged = false;  // contiguous keys (PagedOf<> sets it)
  static constexpr int D = D_, G = G_;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BN = 32;                        // keys per KV tile
  static constexpr int RB = 2;                         // score row blocks per wave
  static constexpr int kRowsPerWave = 16 * RB;
  static constexpr int kRows = kWaves * kRowsPerWave;  // rows per workgroup
  static constexpr int kRowBlocks = kRows / 16;
  static constexpr int kPositions = kRows / G;
  static constexpr int kPosPerWave = kRowsPerWave / G;
  static constexpr int kSt = D / 32;                   // QK k-steps (32 head-dim elements)
  static constexpr int kDbW = D / 16 / kWaves;         // output blocks of 16 columns per wave
  static constexpr int kChunks = D / 8;                // 16-byte chunks per row
  static constexpr int kTile = BN * D;                 // elements of one K (or V) tile
  static constexpr int kLoads = BN * kChunks / (64 * kWaves);  // per lane per tensor
  static constexpr int kSwK = kChunks >= 16 ? 15 : kChunks - 1;
  static constexpr int kSwV = kChunks >= 16 ? 14 : kChunks - 2;
  static constexpr int kRing = 3;                      // buffers per K / V ring
  static_assert(D % 64 == 0 && kRowsPerWave % G == 0, "row map");
  static_assert(kLoads >= 1 && BN * kChunks % (64 * kWaves) == 0, "tile load split");
  static_assert((kRowBlocks * kDbW) % (2 * kSt) == 0, "PV MFMAs spread evenly over the groups");
  static_assert((2 * kSt) % (2 * kLoads) == 0, "loads spread evenly over the groups");
  static_assert(kRowBlocks * kDbW * 4 + RB * 2 * 4 * 2 <= 256, "accumulators fit the AGPR file");
};

// One pipelined step's MFMA work, in groups (one K operand each):
// S^T(t+1) = K Q^T for this wave's RB row blocks on the K tile `kt`, and (PV)
// O^T += V^T P^T(t-1) for this wave's kDbW output blocks of every row block,
// V from the tile `vt`, P^T from the exchange buffer `pt`.  The next tiles'
// loads (K rows into `kpre`, V rows into `vpre`) are spread over the groups.
// FIRST: the first PV product starts the accumulator (zero addend).
//   K operand (k-step st, half kb): key row 16*kb + x, logical chunk
//     4*st + gq, physical chunk (4*st + gq) ^ (x & kSwK);
//   V operand (output block db of the wave): rows 4*gq + x/4 and +16,
//     logical chunk 2*(kDbW*w + db) + (x%4)/2, physical chunk
//     ^ ((2*row) & kSwV), element 4*(x%2);
//   P^T operand (row block r): 16 bytes of lane l at pt[64*r + l].
// LDS reads run ahead of their MFMAs (K: kAhead groups, P: two row blocks,
// V: every block of the step up front).  Group i also runs stage i of the
// softmax of the previous tile (sm), between its score and PV MFMAs; the
// groups are fenced (only SALU instructions may cross), so that VALU work
// stays spread over the MFMAs instead of bunching ahead of them.
template <class C, bool PV, bool FIRST, bool DMA, class SM>
__device__ __forceinline__ void split_phase(
    const bf16* __restrict__ kt, const bf16* __restrict__ vt, const bf16x8* __restrict__ pt,
    uint32_t kpre, uint32_t vpre, const u32x4& krs, const u32x4& vrs, int kk0, int vk0,
    uint32_t rs_bytes, int wave, int lane,
    uint32_t krow, uint32_t kq16, uint32_t vrow, uint32_t vc16w, const bf16x8 (*q)[C::kSt],
    f32x4 (*s)[2], f32x4 (*o)[C::kDbW], SM&& sm) {
  constexpr int kN = 2 * C::kSt;                      // groups
  constexpr int kPvPer = C::kRowBlocks * C::kDbW / kN;  // PV MFMAs per group
  constexpr int kEvery = kN / (2 * C::kLoads);        // groups per direct load
  constexpr int kAhead = 3;
  const char* kb0 = reinterpret_cast<const char*>(kt) + krow;
  const char* vb0 = reinterpret_cast<const char*>(vt) + vrow;
  auto kread = [&](int i) {
    return ld_lds_x8(reinterpret_cast<const bf16*>(
        kb0 + (kq16 ^ (uint32_t)((i >> 1) << 6)) + (i & 1) * 32 * C::D));
  };
  auto vread = [&](int db) {
    const bf16* p = reinterpret_cast<const bf16*>(vb0 + (vc16w ^ (uint32_t)(db << 5)));
    return cat8(ld_lds_tr(p), ld_lds_tr(p + 16 * C::D));
  };
  auto pread = [&](int r) { return pt[64 * r + lane]; };

  bf16x8 kop[kAhead], vop[C::kDbW], pop[C::kRowBlocks];
  kop[0] = kread(0);
  if constexpr (PV) {
    pop[0] = pread(0);
#pragma unroll
    for (int db = 0; db < C::kDbW; ++db) vop[db] = vread(db);
  }
#pragma unroll
  for (int i = 1; i < kAhead; ++i) kop[i] = kread(i);
  if constexpr (PV) pop[1] = pread(1);

#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const int st = i >> 1, kb = i & 1;
    const bf16x8 a = kop[i % kAhead];
    if (i + kAhead < kN) kop[i % kAhead] = kread(i + kAhead);
    if constexpr (PV) {
      const int j0 = kPvPer * i;
      if (j0 % C::kDbW == 0 && j0 / C::kDbW + 2 < C::kRowBlocks)
        pop[j0 / C::kDbW + 2] = pread(j0 / C::kDbW + 2);
    }
    if constexpr (DMA) {
      if (i % kEvery == 0) {
        const int j = i / kEvery;
        if ((j & 1) == 0)
          dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(kpre, krs, kk0, j >> 1, rs_bytes, wave,
                                                      lane);
        else
          dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(vpre, vrs, vk0, j >> 1, rs_bytes, wave,
                                                      lane);
      }
    }
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      if (st == 0)
        mfma16_vacc_first(s[rb][kb], a, q[rb][st]);
      else
        mfma16_vacc(s[rb][kb], a, q[rb][st]);
    }
    sm(i);  // stage i of the previous tile's softmax
    if constexpr (PV) {
#pragma unroll
      for (int u = 0; u < kPvPer; ++u) {
        const int j = kPvPer * i + u, r = j / C::kDbW, db = j % C::kDbW;
        o[r][db] = mfma16(vop[db], pop[r], FIRST ? f32x4{} : o[r][db]);
      }
    }
    __builtin_amdgcn_sched_barrier(0x0004);
  }
  mfma_drain();  // the scores are read by VALU code next
}

// O^T += V^T P^T for the last tile (no scores left to form).
template <class C, bool FIRST>
__device__ __forceinline__ void split_pv_last(const bf16* __restrict__ vt,
                                              const bf16x8* __restrict__ pt, int lane,
                                              uint32_t vrow, uint32_t vc16w,
                                              f32x4 (*o)[C::kDbW]) {
  const char* vb0 = reinterpret_cast<const char*>(vt) + vrow;
  bf16x8 vop[C::kDbW];
#pragma unroll
  for (int db = 0; db < C::kDbW; ++db) {
    const bf16* p = reinterpret_cast<const bf16*>(vb0 + (vc16w ^ (uint32_t)(db << 5)));
    vop[db] = cat8(ld_lds_tr(p), ld_lds_tr(p + 16 * C::D));
  }
#pragma unroll
  for (int r = 0; r < C::kRowBlocks; ++r) {
    const bf16x8 b = pt[64 * r + lane];
#pragma unroll
    for (int db = 0; db < C::kDbW; ++db)
      o[r][db] = mfma16(vop[db], b, FIRST ? f32x4{} : o[r][db]);
  }
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::kThreads, C::kThreads),
                          amdgpu_waves_per_eu(1, 1)))
void prefill_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                          const bf16* __restrict__ v, bf16* __restrict__ o,
                          float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                          const int32_t* __restrict__ spans, int num_spans, int hq, int hkv,
                          int window, float c2, int tiles, int nseq, PagedKv pk) {
  constexpr int D = C::D, G = C::G, RB = C::RB, BN = C::BN, NR = C::kRing;
  constexpr int kRB = C::kRowBlocks;
  // K ring and V ring (tile kt lives in buffer (kt - kt0) % NR of each);
  // exchange buffers for P, the accumulator factors and the scaling flags of
  // tile kt (index kt & 1); the final row sums.
  __shared__ __attribute__((aligned(1024))) bf16 ks[NR][C::kTile];
  __shared__ __attribute__((aligned(1024))) bf16 vs[NR][C::kTile];
  __shared__ __attribute__((aligned(1024))) bf16x8 pl[2][kRB * 64];
  __shared__ __attribute__((aligned(16))) float al[2][C::kRows];
  __shared__ __attribute__((aligned(16))) uint32_t fl[2][4];
  __shared__ __attribute__((aligned(16))) float lrow[C::kRows];
  static_assert(C::kWaves == 4, "one flag word per wave, read as one 16-byte word");

  // Logical item = (tile, KV head, sequence), tile fastest; tiles run from
  // the end of the sequence (longest causal rows first).  Tile t covers
  // positions [t*P, (t+1)*P), counted from the first tile holding a query
  // row of the sequence.
  const long long item = xcd_logical_block(blockIdx.x);
  if (item >= (long long)tiles * hkv * nseq) return;
  const int g = (int)((item / tiles) % hkv);
  const int b = (int)(item / ((long long)tiles * hkv));
  constexpr bool PAGED = C::kPaged;
  const SeqGeo sg = seq_geo<PAGED>(cu_seqlens, pk, b);
  const int L = sg.L;
  const int t = sg.qlo / C::kPositions + tiles - 1 - (int)(item % tiles);
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
  // Positions of this wave's score rows (a tile needs masks unless it is
  // fully allowed for every one of them).
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
  // V operand base of this wave's first output block.
  const uint32_t vc16w = ln.vc16 ^ (uint32_t)((C::kDbW * wave) << 5);

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
  // outside the sequence's query rows load its first query row instead;
  // every key is masked for them (qpos = -1) and they are never stored.
  bf16x8 qr[RB][C::kSt];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bf16* qrow =
        q + ((size_t)(seq0 + (qpos[rb] >= 0 ? qpos[rb] : sg.qlo)) * hq + qhead[rb]) * D + 8 * ln.gq;
#pragma unroll
    for (int st = 0; st < C::kSt; ++st) qr[rb][st] = ld_global_x8(qrow + 32 * st);
  }

  const uint32_t rs_bytes = (uint32_t)hkv * D * 2;
  // This KV head's rows of the sequence, loaded through buffer resources of
  // exactly that extent (the host rejects inputs whose rows span 2 GiB or
  // more), or its cache blocks.
  const KvTiles<PAGED> src = kv_tiles<D, PAGED>(k, v, pk, sg, b, g, hkv, window);
  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;
  constexpr int kPerStep = 2 * C::kLoads;  // direct loads per lane per step
  // LDS addresses of the rings (tile kt in buffer (kt - kt0) % NR).
  constexpr uint32_t kTileBytes = C::kTile * 2;
  const uint32_t ks_lds = lds_addr(ks[0]), vs_lds = lds_addr(vs[0]);
  auto load_k = [&](int slot, int kt) {
    u32x4 krsc, vrsc;
    int k0r;
    src.get(kt, kt < kt1, wave, krsc, vrsc, k0r);
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
      dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(ks_lds + slot * kTileBytes, krsc, k0r, i,
                                                  rs_bytes, wave, lane);
  };
  auto load_v = [&](int slot, int kt) {
    u32x4 krsc, vrsc;
    int k0r;
    src.get(kt, kt < kt1, wave, krsc, vrsc, k0r);
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
      dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(vs_lds + slot * kTileBytes, vrsc, k0r, i,
                                                  rs_bytes, wave, lane);
  };

  // Accumulators: O starts at the first PV product (zero addend).
  f32x4 oacc[kRB][C::kDbW];
  RowStats<RB> rs;
  rs.init();

  // Scale the accumulator blocks whose rows moved their reference max in
  // tile kt (flags and factors written by the owning waves in step kt).
  auto rescale_from = [&](int kt) {
    const u32x4 f = *reinterpret_cast<const u32x4*>(fl[kt & 1]);
    const uint32_t mask = __builtin_amdgcn_readfirstlane(
        f[0] | (f[1] << RB) | (f[2] << (2 * RB)) | (f[3] << (3 * RB)));
    if (mask != 0) {
      // In place on the accumulation registers; blocks without a flag take
      // factor 1 (exact).  The nops cover the MFMA-result and the
      // VALU-write-to-MFMA distances around the asm.
      mfma_drain();
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
        const float a = (mask & (1u << r)) ? al[kt & 1][16 * r + ln.x] : 1.f;
#pragma unroll
        for (int db = 0; db < C::kDbW; ++db) scale_acc4(oacc[r][db], a);
      }
      __asm__ volatile("s_nop 4");
    }
  };

  // Prologue: K(kt0), K(kt0+1), then K(kt0+2) with V(kt0) (what step kt0-1
  // would load); wait for K(kt0) and form S(kt0).
  load_k(0, kt0);
  load_k(1, kt0 + 1);
  load_k(2, kt0 + 2);
  load_v(0, kt0);
  wait_vmcnt<C::kLoads + kPerStep>();
  lds_barrier();

  // Scores of consecutive tiles alternate between two arrays (steps are
  // unrolled by two), so nothing is copied.
  f32x4 sa[RB][2], sb[RB][2];
  {
    const u32x4 none = buffer_rsrc(k, 0);
    split_phase<C, false, false, false>(ks[0], vs[0], pl[0], 0, 0, none, none, 0, 0, rs_bytes,
                                        wave, lane, ln.krow, ln.kq16, ln.vrow, vc16w, qr, sa,
                                        oacc, [](int) {});
  }

  // Step kt: wait for K(kt+1) and V(kt-1) (loaded two steps ago), then
  // S(kt+1) and PV(kt-1) on the MFMAs with the loads of K(kt+3) and V(kt+1)
  // among them (into the buffers of K(kt) and V(kt-2), free once every wave
  // is past the barrier), while the VALU takes the softmax of tile kt; the
  // rare reference-max moves are handled after the MFMAs are issued, and P(kt)
  // goes to the exchange buffer.  After the last tile the scores formed are
  // never used (the K buffer holds zeros or an older tile); forming them
  // keeps the step branch-free.  MODE 0: first tile (no PV yet); 1: first PV
  // (starts O); 2: steady state.
  auto step = [&] __device__(int kt, f32x4(&sc)[RB][2], f32x4(&sn)[RB][2], auto mode) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool PV = MODE > 0, FIRST = MODE == 1;
    const int r = (kt - kt0) % NR;
    const bf16* __restrict__ kcur = ks[(r + 1) % NR];       // K(kt+1)
    const uint32_t kpre = ks_lds + r * kTileBytes;           // K(kt+3)
    const bf16* __restrict__ vcur = vs[(r + NR - 1) % NR];  // V(kt-1)
    const uint32_t vpre = vs_lds + ((r + 1) % NR) * kTileBytes;  // V(kt+1)
    const bf16x8* __restrict__ pcur = pl[(kt - 1) & 1];     // P(kt-1)
    const int k0 = kt * BN;
    wait_vmcnt<kPerStep>();
    lds_barrier();
    if constexpr (PV && !FIRST) rescale_from(kt - 1);
    const bool need_mask =
        !(wave_full && k0 + BN - 1 <= pw0 && (!windowed || pw1 - 1 - k0 < window));
    const uint32_t kq16 = opaque(ln.kq16), vcw = opaque(vc16w);
    u32x4 krs, vrs, unused;
    int kk0, vk0;
    src.get(kt + 3, kt + 3 < kt1, wave, krs, unused, kk0);
    src.get(kt + 1, kt + 1 < kt1, wave, unused, vrs, vk0);
    float alpha[RB];
    uint32_t smask = 0;
    bf16x8 pc[RB];
    auto run = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      TileSoftmax<RB, MASK> ts;
      ts.init(k0, ln, qpos, my_ss, my_se);
      split_phase<C, PV, FIRST, true>(kcur, vcur, pcur, kpre, vpre, krs, vrs, kk0, vk0,
                                      rs_bytes, wave, lane, ln.krow, kq16,
                                      ln.vrow, vcw, qr, sn, oacc,
                                      [&](int i) { ts.stage(i, sc, ln, rs); });
      if (ts.finish(rs)) smask = ts.move(sc, k0, ln, qpos, my_ss, my_se, rs, alpha);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) pc[rb] = ts.pb[rb];
    };
    if (need_mask)
      run(std::true_type{});
    else
      run(std::false_type{});
    // Exchange: P(kt) of this wave's row blocks, its scaling flags and (when
    // set) the row factors.
    bf16x8* pw = pl[kt & 1];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) pw[64 * (RB * wave + rb) + lane] = pc[rb];
    if (smask != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if ((smask & (1u << rb)) && ln.gq == 0) al[kt & 1][16 * (RB * wave + rb) + ln.x] = alpha[rb];
    }
    if (lane == 0) fl[kt & 1][wave] = smask;
  };
  using Mode0 = std::integral_constant<int, 0>;
  using Mode1 = std::integral_constant<int, 1>;
  using Mode2 = std::integral_constant<int, 2>;
  step(kt0, sa, sb, Mode0{});
  if (kt0 + 1 < kt1) step(kt0 + 1, sb, sa, Mode1{});
  int kt = kt0 + 2;
  for (; kt + 1 < kt1; kt += 2) {
    step(kt, sa, sb, Mode2{});
    step(kt + 1, sb, sa, Mode2{});
  }
  if (kt < kt1) step(kt, sa, sb, Mode2{});

  // Final row sums of this wave's rows for every wave's epilogue.
  float lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) lsum[rb] = rs.row_sum(rb);
  if (ln.gq == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lrow[C::kRowsPerWave * wave + 16 * rb + ln.x] = lsum[rb];
  }
  // PV of the last tile: every remaining load has landed (the loads after
  // the last tile are zero-length) and P(kt1-1) is in the exchange buffer.
  const int kl = kt1 - 1;
  wait_vmcnt<0>();
  lds_barrier();
  if (kl > kt0) {
    rescale_from(kl);
    split_pv_last<C, false>(vs[(kl - kt0) % NR], pl[kl & 1], lane, ln.vrow, vc16w, oacc);
  } else {
    split_pv_last<C, true>(vs[0], pl[kl & 1], lane, ln.vrow, vc16w, oacc);
  }

  // Epilogue: o = acc / l (IEEE fp32 division), bf16 RNE, store this wave's
  // columns of every row.
#pragma unroll
  for (int r = 0; r < kRB; ++r) {
    const int row = 16 * r + ln.x;
    const int pos = p0 + row / G;
    if (pos < sg.qlo || pos >= sg.qhi) continue;
    const float lr = lrow[row];
    bf16* orow = o + ((size_t)(seq0 + pos) * hq + g * G + row % G) * D + 16 * C::kDbW * wave +
                 4 * ln.gq;
#pragma unroll
    for (int db = 0; db < C::kDbW; ++db) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = to_bf16(oacc[r][db][i] / lr);
      *reinterpret_cast<bf16x4*>(orow + 16 * db) = w;
    }
  }
  if (lse != nullptr && ln.gq == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (qpos[rb] >= 0)
        lse[(size_t)(seq0 + qpos[rb]) * hq + qhead[rb]] =
            (rs.m[rb] + fast_log2(lsum[rb])) * 0.693147180559945309f;
  }
}

template <class C>
static hipError_t launch_split(const PrefillArgs& a, hipStream_t stream) {
  const int tiles = prefill_grid_tiles(a, C::kPositions);
  const long long blocks = xcd_padded_blocks((long long)tiles * a.hkv * a.batch);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const PagedKv pk{a.q_start, a.block_table, a.max_blocks, a.num_blocks, a.max_context};
  if (a.q_start != nullptr)
    hipLaunchKernelGGL(prefill_split_kernel<PagedOf<C>>, dim3((unsigned)blocks), dim3(C::kThreads), 0,
                       stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o,
                       a.lse, a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2,
                       tiles, a.batch, pk);
  else
    hipLaunchKernelGGL(prefill_split_kernel<C>, dim3((unsigned)blocks), dim3(C::kThreads), 0,
                       stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o,
                       a.lse, a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2,
                       tiles, a.batch, pk);
  return hipGetLastError();
}

// One kernel instance per (head_dim, group).
#define INVATTN_SPLIT_TABLE(X) X(256, 1) X(256, 2) X(256, 4) X(256, 8)

bool prefill_split_schedule(int d, int group, PrefillSchedule* s) {
#define X(D, G)                                                               \
  if (d == D && group == G) {                                                 \
    using C = PfSplitCfg<D, G>;                                               \
    *s = PrefillSchedule{C::kRows, C::kPositions, C::BN, C::kThreads};        \
    return true;                                                              \
  }
  INVATTN_SPLIT_TABLE(X)
#undef X
  return false;
}

hipError_t launch_prefill_split(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.hq / a.hkv;
#define X(D, G) \
  if (a.d == D && group == G) return launch_split<PfSplitCfg<D, G>>(a, stream);
  INVATTN_SPLIT_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
