// prefill_ws.hip -- batch-invariant prefill for head dims 256 and 512 with
// the work of a workgroup specialised over two kinds of waves, two waves per
// SIMD.
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
// Why two kinds of waves.  One wave per SIMD that forms scores, runs the
// softmax and accumulates P V issues all of it from one instruction stream:
// the softmax's vector instructions and the LDS reads wait behind that
// wave's own MFMAs.  Here a workgroup has eight waves, two per SIMD: four
// score waves and four PV waves.  The SIMD interleaves the two streams, so
// the softmax of one wave runs while the other's MFMAs do, and each wave
// needs at most 256 registers (which is what lets two of them share a SIMD).
//
// Work map: a workgroup owns `positions` consecutive positions of ONE
// sequence, aligned to the sequence start, for the G query heads of one KV
// head; rows are position-major (row = position*G + head), cut into blocks
// of 16 (8 blocks at head dim 256, 4 at 512).
//   score wave s (0..3): row blocks RB*s .. RB*s+RB-1 (RB = 2 at head dim
//     256, 1 at 512; Q of those rows in 64 VGPRs);
//     S^T(t+1) = K Q^T  (v_mfma_f32_16x16x32_bf16, K operand from LDS, lane l
//                        holds keys 4*(l/16)+i of query row l%16, for 16-key
//                        halves kb = 0, 1),
//     softmax of tile t (fp32; the online rule of prefill_common.h) staged
//     between its MFMAs, P(t) (bf16, RNE) to LDS with the accumulator factors
//     of rows whose reference max moved; loads K(t+NR).
//   PV wave p (0..3): output columns [D/4 * p, D/4 * (p+1)) of every row
//     block; O^T += V^T P^T(t-1) after scaling the blocks whose rows moved
//     in tile t-1; P^T is the score lane's own 8 probabilities (k-slot
//     8*(l/16) + s meaning key 16*(s/4) + 4*(l/16) + s%4), V^T comes through
//     the transpose read in that key order; loads V(t+NR-2); the epilogue.
// K and V tiles (32 keys, ascending) stream HBM -> LDS with direct loads into
// two rings of NR buffers (3 at head dim 256, 2 at 512 where a tile is
// 32 KB); one LDS barrier per step orders the rings, the P exchange and the
// flags.  Keys past the sequence end load as zeros and are masked.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace invattn {

template <int D_, int G_, int RB_, int NR_, int BN_>
struct PfWsCfg {
  static constexpr bool kPaged = false;  // contiguous keys (PagedOf<> sets it)
  static constexpr int D = D_, G = G_;
  static constexpr int kRoleWaves = 4;                 // waves of each kind
  static constexpr int kWaves = 2 * kRoleWaves;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BN = BN_;                       // keys per KV tile: 32 or 16
  static constexpr int kHalves = BN / 16;              // 16-key halves of a tile
  static constexpr int kSlots = 4 * kHalves;           // scores per lane per row block
  // P^T exchange element of one lane and row block: 8 bf16 (32-key tiles,
  // 16x16x32 PV MFMAs) or 4 bf16 (16-key tiles, 16x16x16 PV MFMAs).
  using PT = typename std::conditional<BN == 32, bf16x8, bf16x4>::type;
  static constexpr int RB = RB_;                       // score row blocks per score wave
  static constexpr int kRowsPerWave = 16 * RB;
  static constexpr int kRows = kRoleWaves * kRowsPerWave;  // rows per workgroup
  static constexpr int kRowBlocks = kRows / 16;
  static constexpr int kPositions = kRows / G;
  static constexpr int kPosPerWave = kRowsPerWave / G;
  static constexpr int kSt = D / 32;                   // QK k-steps (32 head-dim elements)
  static constexpr int kDbW = D / 16 / kRoleWaves;     // output blocks of 16 columns per PV wave
  static constexpr int kChunks = D / 8;                // 16-byte chunks per row
  static constexpr int kTile = BN * D;                 // elements of one K (or V) tile
  static constexpr int kLoads = BN * kChunks / (64 * kRoleWaves);  // per lane per tile
  static constexpr int kRowsPerLoader = kLoads * 64 / kChunks;       // tile rows per loading wave
  static constexpr int kSwK = kChunks >= 16 ? 15 : kChunks - 1;
  static constexpr int kSwV = kChunks >= 16 ? 14 : kChunks - 2;
  static constexpr int kRing = NR_;                    // buffers per K / V ring
  // Who issues the K tile loads.  Head dim 256: the PV waves (the score waves
  // are the critical path and the PV waves have slack).  Head dim 512: the
  // score waves (each kind carries 32 MFMAs per step, and the PV waves' own V
  // loads already fill their issue slots).
  static constexpr bool kPvLoadsK = D <= 256;
  // When a step's tile loads are issued.  Head dim 512 (rings of two 64 KB
  // stages): all at the start of the step, since the next step waits for
  // them (7 % shorter steps on the global prefill).  Head dim 256 (three
  // stages): spread over the MFMA groups, which keeps the issue slots of the
  // step's first groups for the MFMAs (4 % shorter steps than issuing them
  // together).
  static constexpr bool kLoadsFirst = D >= 512;
  static_assert(D % 64 == 0 && kRowsPerWave % G == 0, "row map");
  static_assert(kLoads >= 1 && BN * kChunks % (64 * kRoleWaves) == 0, "tile load split");
  static_assert(BN == 16 || BN == 32, "tiles of 16 or 32 keys");
  static_assert(kRowsPerLoader * kRoleWaves == BN && 16 % kRowsPerLoader == 0,
                "KvTiles: loading wave w reads tile rows [RPW*w, RPW*w + RPW) of one cache block");
  static_assert(kRing >= 2 && kRing <= 4, "ring of two to four tiles");
  static_assert(kRing * 2 * kTile * 2 + 2 * kRowBlocks * 64 * (int)sizeof(PT) + 3 * kRows * 4 +
                        32 <= 163840,
                "LDS budget");
};

// Score wave, one step: S^T(t+1) = K Q^T for its RB row blocks on the K tile
// `kt`, in kHalves*kSt groups (one K operand each), with stage i of the previous
// tile's softmax (sm) after group i's MFMAs and, when DMA (the score waves
// load K), the K(t+NR) loads (before the first group, or spread over the
// groups; kLoadsFirst).  The MFMAs are compiler
// builtins with VGPR accumulators (the kernel uses no AGPRs), so the
// compiler tracks their result latency and schedules the softmax's vector
// work around them freely.
template <class C, bool DMA, class SM>
__device__ __forceinline__ void score_phase(const bf16* __restrict__ kt, uint32_t kpre,
                                            const u32x4& krs, int kk0, uint32_t rs_bytes,
                                            int widx, int lane, uint32_t krow, uint32_t kq16,
                                            const bf16x8 (*q)[C::kSt], f32x4 (*s)[2], SM&& sm) {
  constexpr int kN = C::kHalves * C::kSt;     // groups (one K operand each)
  constexpr int kEvery = kN / C::kLoads;      // groups per direct load
  constexpr int kAhead = 3;
  static_assert(kN % C::kLoads == 0, "loads spread evenly over the groups");
  const char* kb0 = reinterpret_cast<const char*>(kt) + krow;
  // Group i: k-step i / kHalves, 16-key half i % kHalves.
  auto kread = [&](int i) {
    return ld_lds_x8(reinterpret_cast<const bf16*>(
        kb0 + (kq16 ^ (uint32_t)((i / C::kHalves) << 6)) + (i % C::kHalves) * 32 * C::D));
  };
  bf16x8 kop[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) kop[i] = kread(i);
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const int st = i / C::kHalves, kb = i % C::kHalves;
    const bf16x8 a = kop[i % kAhead];
    if (i + kAhead < kN) kop[i % kAhead] = kread(i + kAhead);
    if constexpr (DMA) {
      if constexpr (C::kLoadsFirst) {
        if (i == 0) {
#pragma unroll
          for (int j = 0; j < C::kLoads; ++j)
            dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(kpre, krs, kk0, j, rs_bytes, widx, lane);
        }
      } else if (i % kEvery == 0) {
        dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(kpre, krs, kk0, i / kEvery, rs_bytes, widx,
                                                    lane);
      }
    }
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      s[rb][kb] = mfma16(a, q[rb][st], st == 0 ? f32x4{} : s[rb][kb]);
    }
    sm(i);  // stage i of the previous tile's softmax
  }
}

// PV wave, one step: O^T += V^T P^T for its kDbW output blocks of every row
// block, V from the tile `vt`, P^T from the exchange buffer `pt`, with the
// step's tile loads (K first when this wave loads K, then V; kLoads of each
// per lane) before the first group or spread over the groups (kLoadsFirst).
//   V operand (output block db): rows 4*gq + x/4 (and +16 for 32-key tiles),
//     logical chunk 2*(kDbW*p + db) + (x%4)/2, physical chunk ^ ((2*row) &
//     kSwV), element 4*(x%2);
//   P^T operand (row block r): lane l's element pt[64*r + l]; 16x16x32 MFMAs
//     over the 32 keys of a tile, or 16x16x16 MFMAs over the 16 of a
//     16-key tile.
template <class C, bool DMA, class PRE>
__device__ __forceinline__ void pv_phase(const bf16* __restrict__ vt,
                                         const typename C::PT* __restrict__ pt, uint32_t kpre,
                                         const u32x4& krs, int kk0, uint32_t vpre,
                                         const u32x4& vrs, int vk0, uint32_t rs_bytes, int widx,
                                         int lane,
                                         uint32_t vrow, uint32_t vc16w, f32x4 (*o)[C::kDbW],
                                         PRE&& pre) {
  constexpr int kN = C::kRowBlocks;           // one row block per group
  // Loads of the step: K (when this wave loads K) then V.
  constexpr int kKL = C::kPvLoadsK ? C::kLoads : 0;
  constexpr int kL = kKL + C::kLoads;
  // Direct loads spread evenly: one every kEvery groups, or kPer per group.
  constexpr int kEvery = kN >= kL ? kN / kL : 1;
  constexpr int kPer = kN >= kL ? 1 : kL / kN;
  static_assert(kN % kL == 0 || kL % kN == 0, "loads spread evenly over the groups");
  using PT = typename C::PT;
  const char* vb0 = reinterpret_cast<const char*>(vt) + vrow;
  PT vop[C::kDbW];
#pragma unroll
  for (int db = 0; db < C::kDbW; ++db) {
    const bf16* p = reinterpret_cast<const bf16*>(vb0 + (vc16w ^ (uint32_t)(db << 5)));
    if constexpr (C::BN == 32) vop[db] = cat8(ld_lds_tr(p), ld_lds_tr(p + 16 * C::D));
    else vop[db] = ld_lds_tr(p);
  }
  // Every row block's P^T operand of the step, read together with V^T: the
  // step waits for one LDS round trip, not one per row block.
  PT pop[kN];
#pragma unroll
  for (int r = 0; r < kN; ++r) pop[r] = pt[64 * r + lane];
  pre();  // the accumulator scaling of the step, while the reads are in flight
#pragma unroll
  for (int r = 0; r < kN; ++r) {
    if constexpr (DMA) {
      constexpr bool kFirst = C::kLoadsFirst;
      if (kFirst ? r == 0 : r % kEvery == 0) {
#pragma unroll
        for (int u = 0; u < (kFirst ? kL : kPer); ++u) {
          const int j = kFirst ? u : (r / kEvery) * kPer + u;
          if (j < kKL)
            dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(kpre, krs, kk0, j, rs_bytes, widx, lane);
          else
            dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(vpre, vrs, vk0, j - kKL, rs_bytes, widx,
                                                        lane);
        }
      }
    }
#pragma unroll
    for (int db = 0; db < C::kDbW; ++db) {
      if constexpr (C::BN == 32) o[r][db] = mfma16(vop[db], pop[r], o[r][db]);
      else o[r][db] = mfma16k16(vop[db], pop[r], o[r][db]);
    }
  }
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::kThreads, C::kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void prefill_ws_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
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
  __shared__ __attribute__((aligned(1024))) typename C::PT pl[2][kRB * 64];
  __shared__ __attribute__((aligned(16))) float al[2][C::kRows];
  __shared__ __attribute__((aligned(16))) uint32_t fl[2][4];
  __shared__ __attribute__((aligned(16))) float lrow[C::kRows];
  static_assert(C::kRoleWaves == 4, "one flag word per score wave, read as one 16-byte word");

  // Item = (tile, KV head, sequence) in run-major order (kernels.h); tiles
  // are numbered from the end of the sequence (longest causal rows first).
  // Tile t covers positions [t*P, (t+1)*P), counted from the first tile
  // holding a query row of the sequence.
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
  const bool pv_wave = wave >= C::kRoleWaves;
  const int widx = wave & (C::kRoleWaves - 1);  // index among the waves of its kind
  const bool windowed = window > 0;

  // Key range of the workgroup: the window below its first row, the span
  // holding its first row, its last row, the span holding its last row.
  // Spans [sp0, sp1) are those meeting the workgroup's positions [p0, p1).
  int lo = windowed ? max(0, p0 - window + 1) : 0;
  int hi = p1;
  int sp0 = 0, sp1 = 0;
  if (num_spans > 0) {
    spans_meeting(spans, num_spans, seq0 + p0, seq0 + p1, sp0, sp1);
    if (sp0 < sp1) {
      const int s_first = span_word(spans, 2 * sp0);
      const int e_last = span_word(spans, 2 * sp1 - 1);
      if (s_first <= seq0 + p0) lo = min(lo, max(s_first - seq0, 0));
      if (e_last > seq0 + p1 - 1) hi = max(hi, min(e_last - seq0, L));
    }
  }
  const int kt0 = lo / BN, kt1 = (hi + BN - 1) / BN;

  const uint32_t rs_bytes = (uint32_t)hkv * D * 2;
  // This KV head's rows of the sequence, loaded through buffer resources of
  // exactly that extent (the host rejects inputs whose rows span 2 GiB or
  // more), or its cache blocks.  Score waves load K, PV waves load V.
  const KvTiles<PAGED> src = kv_tiles<D, PAGED>(k, v, pk, sg, b, g, hkv, window);
  constexpr uint32_t kTileBytes = C::kTile * 2;
  const uint32_t ks_lds = lds_addr(ks[0]), vs_lds = lds_addr(vs[0]);

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

  using Mode0 = std::integral_constant<int, 0>;
  using Mode1 = std::integral_constant<int, 1>;
  using Mode2 = std::integral_constant<int, 2>;

  if (!pv_wave) {
    // ------------------------------------------------------------ score wave
    const int pw0 = p0 + widx * C::kPosPerWave;
    const int pw1 = min(pw0 + C::kPosPerWave, sg.qhi);
    const bool wave_full = pw0 >= sg.qlo && pw0 + C::kPosPerWave <= sg.qhi;
    int qpos[RB], qhead[RB], my_ss[RB], my_se[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = C::kRowsPerWave * widx + 16 * rb + ln.x;
      const int pos = p0 + row / G;
      qhead[rb] = g * G + row % G;
      const bool valid = pos >= sg.qlo && pos < sg.qhi;
      qpos[rb] = valid ? pos : -1;  // an invalid row admits no key
    }
    // Q^T operands: lane holds q[row][32*st + 8*gq .. +7] for every st.
    // Rows outside the sequence's query rows load its first query row
    // instead; every key is masked for them and they are never stored.
    bf16x8 qr[RB][C::kSt];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bf16* qrow = q + ((size_t)(seq0 + (qpos[rb] >= 0 ? qpos[rb] : sg.qlo)) * hq +
                              qhead[rb]) * D + 8 * ln.gq;
#pragma unroll
      for (int st = 0; st < C::kSt; ++st) qr[rb][st] = ld_global_x8(qrow + 32 * st);
    }
    // Each row's span (while Q is in flight): the one of the workgroup's
    // spans that holds it, if any.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      my_ss[rb] = 0;
      my_se[rb] = 0;
    }
    for (int i = sp0; i < sp1; ++i) {
      const int s_i = span_word(spans, 2 * i), e_i = span_word(spans, 2 * i + 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int tok = seq0 + qpos[rb];
        if (qpos[rb] >= 0 && tok >= s_i && tok < e_i) {
          my_ss[rb] = s_i - seq0;
          my_se[rb] = min(e_i - seq0, L);
        }
      }
    }
    RowStats<RB> rs;
    rs.init();

    constexpr bool kLoadK = !C::kPvLoadsK;  // this wave loads the K ring
    // Prologue: K(kt0) .. K(kt0+NR-1) in flight, K(kt0) landed before the
    // first barrier (issued here, or by the PV waves); form S(kt0).
    if constexpr (kLoadK) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        u32x4 krsc, vrsc;
        int k0r;
        src.template get<C::BN, C::kRowsPerLoader>(kt0 + i, kt0 + i < kt1, widx, krsc, vrsc,
                                                   k0r);
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j)
          dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(ks_lds + i * kTileBytes, krsc, k0r, j,
                                                      rs_bytes, widx, lane);
      }
      wait_vmcnt<(NR - 1) * C::kLoads>();
    }
    lds_barrier();
    f32x4 sa[RB][2], sb[RB][2];
    {
      const u32x4 none = buffer_rsrc(k, 0);
      score_phase<C, false>(ks[0], 0, none, 0, rs_bytes, widx, lane, ln.krow, ln.kq16, qr, sa,
                            [](int) {});
    }
    // Step kt: K(kt+1) has landed (waited for before the barrier by the wave
    // that loaded it), then S(kt+1) on the MFMAs (with the K(kt+NR) loads
    // among them when this wave loads K, into the buffer of K(kt), free once
    // every wave is past the barrier) while the VALU takes the softmax of
    // tile kt; the rare reference-max moves are handled after the MFMAs are
    // issued, and P(kt) goes to the exchange buffer.  After the last tile the
    // scores formed are never used (the K buffer holds zeros or an older
    // tile); forming them keeps the step branch-free.
    auto step = [&] __device__(int kt, f32x4(&sc)[RB][2], f32x4(&sn)[RB][2]) {
      const int r = (kt - kt0) % NR;
      const bf16* __restrict__ kcur = ks[(r + 1) % NR];  // K(kt+1)
      const uint32_t kpre = ks_lds + r * kTileBytes;      // K(kt+NR)
      const int k0 = kt * BN;
      if constexpr (kLoadK) wait_vmcnt<(NR - 2) * C::kLoads>();
      lds_barrier();
      const bool need_mask =
          !(wave_full && k0 + BN - 1 <= pw0 && (!windowed || pw1 - 1 - k0 < window));
      const uint32_t kq16 = opaque(ln.kq16);
      u32x4 krs, unused;
      int kk0 = 0;
      if constexpr (kLoadK)
        src.template get<C::BN, C::kRowsPerLoader>(kt + NR, kt + NR < kt1, widx, krs, unused, kk0);
      else krs = unused = u32x4{};
      float alpha[RB];
      uint32_t smask = 0;
      bf16x8 pc[RB];
      auto run = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        TileSoftmax<RB, MASK, C::kSlots> ts;
        ts.init(k0, ln, qpos, my_ss, my_se);
        score_phase<C, kLoadK>(kcur, kpre, krs, kk0, rs_bytes, widx, lane, ln.krow, kq16, qr, sn,
                               [&](int i) { ts.stage(i, sc, ln, rs); });
        if (ts.finish(rs)) smask = ts.move(sc, k0, ln, qpos, my_ss, my_se, rs, alpha);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) pc[rb] = ts.pb[rb];
      };
      if (need_mask)
        run(std::true_type{});
      else
        run(std::false_type{});
      // Exchange: P(kt) of this wave's row blocks, its scaling flags and
      // (when set) the row factors.
      typename C::PT* pw = pl[kt & 1];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (C::BN == 32) pw[64 * (RB * widx + rb) + lane] = pc[rb];
        else pw[64 * (RB * widx + rb) + lane] = bf16x4{pc[rb][0], pc[rb][1], pc[rb][2], pc[rb][3]};
      }
      if (smask != 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if ((smask & (1u << rb)) && ln.gq == 0)
            al[kt & 1][16 * (RB * widx + rb) + ln.x] = alpha[rb];
      }
      if (lane == 0) fl[kt & 1][widx] = smask;
    };
    step(kt0, sa, sb);
    int kt = kt0 + 1;
    for (; kt + 1 < kt1; kt += 2) {
      step(kt, sb, sa);
      step(kt + 1, sa, sb);
    }
    if (kt < kt1) step(kt, sb, sa);

    // Final row sums of this wave's rows for the PV waves' epilogue.
    float lsum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lsum[rb] = rs.row_sum(rb);
    if (ln.gq == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) lrow[C::kRowsPerWave * widx + 16 * rb + ln.x] = lsum[rb];
    }
    if constexpr (kLoadK) wait_vmcnt<0>();
    lds_barrier();
    if (lse != nullptr && ln.gq == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (qpos[rb] >= 0)
          lse[(size_t)(seq0 + qpos[rb]) * hq + qhead[rb]] =
              (rs.m[rb] + fast_log2(lsum[rb])) * 0.693147180559945309f;
    }
    return;
  }

  // ---------------------------------------------------------------- PV wave
  // V operand base of this wave's first output block.
  const uint32_t vc16w = ln.vc16 ^ (uint32_t)((C::kDbW * widx) << 5);
  // Loads of tile kt into ring buffer `slot`: K rows (WHICH & 1) and V rows
  // (WHICH & 2), this wave's share of each.
  auto load_tile = [&](int slot, int kt, int which) {
    u32x4 krsc, vrsc;
    int k0r;
    src.template get<C::BN, C::kRowsPerLoader>(kt, kt < kt1, widx, krsc, vrsc, k0r);
    if (which & 1) {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i)
        dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(ks_lds + slot * kTileBytes, krsc, k0r, i,
                                                    rs_bytes, widx, lane);
    }
    if (which & 2) {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i)
        dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(vs_lds + slot * kTileBytes, vrsc, k0r, i,
                                                    rs_bytes, widx, lane);
    }
  };
  // Accumulators start at +0: the first PV product adds to +0, which is the
  // product itself (as with a zero addend).
  f32x4 oacc[kRB][C::kDbW];
#pragma unroll
  for (int r = 0; r < kRB; ++r)
#pragma unroll
    for (int db = 0; db < C::kDbW; ++db) oacc[r][db] = f32x4{};

  // Scale the accumulator blocks whose rows moved their reference max in
  // tile kt (flags and factors written by the score waves in step kt).
  // The flags are read before the step's operands (flags_of), and used once
  // those reads are in flight (rescale_with).
  auto flags_of = [&](int kt) { return *reinterpret_cast<const u32x4*>(fl[kt & 1]); };
  auto rescale_with = [&](int kt, const u32x4& f) {
    const uint32_t mask = __builtin_amdgcn_readfirstlane(
        f[0] | (f[1] << RB) | (f[2] << (2 * RB)) | (f[3] << (3 * RB)));
    if (mask != 0) {
      // Blocks without a flag take factor 1 (exact).
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
        const float a = (mask & (1u << r)) ? al[kt & 1][16 * r + ln.x] : 1.f;
#pragma unroll
        for (int db = 0; db < C::kDbW; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[r][db][i] = oacc[r][db][i] * a;
      }
    }
  };

  // Tile loads.  Step kt issues K(kt+NR) (by the PV waves at head dim 256,
  // else by the score waves) and V(kt+NR-2); K(kt+NR) goes to the buffer of
  // K(kt) (read by the score waves in step kt-1), V(kt+NR-2) to the buffer of
  // V(kt-2) (read by PV(kt-2) in step kt-1), both free once every wave is
  // past the step's barrier.  Before the barrier of step kt the loading
  // waves wait for K(kt+1) (for the score waves) and V(kt-1) (for PV(kt-1)),
  // the loads of step kt+1-NR, so the NR-2 newer steps' loads may stay in
  // flight.  Prologue: the loads of the steps before kt0 -- K(kt0) ..
  // K(kt0+NR-1) when this wave loads K, and V(kt0) .. V(kt0+NR-3), issued in
  // the order those steps would have issued them (step kt0-NR+i: K(kt0+i),
  // then V(kt0+i-2)), so that from the first step on the loads a step waits
  // for are the oldest in flight; K(kt0) must land before the first barrier.
  constexpr bool kLoadK = C::kPvLoadsK;
  constexpr int kStepLoads = (kLoadK ? 2 : 1) * C::kLoads;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if constexpr (kLoadK) load_tile(i, kt0 + i, 1);
    if (i >= 2) load_tile(i - 2, kt0 + i - 2, 2);
  }
  if constexpr (kLoadK) wait_vmcnt<(2 * NR - 3) * C::kLoads>();
  lds_barrier();

  // Step kt: wait, barrier, scale for the moves of tile kt-1, then PV(kt-1)
  // with the step's loads among the MFMAs.  MODE 0: first tile (no PV yet);
  // 1: first PV (nothing to scale yet); 2: steady state.
  auto step = [&] __device__(int kt, auto mode) {
    constexpr int MODE = decltype(mode)::value;
    const int r = (kt - kt0) % NR;
    const bf16* __restrict__ vcur = vs[(r + NR - 1) % NR];           // V(kt-1)
    const uint32_t kpre = ks_lds + r * kTileBytes;                    // K(kt+NR)
    const uint32_t vpre = vs_lds + ((r + NR - 2) % NR) * kTileBytes;  // V(kt+NR-2)
    const typename C::PT* __restrict__ pcur = pl[(kt - 1) & 1];     // P(kt-1)
    wait_vmcnt<(NR - 2) * kStepLoads>();
    lds_barrier();
    u32x4 krs{}, vrs, unused;
    int kk0 = 0, vk0;
    if constexpr (kLoadK)
      src.template get<C::BN, C::kRowsPerLoader>(kt + NR, kt + NR < kt1, widx, krs, unused, kk0);
    src.template get<C::BN, C::kRowsPerLoader>(kt + NR - 2, kt + NR - 2 < kt1, widx, unused, vrs,
                                               vk0);
    if constexpr (MODE == 0) {
      // No PV yet: only the loads.
      if constexpr (kLoadK) {
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i)
          dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(kpre, krs, kk0, i, rs_bytes, widx, lane);
      }
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i)
        dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(vpre, vrs, vk0, i, rs_bytes, widx, lane);
    } else {
      const u32x4 f = MODE == 2 ? flags_of(kt - 1) : u32x4{};
      pv_phase<C, true>(vcur, pcur, kpre, krs, kk0, vpre, vrs, vk0, rs_bytes, widx, lane,
                        ln.vrow, opaque(vc16w), oacc, [&] {
                          if constexpr (MODE == 2) rescale_with(kt - 1, f);
                        });
    }
  };
  step(kt0, Mode0{});
  if (kt0 + 1 < kt1) step(kt0 + 1, Mode1{});
  for (int kt = kt0 + 2; kt < kt1; ++kt) step(kt, Mode2{});

  // PV of the last tile: every remaining load has landed (the loads after
  // the last tile are zero-length) and P(kt1-1) is in the exchange buffer.
  const int kl = kt1 - 1;
  wait_vmcnt<0>();
  lds_barrier();
  {
    const u32x4 none = buffer_rsrc(v, 0);
    const u32x4 f = flags_of(kl);
    pv_phase<C, false>(vs[(kl - kt0) % NR], pl[kl & 1], 0, none, 0, 0, none, 0, rs_bytes, widx,
                       lane, ln.vrow, vc16w, oacc, [&] {
                         if (kl > kt0) rescale_with(kl, f);
                       });
  }

  // Epilogue: o = acc / l (the IEEE fp32 quotient), bf16 RNE, store this
  // wave's columns of every row.  The quotients come from the row's
  // correctly rounded reciprocal and one correction each (div_by_recip): the
  // same bits as dividing, at a quarter of the instructions.  A row block in
  // which some live row's quotient is below kRecipDivMin, zero or NaN divides
  // instead.
  // Every row block's sum and reciprocal first (independent of each other),
  // so that their latencies overlap.
  float lrs[kRB], ys[kRB];
#pragma unroll
  for (int r = 0; r < kRB; ++r) lrs[r] = lrow[16 * r + ln.x];
#pragma unroll
  for (int r = 0; r < kRB; ++r) ys[r] = 1.0f / lrs[r];
#pragma unroll
  for (int r = 0; r < kRB; ++r) {
    const int row = 16 * r + ln.x;
    const int pos = p0 + row / G;
    const bool live = pos >= sg.qlo && pos < sg.qhi;
    const float lr = lrs[r];
    const float y = ys[r];
    float qv[C::kDbW][4];
    bool small = false;
#pragma unroll
    for (int db = 0; db < C::kDbW; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[db][i] = div_by_recip(oacc[r][db][i], lr, y);
        small |= !(__builtin_fabsf(qv[db][i]) >= kRecipDivMin);
      }
    if (__builtin_amdgcn_ballot_w64(live && small) != 0) {
#pragma unroll
      for (int db = 0; db < C::kDbW; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[db][i] = oacc[r][db][i] / lr;
    }
    if (live) {
      bf16* orow = o + ((size_t)(seq0 + pos) * hq + g * G + row % G) * D +
                   16 * C::kDbW * widx + 4 * ln.gq;
#pragma unroll
      for (int db = 0; db < C::kDbW; ++db) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = to_bf16(qv[db][i]);
        *reinterpret_cast<bf16x4*>(orow + 16 * db) = w;
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one row block at a time
  }
}

template <class C>
static hipError_t launch_ws(const PrefillArgs& a, hipStream_t stream) {
  const int tiles = prefill_grid_tiles(a, C::kPositions);
  const long long blocks = run_major_blocks(tiles, (long long)a.hkv * a.batch);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const PagedKv pk{a.q_start, a.block_table, a.max_blocks, a.num_blocks, a.max_context};
  if (a.q_start != nullptr)
    hipLaunchKernelGGL(prefill_ws_kernel<PagedOf<C>>, dim3((unsigned)blocks), dim3(C::kThreads),
                       0, stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                       (bf16*)a.o, a.lse, a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv,
                       a.window, a.c2, tiles, a.batch, pk);
  else
    hipLaunchKernelGGL(prefill_ws_kernel<C>, dim3((unsigned)blocks), dim3(C::kThreads), 0,
                       stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o,
                       a.lse, a.cu_seqlens, a.spans, a.num_spans, a.hq, a.hkv, a.window, a.c2,
                       tiles, a.batch, pk);
  return hipGetLastError();
}

// One kernel instance per (head_dim, group).  Parameters after (D, G): score
// row blocks per score wave (Q of 16*RB rows in 64 VGPRs: 2 at head dim 256,
// 1 at 512), buffers per K/V ring (3 at 256; 2 at 512, where a 32-key tile
// is 32 KB), keys per tile.  (Head dim 512 on 16-key tiles in rings of four
// runs its loads three 16-key steps ahead instead of one 32-key step: the
// one-token chunks of the paged entry point gain, but the prefill loses to
// the doubled per-step cost, so 32-key tiles stay.)
#define INVATTN_WS_TABLE(X)                                               \
  X(256, 1, 2, 3, 32) X(256, 2, 2, 3, 32) X(256, 4, 2, 3, 32) X(256, 8, 2, 3, 32) \
  X(512, 1, 1, 2, 32) X(512, 2, 1, 2, 32) X(512, 4, 1, 2, 32) X(512, 8, 1, 2, 32)

bool prefill_ws_schedule(int d, int group, PrefillSchedule* s) {
#define X(D, G, RB, NR, TBN)                                                         \
  if (d == D && group == G) {                                                        \
    using C = PfWsCfg<D, G, RB, NR, TBN>;                                            \
    *s = PrefillSchedule{C::kRows, C::kPositions, C::BN, C::kThreads,                \
                         "prefill_ws_kernel<" #D "," #G "," #RB "," #NR "," #TBN ">"}; \
    return true;                                                                     \
  }
  INVATTN_WS_TABLE(X)
#undef X
  return false;
}

hipError_t launch_prefill_ws(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.hq / a.hkv;
#define X(D, G, RB, NR, TBN) \
  if (a.d == D && group == G) return launch_ws<PfWsCfg<D, G, RB, NR, TBN>>(a, stream);
  INVATTN_WS_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
