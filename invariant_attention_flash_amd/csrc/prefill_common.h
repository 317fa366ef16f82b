// prefill_common.h -- pieces shared by the 16x16x32 prefill kernels
// (prefill.hip, prefill_ws.hip) and decode: per-lane constants, the direct
// HBM -> LDS tile loads and the online softmax of one 32-key tile.
//
// Sources: the numerical contract of "RFC: Gemma-4-31B-it train/rollout
// consistency", section 4 (fixed fp32 accumulators, one reduction order that
// does not depend on batch, packing, launch geometry or occupancy, declared
// casts, no fast-math); the masks of section 6 (sliding_attention_core /
// global_attention_core) and of the bidirectional soft-token spans (section
// 1, Phase B).
//
// Score layout (S^T = K Q^T on v_mfma_f32_16x16x32_bf16): for a row block of
// 16 query rows, lane l = 16*gq + x holds query row x, keys 4*gq + i
// (i = 0..3) of each 16-key half kb = 0, 1 of the tile; slot e = 4*kb + i.
#pragma once

#include "device_common.h"

namespace invattn {

// Reference-max hysteresis (log2 units): m moves only when a tile max
// exceeds it by more than this.  A fixed constant of the arithmetic.
constexpr float kRescale = 8.0f;

// Per-lane constants.  LDS operand addresses are byte offsets: a lane base
// plus (lane xor ^ step constant); the xors are laundered once per tile step
// (opaque) so the compiler forms each address next to its read instead of
// keeping one register per (buffer, step) alive across the loop.
struct Lane16 {
  int x, gq;           // lane = 16*gq + x
  uint32_t krow;       // K operand: byte offset of key row x
  uint32_t kq16;       // K operand: (logical chunk ^ physical chunk) of k-step 0, in bytes
  uint32_t vrow;       // V transpose read: byte offset of row 4*gq + x/4, element 4*(x%2)
  uint32_t vc16;       // V transpose read: physical chunk of block 0, in bytes
  int wlim;            // window (or a huge value for global layers)
  float c2;            // fl32(scale * log2 e)
};

template <class T>
__device__ __forceinline__ T opaque(T x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Buffer resource (gfx9 family) for bytes [base, base + nbytes): 32-bit
// data format, no swizzle, no index stride; loads past nbytes return zeros.
// Wave-uniform: readfirstlane keeps it in scalar registers.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, int nbytes) {
  auto uni = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4{uni((uint32_t)b), uni((uint32_t)(b >> 32) & 0xffffu), uni((uint32_t)nbytes),
               (uint32_t)kBufferFlags};
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(LDS_PTR(const void, p));
}

// Direct HBM -> LDS load (buffer_load_dwordx4 with the LDS bit: lane i's 16
// bytes land at LDS address M0 + 16*i) number i of a lane's share of one tile
// of 32 rows x CHUNKS 16-byte chunks into the tile at LDS address `tile`: a
// load fills 64 consecutive 16-byte LDS slots (loads are numbered
// wave-major, LOADS per lane), slot s holding row s / CHUNKS, physical chunk
// pc = s % CHUNKS, which receives logical chunk pc ^ ((row << SH) & SW).
// Rows come from byte (k0 + row) * rs_bytes of the resource `rs`: rows past
// its end are out of range and land as zeros, and an empty resource (no
// tile) loads nothing and writes zeros, so the caller stays branch-free.
//
// Issued from inline assembly so that the compiler does not track these
// loads: it cannot tell ring buffers apart across loop iterations and would
// otherwise wait for every load in flight before the first LDS read of a
// step.  The kernels wait for them explicitly (wait_vmcnt before the barrier
// that publishes a tile).  M0 carries the LDS address, with one wait state
// between its write and the load; the kernels leave M0 to these loads (the
// compiler emits no M0 use of its own in them, which a build test checks).
template <int CHUNKS, int LOADS, int SH, int SW>
__device__ __forceinline__ void dma_rows(uint32_t tile, const u32x4& rs, int k0, int i,
                                         uint32_t rs_bytes, int wave, int lane) {
  const int slot = (wave * LOADS + i) * 64;  // first 16-byte slot of this load
  const int pch = slot + lane;
  const int row = pch / CHUNKS;
  const int pc = pch % CHUNKS;
  const uint32_t voff = (uint32_t)(k0 + row) * rs_bytes + ((pc ^ ((row << SH) & SW)) << 4);
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(tile + slot * 16));
  __asm__ volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}

// ---------------------------------------------------------------------------
// Where a sequence's query rows and keys are.
//
// Contiguous layout (attn_prefill_varlen): positions [0, L) are the packed
// rows [cu[b], cu[b+1]) of q / o, and keys [0, L) the K/V rows of the same
// packed indices.  Paged layout (attn_prefill_paged): positions
// [q_start[b], q_start[b] + n) are the packed rows [cu[b], cu[b+1]) of q / o
// (n = cu[b+1] - cu[b]), and keys [0, q_start[b] + n) are read from the paged
// cache through the sequence's block-table row.  Position tiles stay aligned
// to position 0 in both layouts, so a row lands in the same wave, lane and
// MFMA slot and visits the same key tiles either way: its bytes are the same.

struct PagedKv {
  const int32_t* q_start;      // [batch]; nullptr: contiguous layout
  const int32_t* block_table;  // [batch, max_blocks]
  int max_blocks;
  int num_blocks;
  int max_context;             // bound on q_start[b] + n (at most 16 * max_blocks)
};

// Kernel configuration C with keys read from the paged cache (C::kPaged is
// false for the contiguous layout): a separate kernel instance, so the
// contiguous kernels carry no paged addressing.
template <class C>
struct PagedOf : C {
  static constexpr bool kPaged = true;
};

struct SeqGeo {
  int qlo, qhi;      // query positions [qlo, qhi)
  int L;             // keys [0, L)
  int qbase;         // packed row of position p: qbase + p
};

template <bool PAGED>
__device__ __forceinline__ SeqGeo seq_geo(const int32_t* cu, const PagedKv& pk, int b) {
  SeqGeo s;
  const int r0 = cu[b], n = cu[b + 1] - r0;
  s.qlo = PAGED ? pk.q_start[b] : 0;
  // A paged sequence outside the contract (negative start, or ending past
  // max_context) has no rows: nothing is read or written for it.
  if (PAGED && (s.qlo < 0 || (long long)s.qlo + n > pk.max_context)) {
    s.qlo = 0;
    s.qhi = 0;
  } else {
    s.qhi = s.qlo + n;
  }
  s.L = s.qhi;
  s.qbase = r0 - s.qlo;
  return s;
}

// Sources of the direct loads of one tile of BN keys.  With four loading
// waves, wave w loads tile rows [RPW*w, RPW*w + RPW), which in the paged
// layout (16-key cache blocks) lie in block (BN*kt + RPW*w) / 16.  `live` =
// false gives empty resources (the loads write zeros).  k0 is the row offset
// dma_rows adds to the tile row.
//
// Paged layout: only cache blocks holding keys in [klo, L) are read (klo =
// the first key the sequence's first query row may attend); the other rows of
// a tile land as zeros and are masked for every row that meets them.  Table
// reads stay inside the sequence's row, and an entry outside [0, num_blocks)
// is clamped into it, so a bad table cannot make the loads leave the cache.
template <bool PAGED>
struct KvTiles {
  const bf16* kbase;   // contiguous: this KV head's row 0 of the sequence; paged: cache + g*D
  const bf16* vbase;
  const int32_t* bt;   // paged: the sequence's block-table row
  int num_blocks;
  int max_blocks;
  int klo;
  size_t block_elems;  // paged: elements of one cache block (16 * Hkv * D)
  int L;
  uint32_t rs_bytes;   // bytes between consecutive keys of one KV head

  // BN: keys per tile; RPW: tile rows each loading wave loads (wave w loads
  // rows [RPW*w, RPW*w + RPW), all inside one 16-key cache block).
  template <int BN = 32, int RPW = 8>
  __device__ __forceinline__ void get(int kt, bool live, int wave, u32x4& krs, u32x4& vrs,
                                      int& k0) const {
    static_assert(16 % RPW == 0 && BN % 16 == 0, "a wave's rows lie in one cache block");
    if constexpr (!PAGED) {
      const int nb = live ? (int)((uint32_t)L * rs_bytes) : 0;
      krs = buffer_rsrc(kbase, nb);
      vrs = buffer_rsrc(vbase, nb);
      k0 = kt * BN;
    } else {
      // Branch-free: the table entry is always read (its index clamped into
      // the row), then dropped through rows = 0 when the block is not needed.
      const int first = RPW * wave;  // first tile row of this wave
      const int j = (kt * BN + first) >> 4;
      const int left = L - 16 * j;
      int rows = left < 16 ? left : 16;
      const bool need = live && left > 0 && j < max_blocks && 16 * j + 16 > klo;
      rows = need ? rows : 0;
      // The table is read through the constant address space: a scalar load
      // (the index is wave-uniform), waited on with the LDS counter.  A
      // vector load here would make the compiler wait for every load in
      // flight, the tile loads it cannot see included.
      using ConstI32 = const __attribute__((address_space(4))) int32_t;
      const int jc = j < max_blocks ? j : max_blocks - 1;
      int id = ((ConstI32*)bt)[jc];
      id = id < 0 ? 0 : id;
      id = id < num_blocks ? id : num_blocks - 1;
      const size_t off = (size_t)(uint32_t)id * block_elems;
      const int nb = (int)((uint32_t)rows * rs_bytes);
      krs = buffer_rsrc(kbase + off, nb);
      vrs = buffer_rsrc(vbase + off, nb);
      k0 = -16 * (first >> 4);
    }
  }
};

// Key sources of KV head g of sequence b (head dim D, hkv KV heads).
template <int D, bool PAGED>
__device__ __forceinline__ KvTiles<PAGED> kv_tiles(const bf16* k, const bf16* v,
                                                   const PagedKv& pk, const SeqGeo& sg, int b,
                                                   int g, int hkv, int window) {
  KvTiles<PAGED> src;
  src.L = sg.L;
  src.rs_bytes = (uint32_t)hkv * D * 2;
  if constexpr (!PAGED) {
    src.kbase = k + ((size_t)sg.qbase * hkv + g) * D;
    src.vbase = v + ((size_t)sg.qbase * hkv + g) * D;
    src.bt = nullptr;
    src.num_blocks = src.max_blocks = src.klo = 0;
    src.block_elems = 0;
  } else {
    src.kbase = k + (size_t)g * D;
    src.vbase = v + (size_t)g * D;
    src.bt = pk.block_table + (size_t)b * pk.max_blocks;
    src.num_blocks = pk.num_blocks;
    src.max_blocks = pk.max_blocks;
    src.klo = window > 0 ? max(0, sg.qlo - window + 1) : 0;
    src.block_elems = (size_t)16 * hkv * D;
  }
  return src;
}

// Scores of row block rb as NS slot values (8 for 32-key tiles, 4 for 16),
// masked when MASK.  Key j is
// allowed for a row at position qp when 0 <= qp - j < wlim (causal, window)
// or j lies in the row's span [ss, se); both tests are one unsigned compare
// each: wbase = qp - k0 - 4*gq, sbase = k0 + 4*gq - ss.
template <bool MASK, int NS = 8>
__device__ __forceinline__ void tile_values(const f32x4 (*s)[2], int rb, int k0, const Lane16& ln,
                                            const int* qpos, const int* ss, const int* se,
                                            float* v) {
#pragma unroll
  for (int e = 0; e < NS; ++e) v[e] = s[rb][e >> 2][e & 3];
  if constexpr (MASK) {
    const int wbase = qpos[rb] - k0 - 4 * ln.gq;
    const int sbase = k0 + 4 * ln.gq - ss[rb];
    const uint32_t slen = (uint32_t)(se[rb] - ss[rb]);
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      const int c = 16 * (e >> 2) + (e & 3);  // key j = k0 + 4*gq + c
      const bool ok = ((uint32_t)(wbase - c) < (uint32_t)ln.wlim) | ((uint32_t)(sbase + c) < slen);
      v[e] = ok ? v[e] : kNegInf;
    }
  }
}

// p = exp2(fma(s, c, -msub)) for the 8 slots of a row block, their sum in
// the fixed pairwise order ((p0+p1)+(p2+p3)) + ((p4+p5)+(p6+p7)), then across
// lanes l^32 and l^16 (each step: lower lane's value + upper lane's value),
// and the bf16 operand (round to nearest even).
__device__ __forceinline__ float probs(const float* v, float c2, float msub, bf16x8& pb) {
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(v[e], c2, -msub));
#pragma unroll
  for (int e = 0; e < 8; ++e) pb[e] = to_bf16(p[e]);
  float sum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  HalfPair hp = half_pair(sum);
  sum = hp.lo + hp.hi;
  hp = row_pair(sum);
  return hp.lo + hp.hi;
}

// Scaled tile max of a row (max over the NS slots, then lanes l^32, l^16).
template <int NS = 8>
__device__ __forceinline__ float row_max_scaled(const float* v, float c2) {
  float t = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  if constexpr (NS == 8) t = fmaxf(t, fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
  HalfPair hp = half_pair(t);
  t = fmaxf(hp.lo, hp.hi);
  hp = row_pair(t);
  return fmaxf(hp.lo, hp.hi) * c2;
}

// Softmax of one tile for RB row blocks, fast path.  Returns true when some
// row's reference max must move (tile max > m + kRescale, or the first
// allowed keys); then softmax_move() redoes the tile.  Otherwise p used m,
// alpha = 1 and l += sum -- bitwise what the moving rule gives.
template <int RB, bool MASK>
__device__ __forceinline__ bool softmax_fast(const f32x4 (*s)[2], int k0, const Lane16& ln,
                                             const int* qpos, const int* ss, const int* se,
                                             const float* m, float* l, bf16x8* pb) {
  bool any = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float v[8];
    tile_values<MASK>(s, rb, k0, ln, qpos, ss, se, v);
    const float m_old = m[rb];
    const float sum = probs(v, ln.c2, m_old == kNegInf ? 0.f : m_old, pb[rb]);
    const float tmax = row_max_scaled(v, ln.c2);
    const bool move = (tmax > m_old + kRescale) | ((m_old == kNegInf) & (tmax != kNegInf));
    any |= move;
    l[rb] = move ? l[rb] : l[rb] + sum;
  }
  return __builtin_amdgcn_ballot_w64(any) != 0;
}

// The rare path: rows whose tile max exceeds m + kRescale (or whose first
// allowed keys are in this tile) move m to the tile max, scale l by
// alpha = 2^(m_old - m_new) (1 when m_old = -inf: the accumulator and sum
// are still exact zeros) and recompute p with the new m.  alpha[rb] is the
// lane's row factor for the accumulator; bit rb of the returned mask is set
// when some row of block rb has alpha != 1 (the caller scales that block's
// accumulator, which is exact for the rows with alpha = 1).
template <int RB, bool MASK>
__device__ __forceinline__ uint32_t softmax_move(const f32x4 (*s)[2], int k0, const Lane16& ln,
                                                 const int* qpos, const int* ss, const int* se,
                                                 float* m, float* l, bf16x8* pb, float* alpha) {
  uint32_t scale = 0;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    alpha[rb] = 1.f;
    float v[8];
    tile_values<MASK>(s, rb, k0, ln, qpos, ss, se, v);
    const float m_old = m[rb];
    const float tmax = row_max_scaled(v, ln.c2);
    const bool move = (tmax > m_old + kRescale) | ((m_old == kNegInf) & (tmax != kNegInf));
    if (__builtin_amdgcn_ballot_w64(move) == 0) continue;
    const float m_new = move ? tmax : m_old;
    const float a = (move & (m_old != kNegInf)) ? fast_exp2(m_old - m_new) : 1.f;
    bf16x8 pnew;
    const float sum = probs(v, ln.c2, m_new == kNegInf ? 0.f : m_new, pnew);
    if (move) {
      pb[rb] = pnew;
      l[rb] = l[rb] * a + sum;
      m[rb] = m_new;
    }
    alpha[rb] = a;
    if (__builtin_amdgcn_ballot_w64(a != 1.f)) scale |= 1u << rb;
  }
  return scale;
}

// ---------------------------------------------------------------------------
// Staged online softmax.  The same tile softmax as above, cut into stages
// that a caller places between its MFMA groups, so the VALU work overlaps the
// matrix core instead of running before it.  Measured on gfx950 with one
// wave per SIMD: a short chain of dependent VALU ops between two MFMAs costs
// almost nothing, while as many independent ops cost three to four cycles
// each; so each stage takes ONE score through fma, exp2, the running sum
// and max and the bf16 cast, a dependent chain.
//
// Two rules differ from the one-shot form above:
//   * a row's reference max m moves when one of its lanes' sums of the
//     tile's p = 2^(fma(s, c, -m)) (eight slots) exceeds 2^kRescale (so no
//     p of the row exceeds it without a move), or, while m = -inf, when the
//     tile holds an allowed key (whatever its p against the provisional 0);
//     the fast path then needs no row max;
//   * the running sum is kept per lane: each lane adds its NS slots of a
//     tile in slot order, ((p0 + p1) + p2) + ..., to its own l (scaled by
//     alpha on a move), and the four lanes of a row are combined once, after
//     the last tile, as (l + l^32) then + l^16 (each step: lower lane's value
//     + upper lane's value).

// Row state: reference max m (scaled log2 units; -inf before the first
// allowed key), msub = m (0 while m = -inf), thr = the p threshold of a move
// (2^kRescale, 0 while m = -inf), the lane's running sum l.
template <int RB>
struct RowStats {
  float m[RB], msub[RB], thr[RB], l[RB];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m[rb] = kNegInf;
      msub[rb] = 0.f;
      thr[rb] = 0.f;
      l[rb] = 0.f;
    }
  }
  // The row's sum: the lanes' sums combined in the fixed order above.
  __device__ __forceinline__ float row_sum(int rb) const {
    HalfPair hp = half_pair(l[rb]);
    const float t = hp.lo + hp.hi;
    hp = row_pair(t);
    return hp.lo + hp.hi;
  }
};

// p of one row block (recomputed on the rare path) and the lane's sum of its
// NS slots in slot order.
template <int NS = 8>
__device__ __forceinline__ float probs_lane(const float* v, float c2, float msub, bf16x8& pb) {
  float p[NS];
#pragma unroll
  for (int e = 0; e < NS; ++e) p[e] = fast_exp2(__builtin_fmaf(v[e], c2, -msub));
#pragma unroll
  for (int e = 0; e < NS; ++e) pb[e] = to_bf16(p[e]);
  float sum = p[0];
#pragma unroll
  for (int e = 1; e < NS; ++e) sum = sum + p[e];
  return sum;
}

// Fast-path state of one tile: stage g (g < NS*RB) takes slot g%NS of row
// block g/NS (NS = 8 slots for 32-key tiles, 4 for 16-key tiles).
template <int RB, bool MASK, int NS = 8>
struct TileSoftmax {
  static constexpr int kStages = NS * RB;
  float part[RB];   // the lane's tile sum (slot order); also the move test
  bool anyok[RB];   // MASK: some slot of the lane holds an allowed key
  bf16x8 pb[RB];    // P operand
  int wbase[RB], sbase[RB];
  uint32_t slen[RB];

  __device__ __forceinline__ void init(int k0, const Lane16& ln, const int* qpos, const int* ss,
                                       const int* se) {
    if constexpr (MASK) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        wbase[rb] = qpos[rb] - k0 - 4 * ln.gq;
        sbase[rb] = k0 + 4 * ln.gq - ss[rb];
        slen[rb] = (uint32_t)(se[rb] - ss[rb]);
      }
    }
  }

  // Stage g (a constant after unrolling); stages past kStages do nothing.
  __device__ __forceinline__ void stage(int g, const f32x4 (*s)[2], const Lane16& ln,
                                        const RowStats<RB>& st) {
    if (g < 0 || g >= kStages) return;
    const int rb = g / NS, e = g % NS;
    float x = s[rb][e >> 2][e & 3];
    if constexpr (MASK) {
      const int c = 16 * (e >> 2) + (e & 3);  // key k0 + 4*gq + c
      const bool ok = ((uint32_t)(wbase[rb] - c) < (uint32_t)ln.wlim) |
                      ((uint32_t)(sbase[rb] + c) < slen[rb]);
      x = ok ? x : kNegInf;
      anyok[rb] = e == 0 ? ok : (anyok[rb] | ok);
    }
    const float p = fast_exp2(__builtin_fmaf(x, ln.c2, -st.msub[rb]));
    pb[rb][e] = to_bf16(p);
    part[rb] = e == 0 ? p : part[rb] + p;
  }

  // After the stages: true when some row of the wave may move (then move()
  // finishes the tile), else every lane adds its tile sum.  A row may move
  // when one of its lanes' tile sums exceeds the threshold (every p of the
  // lane is at most that sum), or, while its m = -inf (thr = 0), when one of
  // its keys in the tile is allowed: its scores may all be so low that every
  // p underflows to 0 against the provisional msub = 0, and the row must
  // still take its first reference max here.
  __device__ __forceinline__ bool finish(RowStats<RB>& st) {
    bool trig = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool first = st.thr[rb] == 0.f;
      trig |= (part[rb] > st.thr[rb]) | (first & (MASK ? anyok[rb] : true));
    }
    if (__builtin_amdgcn_ballot_w64(trig) != 0) return true;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) st.l[rb] += part[rb];
    return false;
  }

  // The rare path.  A row moves when its largest lane tile sum (over the
  // row's four lanes) exceeds its threshold, or, while m = -inf, when the
  // tile holds one of its allowed keys: m moves to the tile max, the lane
  // sums and the
  // accumulator scale by alpha = 2^(m_old - m_new) (1 when m_old = -inf:
  // both are still exact zeros) and p is recomputed; other rows add their
  // fast-path sums.  Returns the scaling mask (bit rb: some row of block rb
  // has alpha != 1) with the lane's row factors in alpha[].
  __device__ __forceinline__ uint32_t move(const f32x4 (*s)[2], int k0, const Lane16& ln,
                                           const int* qpos, const int* ss, const int* se,
                                           RowStats<RB>& st, float* alpha) {
    uint32_t scale = 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      alpha[rb] = 1.f;
      HalfPair hp = half_pair(part[rb]);
      const float t = fmaxf(hp.lo, hp.hi);
      hp = row_pair(t);
      bool mv = fmaxf(hp.lo, hp.hi) > st.thr[rb];
      const float m_old = st.m[rb];
      const bool first = m_old == kNegInf;
      if (__builtin_amdgcn_ballot_w64(mv | first) == 0) {
        st.l[rb] += part[rb];
        continue;
      }
      float x[NS];
      tile_values<MASK, NS>(s, rb, k0, ln, qpos, ss, se, x);
      const float tmax = row_max_scaled<NS>(x, ln.c2);
      mv = first ? (tmax != kNegInf) : mv;
      const float m_new = mv ? tmax : m_old;
      const float a = (mv & !first) ? fast_exp2(m_old - m_new) : 1.f;
      bf16x8 pnew = {};
      const float snew = probs_lane<NS>(x, ln.c2, mv ? m_new : st.msub[rb], pnew);
      if (mv) {
        pb[rb] = pnew;
        st.l[rb] = st.l[rb] * a + snew;
        st.m[rb] = m_new;
        st.msub[rb] = m_new;
        st.thr[rb] = (float)(1 << (int)kRescale);
      } else {
        st.l[rb] += part[rb];
      }
      alpha[rb] = a;
      if (__builtin_amdgcn_ballot_w64(a != 1.f)) scale |= 1u << rb;
    }
    return scale;
  }
};

}  // namespace invattn
