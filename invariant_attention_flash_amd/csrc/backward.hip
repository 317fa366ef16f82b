// backward.hip -- deterministic attention backward (dq, dk, dv) for packed
// variable-length prefill on the matrix cores, with every sum in a fixed
// order and no atomics.
//
// Sources: the train/rollout consistency goal covers the training step
// ("RFC: Gemma-4-31B-it train/rollout consistency", section 1 and section 4
// item 1: every reduction has a declared fp32 accumulator and a fixed order;
// item 3: no split-K, Stream-K or cross-workgroup atomics); the gradient is
// the chain rule on the forward's definition (same masks, spans and GQA map
// as the prefill kernels).
//
// Arithmetic (c = fl32(scale * log2 e); the forward's natural-log LSE enters
// as lse2 = fl32(lse * log2 e)):
//   s_ij, dp_ij, delta_i  bf16 MFMA dot products (fp32 accumulation) of
//           q_i.k_j, v_j.dout_i and o_i.dout_i (o: the forward's bf16 output;
//           delta by the same MFMA sequence as dp)
//   p_ij    = exp2(fma(s_ij, c, -lse2_i))   (0 where the mask excludes j)
//   ds_ij   = p_ij * (dp_ij - delta_i)
//   dq_i    = scale * sum_j bf16(ds_ij) k_j          32 keys per MFMA (key
//                                                    tiles at multiples of
//                                                    32), ascending
//   dk_j    = scale * sum_(i,h) bf16(ds_ij) q_(i,h)  32 (row, head) pairs per
//   dv_j    =         sum_(i,h) bf16(p_ij) dout_(i,h) MFMA: rows ascending, then
//                                                    the group's heads
// A tile's keys (or pairs) start at a position fixed by the row (or key)
// tile alone, and every output element is written once by one lane, so the
// result does not depend on the batch, the packing or the grid.
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): lane l = 16*g + x supplies
// A[x][8g..8g+7] and B[8g..8g+7][x] and receives D[4g..4g+3][x].  Scores come
// out as S^T (keys in M, rows in N), so lane (g, x) holds keys 4g+i and
// 16+4g+i of row x.  Those eight values are the lane's B operand of the
// gradient products as they stand: k-slot j stands for key 16*(j/4) + 4g +
// j%4, and the A operand (K, Q or dout transposed) is read from LDS in the
// same key order with transpose reads.
#include "device_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace invattn {

namespace {

constexpr int kBwdThreads = 256;   // four waves
constexpr int kBwdRows = 64;       // rows (dq) or keys (dk, dv) per workgroup: 16 per wave
constexpr int kBwdTile = 32;       // keys (dq) or (row, head) pairs (dk, dv) per step

template <int D>
struct BwdCfg {
  static constexpr int kSt = D / 32;     // k-steps over the head dim
  static constexpr int kDb = D / 16;     // 16-column blocks of the head dim
  // LDS row stride in bf16: 32 bytes of padding put the rows 8 banks apart,
  // so neither the 16-byte row reads (8 rows) nor the transpose reads (4
  // rows x 4 column groups) of a pass share a bank.
  static constexpr int kLd = D + 16;
  // dk/dv: 32-pair halves per step (two independent halves where the LDS
  // budget allows); each half is one MFMA group of the fixed pair order.
  static constexpr int kHalves = D <= 256 ? 2 : 1;
  // dk/dv: next pair tile's loads held in registers during the current one.
  // At head dim 512 the accumulators leave no room for that: the next tile
  // goes straight to LDS with direct loads instead (bwd_dkv_kernel, dma_row).
  static constexpr bool kPrefetch = D <= 256;
  static constexpr int kPairs = kBwdTile * kHalves;
  static_assert(D % 32 == 0, "head dim in MFMA k-steps");
};

// Key j is in row i's allowed set.  BITWISE: without short-circuits, so
// that callers select rather than branch (the one-kind dk/dv kernel at head
// dim 512 keeps the short-circuit form, which needs fewer live registers).
template <bool BITWISE = true>
__device__ __forceinline__ bool admits(int i, int j, int window, int ss, int se) {
  if constexpr (BITWISE) {
    const bool causal = (j <= i) & ((window < 0) | (i - j < window));
    return causal | ((j >= ss) & (j < se));
  } else {
    const bool causal = j <= i && (window < 0 || i - j < window);
    return causal || (j >= ss && j < se);
  }
}

// p = ok ? exp2(arg) : 0.  SELECT: exp2 always, then a select (no branch);
// otherwise the compiler may branch around the exp2 (fewer live registers:
// the one-kind dk/dv kernel at head dim 512 needs that).
template <bool SELECT>
__device__ __forceinline__ float masked_exp2(bool ok, float arg) {
  if constexpr (SELECT) {
    const float ex = fast_exp2(arg);
    return ok ? ex : 0.f;
  } else {
    return ok ? fast_exp2(arg) : 0.f;
  }
}

// Work item of this workgroup: tile `tile` (numbered most work first) of
// sequence b, head h, in run-major order (kernels.h).
__device__ __forceinline__ bool bwd_item(int tiles, int heads, int nseq, int& tile, int& b,
                                         int& h) {
  long long grp;
  if (!run_major_item(blockIdx.x, tiles, (long long)heads * nseq, tile, grp)) return false;
  b = (int)(grp / heads);
  h = (int)(grp % heads);
  return true;
}

__device__ __forceinline__ void st_lds_x8(bf16* p, bf16x8 x) {
  *reinterpret_cast<bf16x8*>(p) = x;
}

// Direct HBM -> LDS load of one 1 KB row (head dim 512, bf16): lane i's 16
// bytes, from byte voff + 16*i of the resource `rs`, land at LDS byte
// address lds + 16*i; out-of-range bytes load as zeros.  Issued from inline
// assembly (see dma_rows): the kernel waits for it explicitly before the
// barrier that publishes the tile, and leaves M0 to these loads.
__device__ __forceinline__ void dma_row(uint32_t lds, const u32x4& rs, uint32_t voff, int lane) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  const uint32_t vo = voff + 16u * (uint32_t)lane;
  __asm__ volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(vo), "s"(rs)
      : "memory");
}

// A operand of the gradient products: X^T for 16 columns [c0, c0 + 16) of
// a staged [32][kLd] tile, k-slot j <-> tile row 16*(j/4) + 4g + j%4.  Lane
// 4a + c of a 16-lane group receives element c of the rows addressed by
// lanes a + 4r; lane m therefore addresses row 4g + m/4 at column c0 +
// 4*(m%4) (plus 16 rows for k-slots 4..7).
template <int LD>
__device__ __forceinline__ bf16x8 lds_t_operand(const bf16* tile, int c0, int g, int x) {
  const bf16* p = tile + (4 * g + x / 4) * LD + c0 + 4 * (x % 4);
  return cat8(ld_lds_tr(p), ld_lds_tr(p + 16 * LD));
}

__device__ __forceinline__ bf16x8 pack8(const f32x4& lo, const f32x4& hi) {
  return bf16x8{to_bf16(lo[0]), to_bf16(lo[1]), to_bf16(lo[2]), to_bf16(lo[3]),
                to_bf16(hi[0]), to_bf16(hi[1]), to_bf16(hi[2]), to_bf16(hi[3])};
}

// A staged tile moves in two halves so that the next tile's global loads
// are in flight while the current one is used: fetch() loads this thread's
// 16-byte chunks into registers (row r from src(r); nullptr: zeros), put()
// stores them into an LDS tile of row stride kLd.
template <int D, int ROWS = kBwdTile>
struct TileRegs {
  static constexpr int kPer = ROWS * D / 8 / kBwdThreads;
  static_assert((ROWS * D / 8) % kBwdThreads == 0, "whole chunks per thread");
  bf16x8 r[kPer];

  template <class Src>
  __device__ __forceinline__ void fetch(Src src, int tid) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kBwdThreads;
      const bf16* s = src(e / (D / 8));
      r[u] = s ? ld_global_x8(s + 8 * (e % (D / 8))) : bf16x8{};
    }
  }
  __device__ __forceinline__ void put(bf16* tile, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kBwdThreads;
      st_lds_x8(tile + (e / (D / 8)) * BwdCfg<D>::kLd + 8 * (e % (D / 8)), r[u]);
    }
  }
};

}  // namespace

// dq of 64 rows of one query head, and delta of those rows.
template <int D>
__global__ __launch_bounds__(kBwdThreads)
void bwd_dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                   const bf16* __restrict__ v, const bf16* __restrict__ o,
                   const float* __restrict__ lse, const bf16* __restrict__ dout,
                   float* __restrict__ dq, float* __restrict__ delta,
                   const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ spans,
                   int num_spans, int hq, int hkv, int window, float scale, float c2,
                   int tiles, int nseq) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 kts[2][kBwdTile * C::kLd];
  __shared__ __attribute__((aligned(16))) bf16 vts[2][kBwdTile * C::kLd];
  __shared__ bf16x8 xch[4][64];   // dS of every wave's row block as B operands
  // Item = (row tile, query head, sequence), row tiles numbered from the end
  // of the sequence (longest causal rows first); neighbouring row tiles share
  // most of their keys.
  int tile, b, h;
  if (!bwd_item(tiles, hq, nseq, tile, b, h)) return;
  const int kvh = h / (hq / hkv);
  const int seq0 = cu_seqlens[b], L = cu_seqlens[b + 1] - seq0;
  const int r0 = (tiles - 1 - tile) * kBwdRows;
  if (r0 >= L) return;
  const int r1 = min(r0 + kBwdRows, L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int x = lane & 15, g = lane >> 4;
  const int i = r0 + 16 * w + x;
  const bool live = i < r1;
  const int ic = live ? i : r0;   // rows past the tile compute on row r0; nothing stored
  const size_t qo = ((size_t)(seq0 + ic) * hq + h) * D;

  // Q and dout as B operands (B[d][row]): lane (g, x) holds d = 32st + 8g + 0..7.
  // delta is the diagonal of O dout^T, formed by the same MFMA sequence as
  // dP^T = V dout^T (A: the row of O or V, B: dout), so that dp_ij equals
  // delta_i bit for bit when v_j = o_i.
  bf16x8 qop[C::kSt], dop[C::kSt];
  f32x4 dd = f32x4{};
#pragma unroll
  for (int st = 0; st < C::kSt; ++st) {
    qop[st] = ld_global_x8(q + qo + 32 * st + 8 * g);
    dop[st] = ld_global_x8(dout + qo + 32 * st + 8 * g);
    dd = mfma16(ld_global_x8(o + qo + 32 * st + 8 * g), dop[st], dd);
  }
  // D[m][x] sits in lane 16*(m/4) + x, element m%4: the diagonal of row x in
  // lane 16*(x/4) + x, element x%4.
  const int dsrc = 16 * (x >> 2) + x;
  const float dsel = (x & 3) == 0 ? dd[0] : (x & 3) == 1 ? dd[1] : (x & 3) == 2 ? dd[2] : dd[3];
  const float del = __shfl(dsel, dsrc);
  if (live && g == 0) delta[(size_t)(seq0 + i) * hq + h] = del;
  const float lse2 = lse[(size_t)(seq0 + ic) * hq + h] * 1.4426950408889634f;

  int ss = 0, se = 0, s0, e0;
  if (num_spans > 0 && find_span(spans, num_spans, seq0 + ic, s0, e0)) {
    ss = s0 - seq0;
    se = e0 - seq0;
  }
  // Keys of the tile's rows: the window below its first row, the span of its
  // first row, up to its last row or the span of its last row.
  int lo = window > 0 ? max(0, r0 - window + 1) : 0;
  int hi = r1;
  if (num_spans > 0) {
    if (find_span(spans, num_spans, seq0 + r0, s0, e0)) lo = min(lo, max(s0 - seq0, 0));
    if (find_span(spans, num_spans, seq0 + r1 - 1, s0, e0)) hi = max(hi, min(e0 - seq0, L));
  }
  // Key tiles on the grid of multiples of kBwdTile from the sequence start
  // (the forward's): which keys share an MFMA then depends on the keys
  // alone, not on where the row tile starts.  Keys below the window edge in
  // the first tile are masked for every row.
  lo &= ~(kBwdTile - 1);

  // The wave accumulates dQ^T for its quarter of the head dim (columns
  // w*D/4 + 16*db + ...) and all four row blocks of the workgroup.
  constexpr int kDq = C::kDb / 4;
  f32x4 acc[kDq][4];
#pragma unroll
  for (int db = 0; db < kDq; ++db) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[db][rb] = f32x4{};
  }

  // Tile loads: through registers, or at head dim 512 (where the
  // accumulators and operands fill the registers) straight to LDS with
  // direct loads of one 1 KB key row each, from a resource that ends at key
  // hi (keys past it load as zeros).
  constexpr bool kDma = D * 2 == 1024;
  TileRegs<D> kr, vr;  // unused with direct loads
  u32x4 krs{}, vrs{};
  if constexpr (kDma) {
    const size_t base = ((size_t)seq0 * hkv + kvh) * D;
    const int nb = hi * hkv * D * 2;
    krs = buffer_rsrc(k + base, nb);
    vrs = buffer_rsrc(v + base, nb);
  }
  auto fetch = [&](int k0) {
    kr.fetch([&](int r) -> const bf16* {
      return k0 + r < hi ? k + ((size_t)(seq0 + k0 + r) * hkv + kvh) * D : nullptr;
    }, tid);
    vr.fetch([&](int r) -> const bf16* {
      return k0 + r < hi ? v + ((size_t)(seq0 + k0 + r) * hkv + kvh) * D : nullptr;
    }, tid);
  };
  // Key rows 8w .. 8w + 7 of the tile at k0 (this wave's share) into `buf`.
  // Load e of this wave's share: K (e even) or V (e odd) of row 8w + e / 2.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto dma_load = [&](int k0, int buf, int e) {
    const int r = (kBwdTile / 4) * wu + e / 2;
    const uint32_t off = (uint32_t)((k0 + r) * hkv * D * 2);
    if (e % 2 == 0) dma_row(lds_addr(kts[buf] + r * C::kLd), krs, off, lane);
    else dma_row(lds_addr(vts[buf] + r * C::kLd), vrs, off, lane);
  };
  // Tile t sits in buffer t & 1; tile t+1's loads fly while tile t is used,
  // one barrier per tile.
  if constexpr (kDma) {
#pragma unroll
    for (int e = 0; e < kBwdTile / 2; ++e) dma_load(lo, 0, e);
    wait_vmem();
  } else {
    fetch(lo);
    kr.put(kts[0], tid);
    vr.put(vts[0], tid);
  }
  __syncthreads();
  for (int k0 = lo, t = 0; k0 < hi; k0 += kBwdTile, ++t) {
    const bool more = k0 + kBwdTile < hi;
    if constexpr (!kDma) {
      if (more) fetch(k0 + kBwdTile);
    }
    const bf16* kt = kts[t & 1];
    const bf16* vt = vts[t & 1];
    // S^T and dP^T: keys 16kb + 4g + e of row x.
    // Four independent MFMA chains (S and dP of both key blocks), k-steps
    // outermost.  At head dim 512 (one wave per SIMD, nothing else to run
    // while a read is outstanding) the operands of k-step st + 2 are read
    // while st runs, and the next tile's direct loads are spread over the
    // k-steps (issued at once, each waits for the memory unit to take the
    // one before).
    constexpr int kAhead = D >= 512 ? 3 : 1;
    auto k_op = [&](int st, int kb) {
      return ld_lds_x8(kt + (16 * kb + x) * C::kLd + 32 * st + 8 * g);
    };
    auto v_op = [&](int st, int kb) {
      return ld_lds_x8(vt + (16 * kb + x) * C::kLd + 32 * st + 8 * g);
    };
    bf16x8 ka[kAhead][2], va[kAhead][2];
#pragma unroll
    for (int a = 0; a < kAhead; ++a) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        ka[a][kb] = k_op(a, kb);
        va[a][kb] = v_op(a, kb);
      }
    }
    f32x4 s[2], dp[2];
#pragma unroll
    for (int st = 0; st < C::kSt; ++st) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma16(ka[st % kAhead][kb], qop[st], st == 0 ? f32x4{} : s[kb]);
        dp[kb] = mfma16(va[st % kAhead][kb], dop[st], st == 0 ? f32x4{} : dp[kb]);
        if (st + kAhead < C::kSt) {
          ka[st % kAhead][kb] = k_op(st + kAhead, kb);
          va[st % kAhead][kb] = v_op(st + kAhead, kb);
        }
      }
      if constexpr (kDma) {
        static_assert(!kDma || C::kSt == kBwdTile / 2, "one direct load per k-step");
        if (more) dma_load(k0 + kBwdTile, (t + 1) & 1, st);
      }
    }
    f32x4 ds[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = k0 + 16 * kb + 4 * g + e;
        const float p = masked_exp2<true>(admits(ic, j, window, ss, se) & (j < hi),
                                          __builtin_fmaf(s[kb][e], c2, -lse2));
        ds[kb][e] = p * (dp[kb][e] - del);
      }
    }
    xch[w][lane] = pack8(ds[0], ds[1]);
    __syncthreads();
    // dQ^T[d][row] += K^T[d][key] dS^T[key][row]; each transpose read serves
    // the four row blocks.
#pragma unroll
    for (int db = 0; db < kDq; ++db) {
      const bf16x8 ak = lds_t_operand<C::kLd>(kt, w * (D / 4) + 16 * db, g, x);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[db][rb] = mfma16(ak, xch[rb][lane], acc[db][rb]);
    }
    if constexpr (kDma) {
      wait_vmem();
    } else if (more) {
      kr.put(kts[(t + 1) & 1], tid);
      vr.put(vts[(t + 1) & 1], tid);
    }
    __syncthreads();
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int ir = r0 + 16 * rb + x;
    if (ir >= r1) continue;
    float* out = dq + ((size_t)(seq0 + ir) * hq + h) * D + w * (D / 4) + 4 * g;
#pragma unroll
    for (int db = 0; db < kDq; ++db) {
      float4 wv;
      wv.x = acc[db][rb][0] * scale;
      wv.y = acc[db][rb][1] * scale;
      wv.z = acc[db][rb][2] * scale;
      wv.w = acc[db][rb][3] * scale;
      *reinterpret_cast<float4*>(out + 16 * db) = wv;
    }
  }
}

// dk and dv of 64 keys of one KV head.
template <int D>
__global__ __launch_bounds__(kBwdThreads)
void bwd_dkv_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ v, const float* __restrict__ lse,
                    const bf16* __restrict__ dout, const float* __restrict__ delta,
                    float* __restrict__ dk, float* __restrict__ dv,
                    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ spans,
                    int num_spans, int hq, int hkv, int window, float scale, float c2,
                   int tiles, int nseq) {
  using C = BwdCfg<D>;
  constexpr int NP = C::kPairs;
  __shared__ __attribute__((aligned(16))) bf16 qts[2][NP * C::kLd];
  __shared__ __attribute__((aligned(16))) bf16 dts[2][NP * C::kLd];
  __shared__ __attribute__((aligned(16))) float plses[2][NP], pdels[2][NP];
  __shared__ __attribute__((aligned(16))) int prows[2][NP], psss[2][NP], pses[2][NP];
  // P and dS of every wave's key block as B operands (bf16x8 per lane).
  __shared__ bf16x8 xch[2][C::kHalves][4][64];
  // Item = (key tile, KV head, sequence), key tiles numbered from the start
  // of the sequence (the most rows first); neighbouring key tiles share most
  // of their rows.
  int tile, b, kvh;
  if (!bwd_item(tiles, hkv, nseq, tile, b, kvh)) return;
  const int G = hq / hkv;
  const int seq0 = cu_seqlens[b], L = cu_seqlens[b + 1] - seq0;
  const int j0 = tile * kBwdRows;
  if (j0 >= L) return;
  const int j1 = min(j0 + kBwdRows, L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int x = lane & 15, g = lane >> 4;
  const int j = j0 + 16 * w + x;
  const bool live = j < j1;
  const int jc = live ? j : j0;
  const size_t ko = ((size_t)(seq0 + jc) * hkv + kvh) * D;

  // K and V as B operands (B[d][key]).
  bf16x8 kop[C::kSt], vop[C::kSt];
#pragma unroll
  for (int st = 0; st < C::kSt; ++st) {
    kop[st] = ld_global_x8(k + ko + 32 * st + 8 * g);
    vop[st] = ld_global_x8(v + ko + 32 * st + 8 * g);
  }
  // The wave accumulates dK^T and dV^T for its quarter of the head dim
  // (columns w*D/4 + 16*db + ...) and all four key blocks of the workgroup.
  constexpr int kDq = C::kDb / 4;
  f32x4 ak[kDq][4], av[kDq][4];
#pragma unroll
  for (int db = 0; db < kDq; ++db) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      ak[db][kb] = f32x4{};
      av[db][kb] = f32x4{};
    }
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
  const int n_pairs = (hi - lo) * G;
  constexpr bool kDma = !C::kPrefetch;
  TileRegs<D, kDma ? kBwdTile : NP> qr, dr;  // unused with direct loads
  int mrow = -1, mss = 0, mse = 0;
  float ml2 = 0.f, mdl = 0.f;
  // Direct loads (head dim 512): the Q and dout rows of rows [lo, hi) of
  // this sequence, so that the pairs past the last one load as zeros.
  u32x4 qrs{}, drs{};
  if constexpr (kDma) {
    static_assert(D * 2 == 1024 && NP % 4 == 0, "one 1 KB row per direct load");
    const size_t base = ((size_t)(seq0 + lo) * hq + kvh * G) * D;
    const int nb = (hi - lo) * hq * D * 2;
    qrs = buffer_rsrc(q + base, nb);
    drs = buffer_rsrc(dout + base, nb);
  }
  // Pair p = (row - lo) * G + head.  Tiles are visited in order, NP pairs
  // each, so a fixed slot's (row - lo, head) advances by (NP / G, NP % G) per
  // tile, with a carry: the loop needs no division.
  const int adv_q = NP / G, adv_m = NP % G;
  auto advance = [&](int& pq, int& pm) {
    pq += adv_q;
    pm += adv_m;
    if (pm >= G) {
      pm -= G;
      ++pq;
    }
  };
  // Direct loads: this wave's slots are pair rows 8w .. 8w + 7 of a tile.
  constexpr int kSlots = NP / 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int sq[kSlots], sm[kSlots];
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    sq[i] = (kSlots * wu + i) / G;
    sm[i] = (kSlots * wu + i) % G;
  }
  // The next tile's row offsets (slot i), then its loads: row e / 2 of Q
  // (e even) or dout (e odd) into buffer `buf`.
  auto dma_offsets = [&](uint32_t* off) {
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      off[i] = (uint32_t)((sq[i] * hq + sm[i]) * D * 2);
      advance(sq[i], sm[i]);
    }
  };
  auto dma_load = [&](int e, int buf, const uint32_t* off) {
    const int r = kSlots * wu + e / 2;
    if (e % 2 == 0) dma_row(lds_addr(qts[buf] + r * C::kLd), qrs, off[e / 2], lane);
    else dma_row(lds_addr(dts[buf] + r * C::kLd), drs, off[e / 2], lane);
  };
  // Metadata lanes (tid < NP): pair w0 + tid of the next tile.
  int lq = tid / G, lm = tid % G;
  auto fetch = [&](int w0) {
    auto pair_src = [&](const bf16* base, int r) -> const bf16* {
      const int pw = w0 + r;
      if (pw >= n_pairs) return nullptr;
      return base + ((size_t)(seq0 + lo + pw / G) * hq + kvh * G + pw % G) * D;
    };
    if constexpr (!kDma) {
      qr.fetch([&](int r) { return pair_src(q, r); }, tid);
      dr.fetch([&](int r) { return pair_src(dout, r); }, tid);
    }
    if (tid < NP) {
      mrow = -1;
      mss = mse = 0;
      ml2 = mdl = 0.f;
      if (lq < hi - lo) {
        mrow = lo + lq;
        const size_t ro = (size_t)(seq0 + mrow) * hq + kvh * G + lm;
        ml2 = lse[ro] * 1.4426950408889634f;
        mdl = delta[ro];
        if (num_spans > 0 && find_span(spans, num_spans, seq0 + mrow, s0, e0)) {
          mss = s0 - seq0;
          mse = e0 - seq0;
        }
      }
      advance(lq, lm);
    }
  };
  auto put = [&](int buf) {
    if constexpr (!kDma) {
      qr.put(qts[buf], tid);
      dr.put(dts[buf], tid);
    }
    if (tid < NP) {
      prows[buf][tid] = mrow;
      psss[buf][tid] = mss;
      pses[buf][tid] = mse;
      plses[buf][tid] = ml2;
      pdels[buf][tid] = mdl;
    }
  };
  // Pair tile t sits in buffer t & 1; tile t+1's loads fly while tile t is
  // used (in registers with prefetch; straight to LDS with direct loads).
  if (n_pairs > 0) {
    if constexpr (kDma) {
      uint32_t off[kSlots];
      dma_offsets(off);
#pragma unroll
      for (int e = 0; e < 2 * kSlots; ++e) dma_load(e, 0, off);
    }
    fetch(0);
    put(0);
  }
  if constexpr (kDma) wait_vmem();
  // K and V have arrived: the loop waits only for the tile it has in flight,
  // at the end of each step.
#pragma unroll
  for (int st = 0; st < C::kSt; ++st) {
    arrived(kop[st]);
    arrived(vop[st]);
  }
  __syncthreads();
  for (int w0 = 0, t = 0; w0 < n_pairs; w0 += NP, ++t) {
    const bool more = w0 + NP < n_pairs;
    // Direct loads of the next tile: offsets here, the loads spread over this
    // step's score MFMAs (issued at once, each waits for the memory unit to
    // take the one before, and nothing else would run meanwhile); its
    // metadata after the first barrier, behind them (ahead of them, a span
    // lookup's waits would wait for them).  Without direct loads, the next
    // tile's registers and metadata now.
    uint32_t doff[kSlots];
    if constexpr (kDma) {
      if (more) dma_offsets(doff);
    } else {
      if (more) fetch(w0 + NP);
    }
    const int cb = t & 1;
    const bf16* qt = qts[cb];
    const bf16* dt = dts[cb];
    const int* prow = prows[cb];
    const int* pss = psss[cb];
    const int* pse = pses[cb];
    const float* plse = plses[cb];
    const float* pdel = pdels[cb];
    // Per half hf: S and dP of pairs 32hf + 16pb + 4g + e for key x of the
    // wave's key block, posted for every wave.
#pragma unroll
    for (int hf = 0; hf < C::kHalves; ++hf) {
      const bf16* qh = qt + 32 * hf * C::kLd;
      const bf16* dh = dt + 32 * hf * C::kLd;
      // MFMA k = (pair block, k-step), pair blocks outermost (at head dim
      // 512 the other order spills); the operands of k + kAhead - 1 are read
      // while k runs.
      constexpr int kK = 2 * C::kSt;
      constexpr int kAhead = kK < 4 ? kK : 4;
      auto q_op = [&](int k) {
        return ld_lds_x8(qh + (16 * (k / C::kSt) + x) * C::kLd + 32 * (k % C::kSt) + 8 * g);
      };
      auto d_op = [&](int k) {
        return ld_lds_x8(dh + (16 * (k / C::kSt) + x) * C::kLd + 32 * (k % C::kSt) + 8 * g);
      };
      bf16x8 qb[kAhead], dbf[kAhead];
#pragma unroll
      for (int a = 0; a < kAhead; ++a) {
        qb[a] = q_op(a);
        dbf[a] = d_op(a);
      }
      f32x4 s[2], dp[2];
#pragma unroll
      for (int k = 0; k < kK; ++k) {
        const int pb = k / C::kSt, st = k % C::kSt;
        s[pb] = mfma16(qb[k % kAhead], kop[st], st == 0 ? f32x4{} : s[pb]);
        dp[pb] = mfma16(dbf[k % kAhead], vop[st], st == 0 ? f32x4{} : dp[pb]);
        if (k + kAhead < kK) {
          qb[k % kAhead] = q_op(k + kAhead);
          dbf[k % kAhead] = d_op(k + kAhead);
        }
        if constexpr (kDma) {
          static_assert(!kDma || kK == 4 * kSlots, "one direct load per two MFMA k-steps");
          if (k % 2 == 0 && more) dma_load(k / 2, cb ^ 1, doff);
        }
      }
      f32x4 p[2], ds[2];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        // The lane's four consecutive pairs: one 16-byte read per array.
        const int t0 = 32 * hf + 16 * pb + 4 * g;
        const int4 rw = *reinterpret_cast<const int4*>(prow + t0);
        const int4 sa = *reinterpret_cast<const int4*>(pss + t0);
        const int4 sb = *reinterpret_cast<const int4*>(pse + t0);
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(plse + t0);
        const f32x4 dl = *reinterpret_cast<const f32x4*>(pdel + t0);
        const int rv[4] = {rw.x, rw.y, rw.z, rw.w};
        const int av0[4] = {sa.x, sa.y, sa.z, sa.w};
        const int av1[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = masked_exp2<(D <= 256)>(
              (rv[e] >= 0) && admits<(D <= 256)>(rv[e], jc, window, av0[e], av1[e]),
              __builtin_fmaf(s[pb][e], c2, -l2[e]));
          p[pb][e] = pv;
          ds[pb][e] = pv * (dp[pb][e] - dl[e]);
        }
      }
      xch[0][hf][w][lane] = pack8(p[0], p[1]);
      xch[1][hf][w][lane] = pack8(ds[0], ds[1]);
    }
    __syncthreads();
    if constexpr (kDma) {
      if (more) fetch(w0 + NP);
    }
    // dV^T[d][key] += dout^T[d][pair] P[pair][key];  dK^T += Q^T dS.  Each
    // transpose read serves the four key blocks; halves in pair order.
#pragma unroll
    for (int db = 0; db < kDq; ++db) {
      const int c0 = w * (D / 4) + 16 * db;
#pragma unroll
      for (int hf = 0; hf < C::kHalves; ++hf) {
        const bf16x8 ad = lds_t_operand<C::kLd>(dt + 32 * hf * C::kLd, c0, g, x);
        const bf16x8 aq = lds_t_operand<C::kLd>(qt + 32 * hf * C::kLd, c0, g, x);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          av[db][kb] = mfma16(ad, xch[0][hf][kb][lane], av[db][kb]);
          ak[db][kb] = mfma16(aq, xch[1][hf][kb][lane], ak[db][kb]);
        }
      }
    }
    if (more) put(cb ^ 1);
    // The next step's loads reuse these registers: wait for this step's here
    // (they were stored above whenever they were issued), not mid-step.
    arrived(mrow);
    arrived(mss);
    arrived(mse);
    arrived(ml2);
    arrived(mdl);
    if constexpr (kDma) wait_vmem();
    __syncthreads();
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int jk = j0 + 16 * kb + x;
    if (jk >= j1) continue;
    const size_t kko = ((size_t)(seq0 + jk) * hkv + kvh) * D + w * (D / 4) + 4 * g;
#pragma unroll
    for (int db = 0; db < kDq; ++db) {
      float4 wk, wv;
      wk.x = ak[db][kb][0] * scale;
      wk.y = ak[db][kb][1] * scale;
      wk.z = ak[db][kb][2] * scale;
      wk.w = ak[db][kb][3] * scale;
      wv.x = av[db][kb][0];
      wv.y = av[db][kb][1];
      wv.z = av[db][kb][2];
      wv.w = av[db][kb][3];
      *reinterpret_cast<float4*>(dk + kko + 16 * db) = wk;
      *reinterpret_cast<float4*>(dv + kko + 16 * db) = wv;
    }
  }
}

// dk and dv of 64 keys of one KV head, two kinds of waves (head dim 256).
// Waves 0-3 (score waves) form S, dP, P and dS of 32 pairs for key
// block w and post P and dS; waves 4-7 (gradient waves) accumulate dV^T and
// dK^T for column quarter w-4 of all four key blocks from the previous
// step's posts.  Pair tiles sit in a ring of three LDS buffers: during step
// t the score waves read tile t, the gradient waves tile t-1, and tile t+1
// lands.  Every accumulator sees the same MFMAs in the same order as in
// bwd_dkv_kernel, so the bytes are the same.
template <int D>
__global__ __launch_bounds__(2 * kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_ws_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                       const bf16* __restrict__ v, const float* __restrict__ lse,
                       const bf16* __restrict__ dout, const float* __restrict__ delta,
                       float* __restrict__ dk, float* __restrict__ dv,
                       const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ spans,
                       int num_spans, int hq, int hkv, int window, float scale, float c2,
                   int tiles, int nseq) {
  using C = BwdCfg<D>;
  constexpr int NP = kBwdTile;
  constexpr int kRing = 3;
  // The gradient waves load every pair tile (the score waves, the longer
  // path, would otherwise stall on their issue): loader lt = tid - 256 holds
  // 16-byte chunks lt + 256u of Q and dout, and lanes lt < NP the metadata.
  constexpr int kPer = NP * D / 8 / kBwdThreads;   // chunks per loader per tensor
  static_assert((NP * D / 8) % kBwdThreads == 0, "whole chunks per loader");
  __shared__ __attribute__((aligned(16))) bf16 qts[kRing][NP * C::kLd];
  __shared__ __attribute__((aligned(16))) bf16 dts[kRing][NP * C::kLd];
  __shared__ __attribute__((aligned(16))) float plses[kRing][NP], pdels[kRing][NP];
  __shared__ __attribute__((aligned(16))) int prows[kRing][NP], psss[kRing][NP], pses[kRing][NP];
  __shared__ bf16x8 xch[2][2][4][64];   // [step parity][P, dS][key block][lane]
  // Item = (key tile, KV head, sequence), key tiles numbered from the start
  // of the sequence (the most rows first); neighbouring key tiles share most
  // of their rows.
  int tile, b, kvh;
  if (!bwd_item(tiles, hkv, nseq, tile, b, kvh)) return;
  const int G = hq / hkv;
  const int seq0 = cu_seqlens[b], L = cu_seqlens[b + 1] - seq0;
  const int j0 = tile * kBwdRows;
  if (j0 >= L) return;
  const int j1 = min(j0 + kBwdRows, L);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool scorer = wv < 4;
  const int w = wv & 3;
  const int x = lane & 15, g = lane >> 4;

  int s0, e0;
  int lo = j0;
  int hi = window > 0 ? min(L, j1 - 1 + window) : L;
  if (num_spans > 0) {
    if (find_span(spans, num_spans, seq0 + j0, s0, e0)) lo = min(lo, max(s0 - seq0, 0));
    if (find_span(spans, num_spans, seq0 + j1 - 1, s0, e0)) hi = max(hi, min(e0 - seq0, L));
  }
  const int n_pairs = (hi - lo) * G;
  const int n_tiles = (n_pairs + NP - 1) / NP;

  const int lt = tid - kBwdThreads;
  bf16x8 qr[kPer], dr[kPer];
  int mrow = -1, mss = 0, mse = 0;
  float ml2 = 0.f, mdl = 0.f;
  auto fetch = [&](int t) {
    if (scorer) return;
    const int w0 = t * NP;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = lt + u * kBwdThreads;
      const int pw = w0 + e / (D / 8), c = 8 * (e % (D / 8));
      if (pw < n_pairs) {
        const size_t ro = ((size_t)(seq0 + lo + pw / G) * hq + kvh * G + pw % G) * D + c;
        qr[u] = ld_global_x8(q + ro);
        dr[u] = ld_global_x8(dout + ro);
      } else {
        qr[u] = bf16x8{};
        dr[u] = bf16x8{};
      }
    }
    if (lt < NP) {
      const int pw = w0 + lt;
      mrow = -1;
      mss = mse = 0;
      ml2 = mdl = 0.f;
      if (pw < n_pairs) {
        mrow = lo + pw / G;
        const size_t ro = (size_t)(seq0 + mrow) * hq + kvh * G + pw % G;
        ml2 = lse[ro] * 1.4426950408889634f;
        mdl = delta[ro];
        if (num_spans > 0 && find_span(spans, num_spans, seq0 + mrow, s0, e0)) {
          mss = s0 - seq0;
          mse = e0 - seq0;
        }
      }
    }
  };
  auto put = [&](int buf) {
    if (scorer) return;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = lt + u * kBwdThreads;
      const int r = e / (D / 8), c = 8 * (e % (D / 8));
      st_lds_x8(qts[buf] + r * C::kLd + c, qr[u]);
      st_lds_x8(dts[buf] + r * C::kLd + c, dr[u]);
    }
    if (lt < NP) {
      prows[buf][lt] = mrow;
      psss[buf][lt] = mss;
      pses[buf][lt] = mse;
      plses[buf][lt] = ml2;
      pdels[buf][lt] = mdl;
    }
  };
  // The next step's loads reuse the fetch registers: wait for this step's at
  // the end of the step (where put stored them), not at the next one's start.
  auto settle_fetch = [&]() {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      arrived(qr[u]);
      arrived(dr[u]);
    }
    arrived(mrow);
    arrived(mss);
    arrived(mse);
    arrived(ml2);
    arrived(mdl);
  };

  // Score waves: K and V of key j as B operands, loaded while the first
  // tile is.
  const int j = j0 + 16 * w + x;
  const int jc = j < j1 ? j : j0;
  bf16x8 kop[C::kSt], vop[C::kSt];
  if (scorer) {
    const size_t ko = ((size_t)(seq0 + jc) * hkv + kvh) * D;
#pragma unroll
    for (int st = 0; st < C::kSt; ++st) {
      kop[st] = ld_global_x8(k + ko + 32 * st + 8 * g);
      vop[st] = ld_global_x8(v + ko + 32 * st + 8 * g);
    }
  }
  if (n_tiles > 0) {
    fetch(0);
    put(0);
  }
  __syncthreads();
  // Each kind runs its own loop (so that its registers do not overlap the
  // other kind's); both pass n_tiles + 1 barriers.
  if (scorer) {
    // K and V have arrived: the loop waits only for the tile in flight.
#pragma unroll
    for (int st = 0; st < C::kSt; ++st) {
      arrived(kop[st]);
      arrived(vop[st]);
    }
    for (int t = 0; t <= n_tiles; ++t) {
      if (t < n_tiles) {
        const int cb = t % kRing;
        const bf16* qt = qts[cb];
        const bf16* dt = dts[cb];
        f32x4 sc[2], dp[2];
#pragma unroll
        for (int st = 0; st < C::kSt; ++st) {
#pragma unroll
          for (int pb = 0; pb < 2; ++pb) {
            const bf16x8 qa = ld_lds_x8(qt + (16 * pb + x) * C::kLd + 32 * st + 8 * g);
            const bf16x8 da = ld_lds_x8(dt + (16 * pb + x) * C::kLd + 32 * st + 8 * g);
            sc[pb] = mfma16(qa, kop[st], st == 0 ? f32x4{} : sc[pb]);
            dp[pb] = mfma16(da, vop[st], st == 0 ? f32x4{} : dp[pb]);
          }
        }
        f32x4 p[2], ds[2];
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          const int t0 = 16 * pb + 4 * g;
          const int4 rw = *reinterpret_cast<const int4*>(prows[cb] + t0);
          const int4 sa = *reinterpret_cast<const int4*>(psss[cb] + t0);
          const int4 sb = *reinterpret_cast<const int4*>(pses[cb] + t0);
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(plses[cb] + t0);
          const f32x4 dl = *reinterpret_cast<const f32x4*>(pdels[cb] + t0);
          const int rv[4] = {rw.x, rw.y, rw.z, rw.w};
          const int av0[4] = {sa.x, sa.y, sa.z, sa.w};
          const int av1[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = masked_exp2<true>(
                (rv[e] >= 0) & admits(rv[e], jc, window, av0[e], av1[e]),
                __builtin_fmaf(sc[pb][e], c2, -l2[e]));
            p[pb][e] = pv;
            ds[pb][e] = pv * (dp[pb][e] - dl[e]);
          }
        }
        xch[t & 1][0][w][lane] = pack8(p[0], p[1]);
        xch[t & 1][1][w][lane] = pack8(ds[0], ds[1]);
      }
      __syncthreads();
    }
    return;
  }
  // Gradient waves: dK^T, dV^T for columns w*D/4 + 16*db + 4g + i, key blocks kb.
  constexpr int kDq = C::kDb / 4;
  f32x4 ak[kDq][4], av[kDq][4];
#pragma unroll
  for (int db = 0; db < kDq; ++db) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      ak[db][kb] = f32x4{};
      av[db][kb] = f32x4{};
    }
  }
  for (int t = 0; t <= n_tiles; ++t) {
    const bool more = t + 1 < n_tiles;
    if (more) fetch(t + 1);
    if (t >= 1) {
      const int pbuf = (t - 1) % kRing;
      const bf16* qt = qts[pbuf];
      const bf16* dt = dts[pbuf];
      bf16x8 px[4], dx[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        px[kb] = xch[(t - 1) & 1][0][kb][lane];
        dx[kb] = xch[(t - 1) & 1][1][kb][lane];
      }
#pragma unroll
      for (int db = 0; db < kDq; ++db) {
        const int c0 = w * (D / 4) + 16 * db;
        const bf16x8 ad = lds_t_operand<C::kLd>(dt, c0, g, x);
        const bf16x8 aq = lds_t_operand<C::kLd>(qt, c0, g, x);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          av[db][kb] = mfma16(ad, px[kb], av[db][kb]);
          ak[db][kb] = mfma16(aq, dx[kb], ak[db][kb]);
        }
      }
    }
    if (more) put((t + 1) % kRing);
    settle_fetch();
    __syncthreads();
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int jk = j0 + 16 * kb + x;
    if (jk >= j1) continue;
    const size_t kko = ((size_t)(seq0 + jk) * hkv + kvh) * D + w * (D / 4) + 4 * g;
#pragma unroll
    for (int db = 0; db < kDq; ++db) {
      float4 wk, wvv;
      wk.x = ak[db][kb][0] * scale;
      wk.y = ak[db][kb][1] * scale;
      wk.z = ak[db][kb][2] * scale;
      wk.w = ak[db][kb][3] * scale;
      wvv.x = av[db][kb][0];
      wvv.y = av[db][kb][1];
      wvv.z = av[db][kb][2];
      wvv.w = av[db][kb][3];
      *reinterpret_cast<float4*>(dk + kko + 16 * db) = wk;
      *reinterpret_cast<float4*>(dv + kko + 16 * db) = wvv;
    }
  }
}

namespace {

template <int D>
hipError_t launch_bwd_d(const BackwardArgs& a, hipStream_t stream) {
  const int tiles = (a.max_seqlen + kBwdRows - 1) / kBwdRows;
  const long long dq_blocks = run_major_blocks(tiles, (long long)a.hq * a.batch);
  const long long kv_blocks = run_major_blocks(tiles, (long long)a.hkv * a.batch);
  if (dq_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)dq_blocks), dim3(kBwdThreads), 0, stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.o,
                     a.lse, (const bf16*)a.dout, a.dq, a.delta, a.cu_seqlens, a.spans,
                     a.num_spans, a.hq, a.hkv, a.window, a.scale, a.c2, tiles, a.batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Head dim 256: dk/dv on the two-kind workgroup; 64 and 512: one kind.
  if constexpr (D == 256)
    hipLaunchKernelGGL(bwd_dkv_ws_kernel<D>, dim3((unsigned)kv_blocks), dim3(2 * kBwdThreads), 0,
                       stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.lse,
                       (const bf16*)a.dout, (const float*)a.delta, a.dk, a.dv, a.cu_seqlens,
                       a.spans, a.num_spans, a.hq, a.hkv, a.window, a.scale, a.c2, tiles,
                       a.batch);
  else
    hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3((unsigned)kv_blocks), dim3(kBwdThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.lse,
                       (const bf16*)a.dout, (const float*)a.delta, a.dk, a.dv, a.cu_seqlens,
                       a.spans, a.num_spans, a.hq, a.hkv, a.window, a.scale, a.c2, tiles,
                       a.batch);
  return hipGetLastError();
}

}  // namespace

int backward_rows_per_tile(int d) {
  return (d == 64 || d == 256 || d == 512) ? kBwdRows : 0;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream, const char** kernel) {
  switch (a.d) {
    case 64:
      *kernel = "bwd_dq_kernel<64>+bwd_dkv_kernel<64>";
      return launch_bwd_d<64>(a, stream);
    case 256:
      *kernel = "bwd_dq_kernel<256>+bwd_dkv_ws_kernel<256>";
      return launch_bwd_d<256>(a, stream);
    case 512:
      *kernel = "bwd_dq_kernel<512>+bwd_dkv_kernel<512>";
      return launch_bwd_d<512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace invattn
