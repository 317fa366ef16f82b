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
// chunk one 16-token cache block at a time, ascending.  The K and V rows of
// a block stream HBM -> LDS with direct loads (16 B per lane) into a ring of
// kStages buffers, so several blocks are in flight while one is computed;
// only blocks that hold attended keys are read, and slots past the sequence
// end read its last key (then masked, p = 0).  Every wave computes the same
// S^T = K Q^T (v_mfma_f32_16x16x32_bf16; the G query heads of the group are
// the 16 MFMA columns, padded with zero queries) and so the same online
// softmax state; each wave owns a quarter of the head dim for
// O^T += V^T P^T (v_mfma_f32_16x16x16_bf16, V^T by the LDS transpose read).
// The record (acc[D], m, l) of the chunk goes to the workspace.
//
// Merge kernel: one workgroup per (query head, sequence) folds the chunk
// records in ascending chunk order (m' = max(m, m_c); acc = acc*2^(m-m') +
// acc_c*2^(m_c-m'); l likewise), then o = bf16_rne(acc / l).
#include "device_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace invattn {

// Reference-max hysteresis inside a chunk (log2 units), as in prefill.
constexpr float kDecodeRescale = 8.0f;

// Two waves per SIMD with the two-stage ring: registers are capped at 256 per
// lane, and two workgroups share a CU (two 32 KB stages each at head dim
// 512), so one workgroup's loads land while the other computes.
constexpr int kDecodeOcc = 2;

template <int D_, int G_, int NST_, int WAVES_>
struct DecodeCfg {
  static constexpr bool kAliasKV = false;  // V read from the K cache (KvAliasOf<> sets it)
  // Waves per SIMD the registers are sized for: the deep ring (four 32 KB
  // stages at head dim 512) leaves room for one workgroup per CU.
  static constexpr int kOcc = NST_ >= 4 ? 1 : kDecodeOcc;
  static constexpr int D = D_, G = G_;
  static constexpr int kWaves = WAVES_;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kStages = NST_;
  static constexpr int kKeys = 16;                  // keys per stage = one cache block
  static constexpr int kTile = kKeys * D;           // elements per K (or V) stage
  static constexpr int kChunks = D / 8;             // 16-byte chunks per row
  static constexpr int kLoadsTotal = kKeys * kChunks / 64;  // direct loads per tensor per stage
  static constexpr int kLoadWaves = kLoadsTotal < kWaves ? kLoadsTotal : kWaves;
  static constexpr int kLoads = kLoadsTotal / kLoadWaves;   // per loading wave
  static constexpr int kSteps = D / 32;             // 16x16x32 k-steps over d
  static constexpr int kDPerWave = D / kWaves;
  static constexpr int kDBlk = kDPerWave / 16;      // 16-wide output blocks per wave
  static constexpr int kRec = decode_record_floats(D);
  static constexpr int kSwK = kChunks >= 16 ? 15 : kChunks - 1;
  static constexpr int kSwV = kChunks >= 16 ? 14 : kChunks - 2;
  static_assert(G <= 16, "group fits one MFMA column block");
  static_assert(kLoadsTotal * 64 == kKeys * kChunks, "stage load split");
  static_assert(kStages >= 2 && kStages <= 4, "ring depth");
  static_assert(kDPerWave % 16 == 0, "head-dim slice per wave");
};

// Configuration C for a V cache that is the K cache (global layers whose K
// and V share one projection): each block is loaded once, and the V operand
// is read from the K rows in LDS.  The operand values are the same as with a
// separate V cache holding the same bytes, so the output bytes are too.
template <class C>
struct KvAliasOf : C {
  static constexpr bool kAliasKV = true;
};

// Direct loads of cache block `blk` (keys k0 .. k0+15) into stage buffer kv
// (K rows then V rows; K rows only when V aliases K), through buffer
// resources that end at the sequence's last key: slots at or past the
// sequence end land as zeros (and are masked).
template <class C>
__device__ __forceinline__ void issue_block(bf16* kv, const bf16* kc, const bf16* vc,
                                           size_t blk_base, int k0, int L, uint32_t slot_stride,
                                           uint32_t head_off, int wave, int lane) {
  if (wave >= C::kLoadWaves) return;
  const uint32_t row_bytes = slot_stride * 2;
  const int rows = max(min(C::kKeys, L - k0), 0);
  const int nbytes = (int)((uint32_t)rows * row_bytes);
  const u32x4 krs = buffer_rsrc(kc + blk_base + head_off, nbytes);
  const u32x4 vrs = buffer_rsrc(vc + blk_base + head_off, nbytes);
  const uint32_t kl = lds_addr(kv), vl = C::kAliasKV ? kl : lds_addr(kv + C::kTile);
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    dma_rows<C::kChunks, C::kLoads, 0, C::kSwK>(kl, krs, 0, i, row_bytes, wave, lane);
    if constexpr (!C::kAliasKV)
      dma_rows<C::kChunks, C::kLoads, 1, C::kSwV>(vl, vrs, 0, i, row_bytes, wave, lane);
  }
}

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::kThreads, C::kThreads),
                          amdgpu_waves_per_eu(C::kOcc, C::kOcc)))
void decode_chunk_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                         const bf16* __restrict__ vc, const int32_t* __restrict__ bt,
                         int max_blocks, const int32_t* __restrict__ seq_lens, int max_seq_len,
                         int num_blocks, int hq, int hkv, int window, float c2,
                         float* __restrict__ ws, int n_chunks) {
  constexpr int D = C::D, G = C::G;
  // Stage buffers: K rows then V rows, or K rows only when V aliases K (the
  // smaller footprint lets more workgroups share a CU).
  constexpr int kStage = C::kAliasKV ? C::kTile : 2 * C::kTile;
  __shared__ __attribute__((aligned(1024))) bf16 kv0[kStage];
  __shared__ __attribute__((aligned(1024))) bf16 kv1[kStage];
  __shared__ __attribute__((aligned(1024))) bf16 kv2[C::kStages > 2 ? kStage : 8];
  __shared__ __attribute__((aligned(1024))) bf16 kv3[C::kStages > 3 ? kStage : 8];

  // Grid (KV head, chunk, sequence): the KV heads of one chunk are
  // neighbours in dispatch order, so the rows they read from each cache block
  // (interleaved by head) are fetched together.
  const int b = blockIdx.z, g = blockIdx.x, c = blockIdx.y;
  int L = seq_lens[b];
  L = min(L, min(max_seq_len, max_blocks * 16));
  if (L <= 0) return;
  const int kv_lo = window > 0 ? max(0, L - window) : 0;
  const int c0 = c * kDecodeChunk;
  const int c1 = min(c0 + kDecodeChunk, L);
  const int a0 = max(c0, kv_lo);
  if (a0 >= c1) return;
  const int kb0 = a0 / C::kKeys, kb1 = (c1 - 1) / C::kKeys + 1;  // cache blocks [kb0, kb1)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const bool qv = col < G;
  const int head = g * G + (qv ? col : 0);

  const int32_t* table = bt + (size_t)b * max_blocks;
  const uint32_t slot_stride = (uint32_t)hkv * D;
  const uint32_t head_off = (uint32_t)g * D;
  const size_t block_elems = (size_t)C::kKeys * hkv * D;
  // Table entries are read with scalar loads (constant address space; the
  // index is wave-uniform), waited on with the LDS/scalar counter.  A vector
  // load here would make the compiler wait for every vector load in flight,
  // the direct block loads it cannot see included, and so drain the ring at
  // every step.
  using ConstI32 = const __attribute__((address_space(4))) int32_t;
  auto block_base = [&](int kb) {
    int id = ((ConstI32*)table)[kb];
    id = min(max(id, 0), num_blocks - 1);  // a bad id reads some block, never out of bounds
    return (size_t)id * block_elems;
  };
  issue_block<C>(kv0, kc, vc, block_base(kb0), kb0 * C::kKeys, L, slot_stride, head_off, wave,
                 lane);
  if (C::kStages > 2 && kb0 + 1 < kb1)
    issue_block<C>(kv1, kc, vc, block_base(kb0 + 1), (kb0 + 1) * C::kKeys, L, slot_stride,
                   head_off, wave, lane);
  if (C::kStages > 3 && kb0 + 2 < kb1)
    issue_block<C>(kv2, kc, vc, block_base(kb0 + 2), (kb0 + 2) * C::kKeys, L, slot_stride,
                   head_off, wave, lane);

  // Q^T operand: column col = query head g*G+col, k = d = 32*t + 8*grp + e.
  bf16x8 qr[C::kSteps];
  {
    const bf16* qrow = q + ((size_t)b * hq + head) * D + 8 * grp;
#pragma unroll
    for (int t = 0; t < C::kSteps; ++t) {
      bf16x8 x = ld_global_x8(qrow + 32 * t);
      qr[t] = qv ? x : bf16x8{};
    }
  }
  f32x4 oacc[C::kDBlk];
#pragma unroll
  for (int db = 0; db < C::kDBlk; ++db) oacc[db] = f32x4{};
  float m = kNegInf, l = 0.f;

  // Per-lane LDS offsets.  K: row col, logical chunk 4*t + grp.  V (transpose
  // read): row 4*grp + lg/4, logical chunk 2*db + (lg&3)/2 of this wave's
  // quarter, in-chunk offset 4*(lg&1).
  const int lg = lane & 15;
  const int vrow = 4 * grp + (lg >> 2);
  const int vc1 = wave * C::kDPerWave / 8 + ((lg & 3) >> 1);
  // V rows carry the V swizzle, or the K swizzle when they are the K rows.
  const int vsw = C::kAliasKV ? (vrow & C::kSwK) : ((vrow << 1) & C::kSwV);
  constexpr int kPerStage = C::kAliasKV ? C::kLoads : 2 * C::kLoads;  // loads per stage

  auto step = [&] __device__(const bf16* cur, bf16* pre, int kb) {
    if (kb + C::kStages - 2 < kb1) wait_vmem_keep<C::kStages - 2>(kPerStage);
    else wait_vmem();
    lds_barrier();
    const int nb = kb + C::kStages - 1;
    if (nb < kb1)
      issue_block<C>(pre, kc, vc, block_base(nb), nb * C::kKeys, L, slot_stride, head_off, wave,
                     lane);
    const bf16* ks = cur;
    const bf16* vs = C::kAliasKV ? cur : cur + C::kTile;
    const int k0 = kb * C::kKeys;
    // S^T for keys k0 + [0, 16): lane holds head col, keys 4*grp + i.  The
    // MFMAs form one dependent chain over the head dim, so every K operand is
    // read from LDS before the chain starts (the chain then waits on no LDS
    // latency), and the V operands of the PV product right after.
    const bf16* krow = ks + col * D;
    bf16x8 kop[C::kSteps];
#pragma unroll
    for (int t = 0; t < C::kSteps; ++t)
      kop[t] = ld_lds_x8(krow + (((4 * t + grp) ^ (col & C::kSwK)) << 3));
    const bf16* vr = vs + vrow * D + 4 * (lg & 1);
    bf16x4 vop[C::kDBlk];
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db) vop[db] = ld_lds_tr(vr + (((vc1 + 2 * db) ^ vsw) << 3));
    __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the chain
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int t = 0; t < C::kSteps; ++t) sacc = mfma16(kop[t], qr[t], sacc);
    float x[4];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = k0 + 4 * grp + i;
      x[i] = (qv && j >= kv_lo && j < L) ? sacc[i] : kNegInf;
      tmax = fmaxf(tmax, x[i]);
    }
    // Reduce over the four lane groups holding the same query (xor 16, 32).
    {
      HalfPair hp = row_pair(tmax);  // lanes l, l^16
      tmax = fmaxf(hp.lo, hp.hi);
      hp = half_pair(tmax);          // lanes l, l^32
      tmax = fmaxf(hp.lo, hp.hi);
    }
    tmax *= c2;
    const bool move = tmax > m + kDecodeRescale || (m == kNegInf && tmax != kNegInf);
    const float m_new = move ? tmax : m;
    const float alpha = move ? fast_exp2(m - m_new) : 1.f;
    const float msub = (m_new == kNegInf) ? 0.f : m_new;
    float psum = 0.f;
    bf16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(__builtin_fmaf(x[i], c2, -msub));
      psum += p;
      pb[i] = to_bf16(p);
    }
    {
      // Each step adds the two lanes' sums; addition commutes exactly, so
      // both lanes hold the same value.
      HalfPair hp = row_pair(psum);
      psum = hp.lo + hp.hi;
      hp = half_pair(psum);
      psum = hp.lo + hp.hi;
    }
    l = l * alpha + psum;
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::kDBlk; ++db) oacc[db] *= alpha;
    }
    // O^T += V^T P^T for this wave's quarter of the head dim; operand slot
    // s covers key 4*grp + s on both sides.
#pragma unroll
    for (int db = 0; db < C::kDBlk; ++db) oacc[db] = mfma16k16(vop[db], pb, oacc[db]);
  };
  for (int kb = kb0; kb < kb1;) {
    if constexpr (C::kStages == 2) {
      step(kv0, kv1, kb++);
      if (kb >= kb1) break;
      step(kv1, kv0, kb++);
    } else if constexpr (C::kStages == 3) {
      step(kv0, kv2, kb++);
      if (kb >= kb1) break;
      step(kv1, kv0, kb++);
      if (kb >= kb1) break;
      step(kv2, kv1, kb++);
    } else {
      step(kv0, kv3, kb++);
      if (kb >= kb1) break;
      step(kv1, kv0, kb++);
      if (kb >= kb1) break;
      step(kv2, kv1, kb++);
      if (kb >= kb1) break;
      step(kv3, kv2, kb++);
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

// Merge kernel: one workgroup per (query head, sequence); thread t owns
// head-dim element t.  The fold over chunks is a dependent chain, so the
// records are loaded up to kBatch chunks at a time ahead of their folds: each
// thread its element of every chunk, and lane c of every wave the running max
// and sum of chunk c (read back as wave-uniform values).  A chunk index past
// the last is clamped to it and never folded.  Every element sees the same
// operations in the same chunk order whatever the thread layout.
template <int D>
struct MergeCfg {
  static constexpr int kThreads = D;
  static constexpr int kBatch = 64;  // one round for contexts up to 64 chunks
  static_assert(kThreads % 64 == 0 && kThreads <= 1024, "merge layout");
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(MergeCfg<D>::kThreads,
                                                      MergeCfg<D>::kThreads)))
void decode_merge_kernel(const float* __restrict__ ws, const int32_t* __restrict__ seq_lens,
                         int max_seq_len, int max_blocks, int hq, int window, int n_chunks,
                         bf16* __restrict__ o) {
  constexpr int kBatch = MergeCfg<D>::kBatch;
  constexpr int kRec = decode_record_floats(D);
  const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  bf16* orow = o + ((size_t)b * hq + head) * D + tid;
  int L = seq_lens[b];
  L = min(L, min(max_seq_len, max_blocks * 16));
  if (L <= 0) {
    *orow = to_bf16(0.f);
    return;
  }
  const int kv_lo = window > 0 ? max(0, L - window) : 0;
  const int c_lo = kv_lo / kDecodeChunk, c_hi = (L - 1) / kDecodeChunk;
  const float* base = ws + ((size_t)b * hq + head) * n_chunks * kRec;
  float m = kNegInf, l = 0.f, acc = 0.f;
  for (int c0 = c_lo; c0 <= c_hi; c0 += kBatch) {
    float x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) x[u] = base[(size_t)min(c0 + u, c_hi) * kRec + tid];
    const float* own = base + (size_t)min(c0 + lane, c_hi) * kRec;
    const float mv = own[D], lv = own[D + 1];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (c0 + u <= c_hi) {
        const float mc = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mv), u));
        const float lc = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), u));
        const float m_new = fmaxf(m, mc);
        const float a = fast_exp2(m - m_new);
        const float bc = fast_exp2(mc - m_new);
        l = l * a + lc * bc;
        acc = acc * a + x[u] * bc;
        m = m_new;
      }
    }
  }
  *orow = to_bf16(acc / l);
}

template <class C>
static hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.hkv, a.n_chunks, a.batch);
  if (a.k_cache == a.v_cache)
    hipLaunchKernelGGL(decode_chunk_kernel<KvAliasOf<C>>, grid, dim3(C::kThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache,
                       a.block_table, a.max_blocks, a.seq_lens, a.max_seq_len, a.num_blocks,
                       a.hq, a.hkv, a.window, a.c2, a.workspace, a.n_chunks);
  else
    hipLaunchKernelGGL(decode_chunk_kernel<C>, grid, dim3(C::kThreads), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache,
                       a.block_table, a.max_blocks, a.seq_lens, a.max_seq_len, a.num_blocks,
                       a.hq, a.hkv, a.window, a.c2, a.workspace, a.n_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<C::D>, dim3(a.hq, a.batch),
                     dim3(MergeCfg<C::D>::kThreads), 0, stream,
                     (const float*)a.workspace, a.seq_lens, a.max_seq_len, a.max_blocks, a.hq,
                     a.window, a.n_chunks, (bf16*)a.o);
  return hipGetLastError();
}

// Ring depth and waves per workgroup.  A launch whose chunk grid fits one
// workgroup per CU (small batches) gives each workgroup a ring of four
// stages (more bytes in flight per CU); larger grids use two stages, so two
// workgroups share a CU.  The depth only changes when loads are issued,
// never an operation on the data: both give the same bytes.  Waves: four, or
// one per 16 head-dim columns at head dim 64.
constexpr int kDecodeRingDeep = 4;
constexpr int kDecodeRing = 2;
#define INVATTN_DECODE_TABLE(X) \
  X(64, 1) X(64, 2) X(64, 4) X(64, 8)     \
  X(256, 1) X(256, 2) X(256, 4) X(256, 8) \
  X(512, 1) X(512, 2) X(512, 4) X(512, 8)

namespace {
// Compute units of the current device (queried once per device).
int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cached[dev] = n > 0 ? n : -1;
  }
  return cached[dev];
}
}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, const char** kernel) {
  const int group = a.hq / a.hkv;
  const bool alias = a.k_cache == a.v_cache;
  const long long grid = (long long)a.hkv * a.n_chunks * a.batch;
  const bool deep = grid <= device_cus();
#define X(D, G)                                                                          \
  if (a.d == D && group == G) {                                                          \
    constexpr int W = D / 16 < 4 ? D / 16 : 4;                                           \
    *kernel = alias ? "decode_chunk_kernel<KvAliasOf<" #D "," #G ">>+decode_merge_kernel<" #D ">" \
                    : "decode_chunk_kernel<" #D "," #G ">+decode_merge_kernel<" #D ">";  \
    return deep ? launch_one<DecodeCfg<D, G, kDecodeRingDeep, W>>(a, stream)            \
                : launch_one<DecodeCfg<D, G, kDecodeRing, W>>(a, stream);                \
  }
  INVATTN_DECODE_TABLE(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace invattn
