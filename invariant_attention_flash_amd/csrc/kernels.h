// kernels.h -- host-side launch interface between the C ABI (api.hip) and the
// kernel translation units (prefill.hip, decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace invattn {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;
  const int32_t* spans;
  int32_t num_spans;
  int32_t batch;
  int32_t max_seqlen;
  int32_t hq;
  int32_t hkv;
  int32_t d;
  int32_t window;  // -1 = none
  float c2;        // fl32(scale * log2(e))
  // Paged layout (attn_prefill_paged): k / v are the caches, max_seqlen
  // bounds the query rows of one sequence.  q_start == nullptr: contiguous.
  const int32_t* q_start = nullptr;
  const int32_t* block_table = nullptr;
  int32_t max_blocks = 0;
  int32_t num_blocks = 0;
  int32_t max_context = 0;
};

// Position tiles the grid covers per sequence: the query rows of a paged
// chunk start anywhere inside a tile, so one more tile is needed.
inline int prefill_grid_tiles(const PrefillArgs& a, int positions) {
  const int t = (a.max_seqlen + positions - 1) / positions;
  return a.q_start != nullptr ? t + 1 : t;
}

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  int32_t batch;
  int32_t max_seq_len;
  int32_t num_blocks;
  int32_t hq;
  int32_t hkv;
  int32_t d;
  int32_t window;
  float c2;
  float* workspace;
  int32_t n_chunks;  // ceil(max_seq_len / chunk)
  void* o;
};

// Tile geometry of the kernel instance chosen for (head_dim, group); fixed
// per instance, never dependent on batch or sequence lengths.
struct PrefillSchedule {
  int rows;       // query rows (position x head) per workgroup
  int positions;  // sequence positions per workgroup
  int bn;         // keys per KV tile
  int threads;
};

// Prefill block order.  The hardware hands consecutive workgroups to the 8
// XCDs in turn (each XCD has its own L2); workgroups that read the same K/V
// rows (consecutive position tiles of one sequence and KV head) should share
// an L2.  Block i therefore takes logical work item
//   chunk (i/8)/kXcdChunk * 8 + i%8, item (i/8) % kXcdChunk of that chunk,
// so each XCD walks runs of kXcdChunk consecutive tiles.  The grid is padded
// to a multiple of 8*kXcdChunk; items past the end exit at once.  Only the
// placement changes: a row's arithmetic never depends on its block.
constexpr int kXcds = 8;
constexpr int kXcdChunk = 8;

__host__ __device__ inline long long xcd_padded_blocks(long long n) {
  const long long q = (long long)kXcds * kXcdChunk;
  return (n + q - 1) / q * q;
}

__device__ inline long long xcd_logical_block(long long i) {
  const long long x = i % kXcds, j = i / kXcds;
  return ((j / kXcdChunk) * kXcds + x) * kXcdChunk + j % kXcdChunk;
}

bool prefill_schedule(int d, int group, PrefillSchedule* s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Head dim 512 (prefill_wide.hip); prefill_schedule / launch_prefill
// dispatch to these.
bool prefill_wide_schedule(int d, int group, PrefillSchedule* s);
hipError_t launch_prefill_wide(const PrefillArgs& a, hipStream_t stream);

// Head dim 256 (prefill_split.hip): the PV product split over head-dim
// columns across the waves of a workgroup.
bool prefill_split_schedule(int d, int group, PrefillSchedule* s);
hipError_t launch_prefill_split(const PrefillArgs& a, hipStream_t stream);
// Head dim 256 (prefill_ws.hip): score waves and PV waves, two per SIMD.
bool prefill_ws_schedule(int d, int group, PrefillSchedule* s);
hipError_t launch_prefill_ws(const PrefillArgs& a, hipStream_t stream);

// Attention backward (backward.hip): dq and delta (one kernel), then dk and
// dv (a second kernel reading delta), on the caller's stream.
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // [T, hq] scratch
  const int32_t* cu_seqlens;
  const int32_t* spans;
  int32_t num_spans;
  int32_t batch;
  int32_t max_seqlen;
  int32_t hq;
  int32_t hkv;
  int32_t d;
  int32_t window;
  float scale;
  float c2;  // fl32(scale * log2(e))
};
int backward_rows_per_tile(int d);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);

constexpr int kDecodeChunk = 512;  // keys per split chunk (fixed; ATTN_DECODE_CHUNK)
constexpr int kDecodeStage = 16;   // keys per pipeline stage inside a chunk (one cache block)
constexpr int decode_record_floats(int d) { return d + 4; }  // acc[d], m, l, pad

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace invattn
