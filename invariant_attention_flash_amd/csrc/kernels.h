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
  const char* kernel;  // the kernel instance: name<head dim, group, parameters>
};

// Block order (prefill and backward).  The hardware hands consecutive
// workgroups to the 8 XCDs in turn (each XCD has its own L2); workgroups that
// read the same K/V rows (consecutive tiles of one sequence and head) should
// share an L2.  So a group's (a sequence and head) tiles are cut into runs of
// kXcdChunk consecutive tiles, one XCD per run, and the runs are ordered by
// their place in the group first: run k of every group, then run k + 1.
// Callers number a group's tiles most work first, so every XCD starts on
// the longest tiles of every group and ends on short ones, whatever the
// sequence lengths (with groups in order, the tiles of the last and perhaps
// longest sequence would start last: the global backward's key tiles took
// 26.6 ms that way against 24.6 in this order, the global prefill 4.84 ms
// against 4.48).  Run group c (eight runs) is rotated by c over the XCDs,
// so that no XCD keeps the same groups.  Block i: x = i % 8, c = (i/8) /
// kXcdChunk, run 8c + (x + c) % 8, tile (i/8) % kXcdChunk of the run.  The
// grid is padded to a multiple of 8*kXcdChunk; blocks past the last tile
// exit at once.  Only the placement changes: a row's arithmetic never
// depends on its block.
constexpr int kXcds = 8;
constexpr int kXcdChunk = 8;

__host__ __device__ inline long long xcd_padded_blocks(long long n) {
  const long long q = (long long)kXcds * kXcdChunk;
  return (n + q - 1) / q * q;
}

//
// Groups of fewer than kXcdChunk tiles (a one-token decode step has one or
// two) share runs instead: a run holds kXcdChunk / s consecutive groups of s
// tile slots each (s the power of two at least `tiles`), so the KV heads of
// a sequence, whose rows interleave in the paged cache, run side by side on
// one XCD (spread over four XCDs, the batch-64 one-token decode took 4.66 ms
// against 3.20).
__host__ __device__ inline int run_slots(int tiles) {
  int s = 1;
  while (s < tiles && s < kXcdChunk) s <<= 1;
  return s;
}

__host__ __device__ inline long long run_major_blocks(int tiles, long long groups) {
  long long runs;
  if (tiles >= kXcdChunk) {
    runs = (long long)((tiles + kXcdChunk - 1) / kXcdChunk) * groups;
  } else {
    const long long per = kXcdChunk / run_slots(tiles);  // groups per run
    runs = (groups + per - 1) / per;
  }
  return xcd_padded_blocks(runs * kXcdChunk);
}

// Tile and group of block i; false for blocks past the last tile.
__device__ inline bool run_major_item(long long i, int tiles, long long groups, int& tile,
                                      long long& group) {
  const long long x = i % kXcds, j = i / kXcds, c = j / kXcdChunk;
  const long long run = c * kXcds + (x + c) % kXcds;
  const int k8 = (int)(j % kXcdChunk);
  if (tiles >= kXcdChunk) {
    group = run % groups;
    tile = (int)((run / groups) * kXcdChunk + k8);
    return tile < tiles;
  }
  const int s = run_slots(tiles);
  group = run * (kXcdChunk / s) + k8 / s;
  tile = k8 % s;
  return tile < tiles && group < groups;
}

bool prefill_schedule(int d, int group, PrefillSchedule* s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Head dims 256 and 512 (prefill_ws.hip): score waves and PV waves, two per
// SIMD; prefill_schedule / launch_prefill dispatch to these.
bool prefill_ws_schedule(int d, int group, PrefillSchedule* s);
hipError_t launch_prefill_ws(const PrefillArgs& a, hipStream_t stream);

// Attention backward (backward.hip): dq and delta (one kernel), then dk and
// dv (a second kernel reading delta), on the caller's stream.
// The attention prologue (prologue.hip): RMSNorm then RoPE of every Q and K
// head vector, in place.  k == nullptr means hkv == 0 here.
struct PrologueArgs {
  void* q;
  void* k;
  const int32_t* positions;
  int tokens, hq, hkv, d;
  const float* q_weight;
  const float* k_weight;
  float eps, offset;
  int rotary_dims, freq_dims;
  double theta;
};

hipError_t launch_qk_prologue(const PrologueArgs& a, hipStream_t stream, const char** kernel);

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
// *kernel: the instances launched (a static string).
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream, const char** kernel);

constexpr int kDecodeChunk = 512;  // keys per split chunk (fixed; ATTN_DECODE_CHUNK)
constexpr int kDecodeStage = 16;   // keys per pipeline stage inside a chunk (one cache block)
constexpr int decode_record_floats(int d) { return d + 4; }  // acc[d], m, l, pad

// *kernel: the instances launched (a static string).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, const char** kernel);

}  // namespace invattn
