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
};

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

bool prefill_schedule(int d, int group, PrefillSchedule* s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

constexpr int kDecodeChunk = 512;  // keys per split chunk (fixed; ATTN_DECODE_CHUNK)
constexpr int kDecodeStage = 16;   // keys per pipeline stage inside a chunk (one cache block)
constexpr int decode_record_floats(int d) { return d + 4; }  // acc[d], m, l, pad

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace invattn
