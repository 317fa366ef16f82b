// api.hip -- the C ABI: argument checks (fail closed), schedule choice,
// launch on the caller's stream, thread-local error text and provenance.
//
// Fail-closed rule and provenance fields: "RFC: Gemma-4-31B-it train/rollout
// consistency", section 4, items 7 and 8.  Input checks before any launch and
// an early return for empty work follow the binding conventions described in
// "Gated RMSNorm CUDA kernel for the GDN block" (Summary: dtype, device and
// shape checks, empty input returns at once, launch errors checked).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "invattn.h"
#include "kernels.h"

using namespace invattn;

// ---------------------------------------------------------------------------
// Scratch of attn_decode_paged_noalloc: the chunk records of one decode call,
// in a static device array that every GPU the library runs on holds until the
// process ends (ATTN_NOALLOC_SCRATCH_BYTES).  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only
// that address is used.  Nothing in it needs to start at zero: the chunk
// kernel writes every record the merge kernel reads.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;
thread_local std::string g_prov;
thread_local bool g_have_prov = false;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool validate_enabled() {
  const char* e = getenv("INVATTN_VALIDATE");
  return e != nullptr && e[0] == '1';
}

// fl32(scale * log2(e)), computed in double and rounded once.
float fold_scale(float scale) {
  return (float)((double)scale * 1.4426950408889634073599246810019);
}

const char* layer_type(int window) { return window < 0 ? "global" : "sliding"; }

std::string device_name(int dev) {
  static thread_local int cached_dev = -1;
  static thread_local std::string cached;
  if (dev != cached_dev) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) cached = p.gcnArchName;
    else cached = "unknown";
    cached_dev = dev;
  }
  return cached;
}

bool trace_enabled() {
  const char* e = getenv("INVATTN_TRACE");
  return e != nullptr && e[0] == '1';
}

// The record of a successful call; with INVATTN_TRACE=1 it is also printed
// to stderr, one line per call.  `tokens` < 0: not known on the host (the
// packed token count lives in device memory unless INVATTN_VALIDATE=1 copied
// it).
void set_provenance(const char* op, const char* kernel, const std::string& schedule,
                    const char* split, int window, int d, int hq, int hkv, int batch,
                    int max_len, long long tokens) {
  int dev = -1;
  (void)hipGetDevice(&dev);
  char tok[32];
  if (tokens >= 0) snprintf(tok, sizeof tok, "%lld", tokens);
  else snprintf(tok, sizeof tok, "null");
  char buf[1280];
  snprintf(buf, sizeof buf,
           "{\"op\":\"%s\",\"requested_backend\":\"invattn-hip\",\"actual_backend\":"
           "\"invattn-hip\",\"kernel_id\":\"%s\",\"schedule_id\":\"%s\",\"split_policy\":\"%s\","
           "\"accumulator_dtype\":\"fp32\",\"layer_type\":\"%s\",\"device\":%d,\"arch\":\"%s\","
           "\"dtype\":\"bf16\",\"shape\":{\"batch\":%d,\"max_len\":%d,\"tokens\":%s,"
           "\"num_q_heads\":%d,\"num_kv_heads\":%d,\"head_dim\":%d,\"window\":%d},"
           "\"casts\":[\"p->bf16 rne\",\"o->bf16 rne\"],\"exp\":\"v_exp_f32\",\"fallback\":\"none\","
           "\"version\":\"%s\"}",
           op, kernel, schedule.c_str(), split, layer_type(window), dev,
           device_name(dev < 0 ? 0 : dev).c_str(), batch, max_len, tok, hq, hkv, d, window,
           attn_version());
  g_prov = buf;
  g_have_prov = true;
  if (trace_enabled()) fprintf(stderr, "invattn: %s\n", buf);
}

int check_heads(int32_t hq, int32_t hkv, int32_t d, int32_t window, float scale) {
  if (hq <= 0 || hkv <= 0 || d <= 0)
    return fail(ATTN_E_SHAPE, "num_q_heads=%d num_kv_heads=%d head_dim=%d must be positive", hq,
                hkv, d);
  if (hq % hkv != 0)
    return fail(ATTN_E_SHAPE, "num_q_heads=%d is not a multiple of num_kv_heads=%d", hq, hkv);
  const int group = hq / hkv;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(ATTN_E_UNSUPPORTED, "group size num_q_heads/num_kv_heads=%d not in {1,2,4,8}",
                group);
  if (d != 64 && d != 256 && d != 512)
    return fail(ATTN_E_UNSUPPORTED, "head_dim=%d not in {64,256,512}", d);
  if (window == 0 || window < -1)
    return fail(ATTN_E_UNSUPPORTED, "window=%d: use ATTN_WINDOW_NONE (-1) or a value >= 1",
                window);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_E_UNSUPPORTED, "softmax_scale=%g must be finite and > 0", (double)scale);
  return ATTN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Copy `n` int32 from device to host on the stream and wait.
int fetch_ints(const int32_t* dev, size_t n, std::vector<int32_t>& out, hipStream_t s,
               const char* what) {
  out.resize(n);
  if (n == 0) return ATTN_OK;
  hipError_t e = hipMemcpyAsync(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, what);
  return ATTN_OK;
}

// INVATTN_VALIDATE content checks of a packed varlen batch: cu_seqlens
// starts at 0, never decreases and no sequence exceeds max_seqlen; spans are
// non-empty, ascending, disjoint and each inside one sequence.  *tokens gets
// cu_seqlens[batch].
int validate_varlen(const int32_t* cu_seqlens, int batch, int max_seqlen, const int32_t* spans,
                    int num_spans, hipStream_t s, long long* tokens) {
  std::vector<int32_t> cu, sp;
  int rc;
  if ((rc = fetch_ints(cu_seqlens, (size_t)batch + 1, cu, s, "copy cu_seqlens")) != ATTN_OK) return rc;
  if (cu[0] != 0) return fail(ATTN_E_VALIDATE, "cu_seqlens[0]=%d must be 0", cu[0]);
  for (int b = 0; b < batch; ++b) {
    const int len = cu[b + 1] - cu[b];
    if (len < 0) return fail(ATTN_E_VALIDATE, "cu_seqlens decreases at %d", b);
    if (len > max_seqlen)
      return fail(ATTN_E_VALIDATE, "sequence %d has length %d > max_seqlen=%d", b, len, max_seqlen);
  }
  *tokens = cu[batch];
  if ((rc = fetch_ints(spans, (size_t)num_spans * 2, sp, s, "copy spans")) != ATTN_OK) return rc;
  int seq = 0;
  for (int i = 0; i < num_spans; ++i) {
    const int a = sp[2 * i], e = sp[2 * i + 1];
    if (a >= e) return fail(ATTN_E_VALIDATE, "span %d is empty or reversed [%d,%d)", i, a, e);
    if (i > 0 && a < sp[2 * i - 1])
      return fail(ATTN_E_VALIDATE, "span %d overlaps or is out of order", i);
    while (seq < batch && cu[seq + 1] <= a) ++seq;
    if (seq >= batch || a < cu[seq] || e > cu[seq + 1])
      return fail(ATTN_E_VALIDATE, "span %d [%d,%d) is not inside one sequence", i, a, e);
  }
  return ATTN_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_E_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(ATTN_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return ATTN_OK;
}

// The decode entry points.  own_scratch: the chunk records go to the
// library's static scratch array (workspace is ignored, workspace_bytes is
// the array's size); otherwise to the caller's workspace.
int decode_impl(const char* op, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                int32_t batch, int32_t max_seq_len, int32_t num_blocks, int32_t block_size,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t window,
                float softmax_scale, void* workspace, size_t workspace_bytes, bool own_scratch,
                void* o, hipStream_t stream) {
  g_err.clear();
  if (batch < 0) return fail(ATTN_E_SHAPE, "batch=%d must be >= 0", batch);
  int rc = check_heads(num_q_heads, num_kv_heads, head_dim, window, softmax_scale);
  if (rc != ATTN_OK) return rc;
  if (block_size != 16) return fail(ATTN_E_UNSUPPORTED, "block_size=%d must be 16", block_size);
  if (batch > 65535) return fail(ATTN_E_UNSUPPORTED, "batch=%d exceeds 65535", batch);
  const int group = num_q_heads / num_kv_heads;
  char sid[128];
  snprintf(sid, sizeof sid, "decode_d%d_g%d_chunk%d_block%d_t256+merge_t%d", head_dim, group,
           kDecodeChunk, kDecodeStage, head_dim >= 256 ? 256 : head_dim);
  char split[128];
  snprintf(split, sizeof split, "fixed chunks of %d keys from position 0; ascending merge",
           kDecodeChunk);
  if (batch == 0) {
    set_provenance(op, "none (empty input)", sid, split, window, head_dim,
                   num_q_heads, num_kv_heads, batch, max_seq_len, 0);
    return ATTN_OK;
  }
  if (max_seq_len <= 0) return fail(ATTN_E_SHAPE, "max_seq_len=%d must be >= 1", max_seq_len);
  if (max_blocks_per_seq <= 0) return fail(ATTN_E_SHAPE, "max_blocks_per_seq=%d must be >= 1", max_blocks_per_seq);
  if (num_blocks <= 0) return fail(ATTN_E_SHAPE, "num_blocks=%d must be >= 1", num_blocks);
  if ((long long)max_blocks_per_seq * block_size < max_seq_len)
    return fail(ATTN_E_SHAPE, "max_blocks_per_seq*block_size=%lld < max_seq_len=%d",
                (long long)max_blocks_per_seq * block_size, max_seq_len);
  if (!q) return fail(ATTN_E_NULL, "q is NULL");
  if (!k_cache) return fail(ATTN_E_NULL, "k_cache is NULL");
  if (!v_cache) return fail(ATTN_E_NULL, "v_cache is NULL");
  if (!block_table) return fail(ATTN_E_NULL, "block_table is NULL");
  if (!seq_lens) return fail(ATTN_E_NULL, "seq_lens is NULL");
  if (!own_scratch && !workspace) return fail(ATTN_E_NULL, "workspace is NULL");
  if (!o) return fail(ATTN_E_NULL, "o is NULL");
  if (!aligned16(q)) return fail(ATTN_E_ALIGN, "q is not 16-byte aligned");
  if (!aligned16(k_cache)) return fail(ATTN_E_ALIGN, "k_cache is not 16-byte aligned");
  if (!aligned16(v_cache)) return fail(ATTN_E_ALIGN, "v_cache is not 16-byte aligned");
  if (!own_scratch && !aligned16(workspace))
    return fail(ATTN_E_ALIGN, "workspace is not 16-byte aligned");
  if (!aligned16(o)) return fail(ATTN_E_ALIGN, "o is not 16-byte aligned");
  if (!aligned4(block_table)) return fail(ATTN_E_ALIGN, "block_table is not 4-byte aligned");
  if (!aligned4(seq_lens)) return fail(ATTN_E_ALIGN, "seq_lens is not 4-byte aligned");
  const size_t need = ::attn_decode_workspace_size(batch, max_seq_len, num_q_heads, head_dim);
  if (workspace_bytes < need) {
    if (own_scratch)
      return fail(ATTN_E_WORKSPACE, "the batch needs %zu bytes of chunk records, more than the "
                  "library's scratch of %zu bytes (use attn_decode_paged with a workspace)", need,
                  workspace_bytes);
    return fail(ATTN_E_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, need);
  }
  hipStream_t s = stream;
  if (own_scratch && (rc = scratch_address(&workspace)) != ATTN_OK) return rc;

  long long tokens = -1;
  if (validate_enabled()) {
    std::vector<int32_t> sl, bt;
    if ((rc = fetch_ints(seq_lens, (size_t)batch, sl, s, "copy seq_lens")) != ATTN_OK) return rc;
    if ((rc = fetch_ints(block_table, (size_t)batch * max_blocks_per_seq, bt, s, "copy block_table")) != ATTN_OK)
      return rc;
    tokens = 0;
    for (int b = 0; b < batch; ++b) {
      const int L = sl[b];
      if (L < 1 || L > max_seq_len)
        return fail(ATTN_E_VALIDATE, "seq_lens[%d]=%d outside [1, max_seq_len=%d]", b, L, max_seq_len);
      tokens += L;
      const int lo = window > 0 ? (L - window > 0 ? L - window : 0) : 0;
      for (int j = lo / block_size; j <= (L - 1) / block_size; ++j) {
        const int id = bt[(size_t)b * max_blocks_per_seq + j];
        if (id < 0 || id >= num_blocks)
          return fail(ATTN_E_VALIDATE, "block_table[%d][%d]=%d outside [0, num_blocks=%d)", b, j,
                      id, num_blocks);
      }
    }
  }

  DecodeArgs a{q, k_cache, v_cache, block_table, max_blocks_per_seq, seq_lens, batch,
               max_seq_len, num_blocks, num_q_heads, num_kv_heads, head_dim, window,
               fold_scale(softmax_scale), reinterpret_cast<float*>(workspace),
               (max_seq_len + kDecodeChunk - 1) / kDecodeChunk, o};
  const char* kernel = "";
  hipError_t e = launch_decode(a, s, &kernel);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  set_provenance(op, kernel, sid, split, window, head_dim, num_q_heads,
                 num_kv_heads, batch, max_seq_len, tokens);
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_version(void) { return "invattn 0.1.0 (gfx950)"; }

const char* attn_last_error(void) { return g_err.c_str(); }

int attn_last_provenance(char* buf, size_t n) {
  if (!g_have_prov) return -1;
  if (buf != nullptr && n > 0) {
    size_t c = g_prov.size() < n - 1 ? g_prov.size() : n - 1;
    memcpy(buf, g_prov.data(), c);
    buf[c] = '\0';
  }
  return (int)g_prov.size();
}

int attn_prefill_varlen(const void* q, const void* k, const void* v, void* o, float* lse_opt,
                        const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t window, float softmax_scale, const int32_t* spans_opt,
                        int32_t num_spans, hipStream_t stream) {
  g_err.clear();
  if (batch < 0) return fail(ATTN_E_SHAPE, "batch=%d must be >= 0", batch);
  if (max_seqlen < 0) return fail(ATTN_E_SHAPE, "max_seqlen=%d must be >= 0", max_seqlen);
  if (num_spans < 0) return fail(ATTN_E_SHAPE, "num_spans=%d must be >= 0", num_spans);
  int rc = check_heads(num_q_heads, num_kv_heads, head_dim, window, softmax_scale);
  if (rc != ATTN_OK) return rc;
  if (batch > 65535) return fail(ATTN_E_UNSUPPORTED, "batch=%d exceeds 65535", batch);
  const int group = num_q_heads / num_kv_heads;
  PrefillSchedule sched;
  if (!prefill_schedule(head_dim, group, &sched))
    return fail(ATTN_E_UNSUPPORTED, "no kernel for head_dim=%d group=%d", head_dim, group);
  char sid[128];
  snprintf(sid, sizeof sid, "prefill_d%d_g%d_rows%d_pos%d_bn%d_t%d", head_dim, group, sched.rows,
           sched.positions, sched.bn, sched.threads);
  if (batch == 0 || max_seqlen == 0) {
    set_provenance("attn_prefill_varlen", "none (empty input)", sid, "none", window, head_dim,
                   num_q_heads, num_kv_heads, batch, max_seqlen, 0);
    return ATTN_OK;
  }
  if (!q) return fail(ATTN_E_NULL, "q is NULL");
  if (!k) return fail(ATTN_E_NULL, "k is NULL");
  if (!v) return fail(ATTN_E_NULL, "v is NULL");
  if (!o) return fail(ATTN_E_NULL, "o is NULL");
  if (!cu_seqlens) return fail(ATTN_E_NULL, "cu_seqlens is NULL");
  if (num_spans > 0 && !spans_opt) return fail(ATTN_E_NULL, "spans_opt is NULL with num_spans=%d", num_spans);
  if (!aligned16(q)) return fail(ATTN_E_ALIGN, "q is not 16-byte aligned");
  if (!aligned16(k)) return fail(ATTN_E_ALIGN, "k is not 16-byte aligned");
  if (!aligned16(v)) return fail(ATTN_E_ALIGN, "v is not 16-byte aligned");
  if (!aligned16(o)) return fail(ATTN_E_ALIGN, "o is not 16-byte aligned");
  if (lse_opt && !aligned4(lse_opt)) return fail(ATTN_E_ALIGN, "lse_opt is not 4-byte aligned");
  if (!aligned4(cu_seqlens)) return fail(ATTN_E_ALIGN, "cu_seqlens is not 4-byte aligned");
  if (spans_opt && !aligned4(spans_opt)) return fail(ATTN_E_ALIGN, "spans_opt is not 4-byte aligned");
  const long long tiles = ((long long)max_seqlen + sched.positions - 1) / sched.positions;
  if (tiles > 0x7fffffffLL) return fail(ATTN_E_UNSUPPORTED, "max_seqlen=%d too large", max_seqlen);
  // One sequence's rows of one KV head are addressed with 32-bit byte offsets.
  if ((long long)max_seqlen * num_kv_heads * head_dim * 2 > 0x7fffffffLL)
    return fail(ATTN_E_UNSUPPORTED, "max_seqlen=%d x num_kv_heads=%d x head_dim=%d spans 2 GiB or more",
                max_seqlen, num_kv_heads, head_dim);
  hipStream_t s = stream;

  long long tokens = -1;
  if (validate_enabled() &&
      (rc = validate_varlen(cu_seqlens, batch, max_seqlen, spans_opt, num_spans, s, &tokens)) !=
          ATTN_OK)
    return rc;

  PrefillArgs a{q, k, v, o, lse_opt, cu_seqlens, spans_opt, num_spans, batch, max_seqlen,
                num_q_heads, num_kv_heads, head_dim, window, fold_scale(softmax_scale)};
  hipError_t e = launch_prefill(a, s);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  set_provenance("attn_prefill_varlen", sched.kernel, sid, "none (one ascending KV walk per row)",
                 window, head_dim, num_q_heads, num_kv_heads, batch, max_seqlen, tokens);
  return ATTN_OK;
}

int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache, void* o,
                       float* lse_opt, const int32_t* cu_seqlens, const int32_t* q_start,
                       const int32_t* block_table, int32_t max_blocks_per_seq, int32_t batch,
                       int32_t max_query_len, int32_t max_context_len, int32_t num_blocks,
                       int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t window, float softmax_scale, hipStream_t stream) {
  g_err.clear();
  if (batch < 0) return fail(ATTN_E_SHAPE, "batch=%d must be >= 0", batch);
  if (max_query_len < 0) return fail(ATTN_E_SHAPE, "max_query_len=%d must be >= 0", max_query_len);
  int rc = check_heads(num_q_heads, num_kv_heads, head_dim, window, softmax_scale);
  if (rc != ATTN_OK) return rc;
  if (block_size != 16) return fail(ATTN_E_UNSUPPORTED, "block_size=%d must be 16", block_size);
  if (batch > 65535) return fail(ATTN_E_UNSUPPORTED, "batch=%d exceeds 65535", batch);
  const int group = num_q_heads / num_kv_heads;
  PrefillSchedule sched;
  if (!prefill_schedule(head_dim, group, &sched))
    return fail(ATTN_E_UNSUPPORTED, "no kernel for head_dim=%d group=%d", head_dim, group);
  char sid[160];
  snprintf(sid, sizeof sid, "prefill_d%d_g%d_rows%d_pos%d_bn%d_t%d_paged16", head_dim, group,
           sched.rows, sched.positions, sched.bn, sched.threads);
  if (batch == 0 || max_query_len == 0) {
    set_provenance("attn_prefill_paged", "none (empty input)", sid, "none", window, head_dim,
                   num_q_heads, num_kv_heads, batch, max_query_len, 0);
    return ATTN_OK;
  }
  if (max_context_len < max_query_len)
    return fail(ATTN_E_SHAPE, "max_context_len=%d < max_query_len=%d", max_context_len,
                max_query_len);
  if (max_blocks_per_seq <= 0)
    return fail(ATTN_E_SHAPE, "max_blocks_per_seq=%d must be >= 1", max_blocks_per_seq);
  if (num_blocks <= 0) return fail(ATTN_E_SHAPE, "num_blocks=%d must be >= 1", num_blocks);
  if ((long long)max_blocks_per_seq * block_size < max_context_len)
    return fail(ATTN_E_SHAPE, "max_blocks_per_seq*block_size=%lld < max_context_len=%d",
                (long long)max_blocks_per_seq * block_size, max_context_len);
  if (!q) return fail(ATTN_E_NULL, "q is NULL");
  if (!k_cache) return fail(ATTN_E_NULL, "k_cache is NULL");
  if (!v_cache) return fail(ATTN_E_NULL, "v_cache is NULL");
  if (!o) return fail(ATTN_E_NULL, "o is NULL");
  if (!cu_seqlens) return fail(ATTN_E_NULL, "cu_seqlens is NULL");
  if (!q_start) return fail(ATTN_E_NULL, "q_start is NULL");
  if (!block_table) return fail(ATTN_E_NULL, "block_table is NULL");
  if (!aligned16(q)) return fail(ATTN_E_ALIGN, "q is not 16-byte aligned");
  if (!aligned16(k_cache)) return fail(ATTN_E_ALIGN, "k_cache is not 16-byte aligned");
  if (!aligned16(v_cache)) return fail(ATTN_E_ALIGN, "v_cache is not 16-byte aligned");
  if (!aligned16(o)) return fail(ATTN_E_ALIGN, "o is not 16-byte aligned");
  if (lse_opt && !aligned4(lse_opt)) return fail(ATTN_E_ALIGN, "lse_opt is not 4-byte aligned");
  if (!aligned4(cu_seqlens)) return fail(ATTN_E_ALIGN, "cu_seqlens is not 4-byte aligned");
  if (!aligned4(q_start)) return fail(ATTN_E_ALIGN, "q_start is not 4-byte aligned");
  if (!aligned4(block_table)) return fail(ATTN_E_ALIGN, "block_table is not 4-byte aligned");
  // The grid covers one more position tile than the query rows need (a chunk
  // starts anywhere inside a tile).
  const long long tiles = ((long long)max_query_len + sched.positions - 1) / sched.positions + 1;
  if (tiles * num_kv_heads * batch > 0x7fffffffLL)
    return fail(ATTN_E_UNSUPPORTED, "max_query_len=%d too large", max_query_len);
  hipStream_t s = stream;

  long long tokens = -1;
  if (validate_enabled()) {
    std::vector<int32_t> cu, qs, bt;
    if ((rc = fetch_ints(cu_seqlens, (size_t)batch + 1, cu, s, "copy cu_seqlens")) != ATTN_OK) return rc;
    if ((rc = fetch_ints(q_start, (size_t)batch, qs, s, "copy q_start")) != ATTN_OK) return rc;
    if ((rc = fetch_ints(block_table, (size_t)batch * max_blocks_per_seq, bt, s, "copy block_table")) != ATTN_OK)
      return rc;
    if (cu[0] != 0) return fail(ATTN_E_VALIDATE, "cu_seqlens[0]=%d must be 0", cu[0]);
    for (int b = 0; b < batch; ++b) {
      const int n = cu[b + 1] - cu[b];
      if (n < 0) return fail(ATTN_E_VALIDATE, "cu_seqlens decreases at %d", b);
      if (n > max_query_len)
        return fail(ATTN_E_VALIDATE, "sequence %d has %d new tokens > max_query_len=%d", b, n,
                    max_query_len);
      if (qs[b] < 0 || (long long)qs[b] + n > max_context_len)
        return fail(ATTN_E_VALIDATE, "q_start[%d]=%d with %d new tokens outside [0, max_context_len=%d]",
                    b, qs[b], n, max_context_len);
      if (n == 0) continue;
      const int L = qs[b] + n;
      const int lo = window > 0 ? (qs[b] - window + 1 > 0 ? qs[b] - window + 1 : 0) : 0;
      for (int j = lo / block_size; j <= (L - 1) / block_size; ++j) {
        const int id = bt[(size_t)b * max_blocks_per_seq + j];
        if (id < 0 || id >= num_blocks)
          return fail(ATTN_E_VALIDATE, "block_table[%d][%d]=%d outside [0, num_blocks=%d)", b, j,
                      id, num_blocks);
      }
    }
    tokens = cu[batch];
  }

  PrefillArgs a{q, k_cache, v_cache, o, lse_opt, cu_seqlens, nullptr, 0, batch, max_query_len,
                num_q_heads, num_kv_heads, head_dim, window, fold_scale(softmax_scale)};
  a.q_start = q_start;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context = max_context_len;
  hipError_t e = launch_prefill(a, s);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  const std::string kid = std::string("PagedOf ") + sched.kernel;
  set_provenance("attn_prefill_paged", kid.c_str(), sid, "none (one ascending KV walk per row)",
                 window, head_dim, num_q_heads, num_kv_heads, batch, max_query_len, tokens);
  return ATTN_OK;
}

int attn_prefill_varlen_backward(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, float* dq, float* dk,
                                 float* dv, float* workspace, int32_t total_tokens,
                                 const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t window, float softmax_scale, const int32_t* spans_opt,
                                 int32_t num_spans, hipStream_t stream) {
  g_err.clear();
  if (batch < 0) return fail(ATTN_E_SHAPE, "batch=%d must be >= 0", batch);
  if (max_seqlen < 0) return fail(ATTN_E_SHAPE, "max_seqlen=%d must be >= 0", max_seqlen);
  if (total_tokens < 0) return fail(ATTN_E_SHAPE, "total_tokens=%d must be >= 0", total_tokens);
  if (num_spans < 0) return fail(ATTN_E_SHAPE, "num_spans=%d must be >= 0", num_spans);
  int rc = check_heads(num_q_heads, num_kv_heads, head_dim, window, softmax_scale);
  if (rc != ATTN_OK) return rc;
  if (batch > 65535) return fail(ATTN_E_UNSUPPORTED, "batch=%d exceeds 65535", batch);
  const int rows = backward_rows_per_tile(head_dim);
  char sid[96];
  snprintf(sid, sizeof sid, "backward_d%d_rows%d_t256_fp32fma", head_dim, rows);
  if (batch == 0 || max_seqlen == 0) {
    set_provenance("attn_prefill_varlen_backward", "none (empty input)", sid, "none", window,
                   head_dim, num_q_heads, num_kv_heads, batch, max_seqlen, 0);
    return ATTN_OK;
  }
  if (!q) return fail(ATTN_E_NULL, "q is NULL");
  if (!k) return fail(ATTN_E_NULL, "k is NULL");
  if (!v) return fail(ATTN_E_NULL, "v is NULL");
  if (!o) return fail(ATTN_E_NULL, "o is NULL");
  if (!lse) return fail(ATTN_E_NULL, "lse is NULL");
  if (!dout) return fail(ATTN_E_NULL, "dout is NULL");
  if (!dq) return fail(ATTN_E_NULL, "dq is NULL");
  if (!dk) return fail(ATTN_E_NULL, "dk is NULL");
  if (!dv) return fail(ATTN_E_NULL, "dv is NULL");
  if (!workspace) return fail(ATTN_E_NULL, "workspace is NULL");
  if (!cu_seqlens) return fail(ATTN_E_NULL, "cu_seqlens is NULL");
  if (num_spans > 0 && !spans_opt) return fail(ATTN_E_NULL, "spans_opt is NULL with num_spans=%d", num_spans);
  const void* a16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
  const char* n16[] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv", "workspace"};
  for (int i = 0; i < 9; ++i)
    if (!aligned16(a16[i])) return fail(ATTN_E_ALIGN, "%s is not 16-byte aligned", n16[i]);
  if (!aligned4(lse)) return fail(ATTN_E_ALIGN, "lse is not 4-byte aligned");
  if (!aligned4(cu_seqlens)) return fail(ATTN_E_ALIGN, "cu_seqlens is not 4-byte aligned");
  if (spans_opt && !aligned4(spans_opt)) return fail(ATTN_E_ALIGN, "spans_opt is not 4-byte aligned");
  const long long tiles = ((long long)max_seqlen + rows - 1) / rows;
  if (tiles * num_q_heads * batch > 0x7fffffffLL)
    return fail(ATTN_E_UNSUPPORTED, "max_seqlen=%d x num_q_heads=%d x batch=%d needs more than 2^31 "
                "workgroups", max_seqlen, num_q_heads, batch);
  hipStream_t s = stream;

  long long tokens = -1;
  if (validate_enabled()) {
    if ((rc = validate_varlen(cu_seqlens, batch, max_seqlen, spans_opt, num_spans, s, &tokens)) !=
        ATTN_OK)
      return rc;
    if (tokens > total_tokens)
      return fail(ATTN_E_VALIDATE, "cu_seqlens[batch]=%lld > total_tokens=%d", tokens, total_tokens);
  }

  BackwardArgs a{q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, spans_opt, num_spans,
                 batch, max_seqlen, num_q_heads, num_kv_heads, head_dim, window, softmax_scale,
                 fold_scale(softmax_scale)};
  const char* kernel = "";
  hipError_t e = launch_backward(a, s, &kernel);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  set_provenance("attn_prefill_varlen_backward", kernel, sid,
                 "none (one ascending walk per row and per key)", window, head_dim, num_q_heads,
                 num_kv_heads, batch, max_seqlen, tokens);
  return ATTN_OK;
}

int attn_qk_prologue(void* q, void* k, const int32_t* positions, int32_t num_tokens,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     const float* q_weight, const float* k_weight, float eps,
                     float weight_offset, int32_t rotary_dims, int32_t freq_dims,
                     double rope_theta, hipStream_t stream) {
  g_err.clear();
  if (num_tokens < 0) return fail(ATTN_E_SHAPE, "num_tokens=%d must be >= 0", num_tokens);
  if (num_q_heads <= 0) return fail(ATTN_E_SHAPE, "num_q_heads=%d must be positive", num_q_heads);
  if (k != nullptr && num_kv_heads <= 0)
    return fail(ATTN_E_SHAPE, "num_kv_heads=%d must be positive when k is given", num_kv_heads);
  if (head_dim != 64 && head_dim != 256 && head_dim != 512)
    return fail(ATTN_E_UNSUPPORTED, "head_dim=%d not in {64,256,512}", head_dim);
  const int per_lane = head_dim / 64;
  if (rotary_dims < 0 || rotary_dims > head_dim || rotary_dims % (2 * per_lane) != 0)
    return fail(ATTN_E_UNSUPPORTED, "rotary_dims=%d must lie in [0, %d] and be a multiple of %d",
                rotary_dims, head_dim, 2 * per_lane);
  if (rotary_dims > 0 && freq_dims <= 0)
    return fail(ATTN_E_UNSUPPORTED, "freq_dims=%d must be positive", freq_dims);
  if (rotary_dims > 0 && (!std::isfinite(rope_theta) || !(rope_theta > 0.0)))
    return fail(ATTN_E_UNSUPPORTED, "rope_theta=%g must be finite and > 0", rope_theta);
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(ATTN_E_UNSUPPORTED, "eps=%g must be finite and >= 0", (double)eps);
  if (!std::isfinite(weight_offset))
    return fail(ATTN_E_UNSUPPORTED, "weight_offset=%g must be finite", (double)weight_offset);
  const int hkv = k != nullptr ? num_kv_heads : 0;
  if ((long long)num_q_heads + hkv > 65536)
    return fail(ATTN_E_UNSUPPORTED, "num_q_heads + num_kv_heads = %d exceeds 65536",
                num_q_heads + hkv);
  char sid[128];
  snprintf(sid, sizeof sid, "prologue_d%d_rmsnorm%s%s_rope%d_f%d_t256", head_dim,
           q_weight ? "_q" : "", (k && k_weight) ? "_k" : "", rotary_dims, freq_dims);
  const char* kernel = "none (empty input)";
  if (num_tokens > 0) {
    if (!q) return fail(ATTN_E_NULL, "q is NULL");
    if (!positions) return fail(ATTN_E_NULL, "positions is NULL");
    if (!aligned16(q)) return fail(ATTN_E_ALIGN, "q is not 16-byte aligned");
    if (k && !aligned16(k)) return fail(ATTN_E_ALIGN, "k is not 16-byte aligned");
    if (!aligned4(positions)) return fail(ATTN_E_ALIGN, "positions is not 4-byte aligned");
    if (q_weight && !aligned4(q_weight)) return fail(ATTN_E_ALIGN, "q_weight is not 4-byte aligned");
    if (k_weight && !aligned4(k_weight)) return fail(ATTN_E_ALIGN, "k_weight is not 4-byte aligned");
    PrologueArgs a{q, k, positions, num_tokens, num_q_heads, hkv, head_dim, q_weight,
                   k ? k_weight : nullptr, eps, weight_offset, rotary_dims, freq_dims, rope_theta};
    hipError_t e = launch_qk_prologue(a, stream, &kernel);
    if (e != hipSuccess) return hip_fail(e, "prologue launch");
  }
  int dev = -1;
  (void)hipGetDevice(&dev);
  char buf[768];
  snprintf(buf, sizeof buf,
           "{\"op\":\"attn_qk_prologue\",\"requested_backend\":\"invattn-hip\",\"actual_backend\":"
           "\"invattn-hip\",\"kernel_id\":\"%s\",\"schedule_id\":\"%s\",\"split_policy\":\"none\","
           "\"accumulator_dtype\":\"fp32\",\"layer_type\":\"%s\",\"device\":%d,\"arch\":\"%s\","
           "\"dtype\":\"bf16\",\"shape\":{\"tokens\":%d,\"num_q_heads\":%d,\"num_kv_heads\":%d,"
           "\"head_dim\":%d,\"rotary_dims\":%d,\"freq_dims\":%d},\"casts\":[\"out->bf16 rne\"],"
           "\"angles\":\"fp64, reduced by pi/2\",\"fallback\":\"none\",\"version\":\"%s\"}",
           kernel, sid, rotary_dims < head_dim ? "partial rope" : "full rope", dev,
           device_name(dev < 0 ? 0 : dev).c_str(), num_tokens, num_q_heads, hkv, head_dim,
           rotary_dims, freq_dims, attn_version());
  g_prov = buf;
  g_have_prov = true;
  if (trace_enabled()) fprintf(stderr, "invattn: %s\n", buf);
  return ATTN_OK;
}

size_t attn_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t num_q_heads,
                                  int32_t head_dim) {
  if (batch <= 0 || max_seq_len <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const size_t chunks = ((size_t)max_seq_len + kDecodeChunk - 1) / kDecodeChunk;
  return (size_t)batch * num_q_heads * chunks * decode_record_floats(head_dim) * sizeof(float);
}

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                      int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t window,
                      float softmax_scale, void* workspace, size_t workspace_bytes, void* o,
                      hipStream_t stream) {
  return decode_impl("attn_decode_paged", q, k_cache, v_cache, block_table, max_blocks_per_seq,
                     seq_lens, batch, max_seq_len, num_blocks, block_size, num_q_heads,
                     num_kv_heads, head_dim, window, softmax_scale, workspace, workspace_bytes,
                     false, o, stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                              int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t window,
                              float softmax_scale, void* o, hipStream_t stream) {
  return decode_impl("attn_decode_paged_noalloc", q, k_cache, v_cache, block_table,
                     max_blocks_per_seq, seq_lens, batch, max_seq_len, num_blocks, block_size,
                     num_q_heads, num_kv_heads, head_dim, window, softmax_scale, nullptr,
                     (size_t)ATTN_NOALLOC_SCRATCH_BYTES, true, o, stream);
}

}  // extern "C"
