// C ABI of libpaged_attn.so: argument validation, status codes and dispatch to
// the gfx950 launchers.  Every check below runs before the first HIP call, so
// a malformed call fails without touching the device.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <climits>
#include <mutex>
#include <string>

#include "../../include/paged_attn.h"
#include "launch.h"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int32_t dtype) { return dtype == PA_DTYPE_F32 || dtype == PA_DTYPE_BF16; }
int elem_size(int32_t dtype) { return dtype == PA_DTYPE_BF16 ? 2 : (dtype == PA_DTYPE_FP8_E4M3 ? 1 : 4); }

#define PA_REQUIRE(cond, status, ...) \
  do {                                \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

// Checks shared by decode and prefill.
int check_attn(const char* fn, int32_t num_seqs, int32_t hq, int32_t hkv, int32_t head_dim,
               int32_t block_size, int64_t num_blocks, int32_t max_blocks, int32_t dtype) {
  PA_REQUIRE(num_seqs >= 0, PA_ERR_INVALID, "%s: num_seqs must be >= 0 (got %d)", fn, num_seqs);
  PA_REQUIRE(hq >= 1 && hkv >= 1, PA_ERR_INVALID, "%s: head counts must be >= 1 (got %d, %d)", fn, hq, hkv);
  PA_REQUIRE(hq % hkv == 0, PA_ERR_INVALID,
             "%s: num_q_heads (%d) must be a multiple of num_kv_heads (%d)", fn, hq, hkv);
  PA_REQUIRE(dtype_ok(dtype), PA_ERR_UNSUPPORTED, "%s: unsupported dtype %d", fn, dtype);
  PA_REQUIRE(head_dim == 64 || head_dim == 128, PA_ERR_UNSUPPORTED,
             "%s: head_dim must be 64 or 128 (got %d)", fn, head_dim);
  PA_REQUIRE(block_size >= 1, PA_ERR_INVALID, "%s: block_size must be >= 1 (got %d)", fn, block_size);
  PA_REQUIRE(num_blocks >= 1 && num_blocks <= INT_MAX, PA_ERR_INVALID,
             "%s: num_blocks must be in [1, 2^31) (got %lld)", fn, (long long)num_blocks);
  PA_REQUIRE(max_blocks >= 1, PA_ERR_INVALID, "%s: max_blocks_per_seq must be >= 1 (got %d)", fn,
             max_blocks);
  PA_REQUIRE((int64_t)max_blocks * block_size <= INT_MAX, PA_ERR_INVALID,
             "%s: max_blocks_per_seq * block_size must fit in int32", fn);
  PA_REQUIRE(num_blocks * (int64_t)block_size <= INT_MAX, PA_ERR_INVALID,
             "%s: num_blocks * block_size must fit in int32 (slots are int32)", fn);
  return PA_OK;
}

}  // namespace

namespace pa {

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

}  // namespace pa

extern "C" {

int pa_version(void) { return 100; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_err.c_str(); }

int pa_set_timing_events(void* start_event, void* stop_event) {
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
  return PA_OK;
}

int pa_slot_mapping(const int32_t* block_table, const int32_t* cu_seqlens, const int32_t* context_lens,
                    int32_t* slot_mapping, int32_t num_seqs, int64_t num_tokens, int32_t block_size,
                    int32_t max_blocks_per_seq, void* stream) {
  g_err.clear();
  const char* fn = "pa_slot_mapping";
  PA_REQUIRE(num_seqs >= 0 && num_tokens >= 0, PA_ERR_INVALID, "%s: negative size", fn);
  PA_REQUIRE(num_tokens <= INT_MAX, PA_ERR_INVALID, "%s: num_tokens must fit in int32", fn);
  PA_REQUIRE(block_size >= 1 && max_blocks_per_seq >= 1, PA_ERR_INVALID,
             "%s: block_size and max_blocks_per_seq must be >= 1", fn);
  if (num_tokens == 0) return PA_OK;
  PA_REQUIRE(num_seqs >= 1, PA_ERR_INVALID, "%s: %lld tokens but no sequence", fn, (long long)num_tokens);
  PA_REQUIRE(block_table && cu_seqlens && context_lens && slot_mapping, PA_ERR_INVALID,
             "%s: null pointer argument", fn);
  return hip_status(pa::launch_slot_mapping(block_table, cu_seqlens, context_lens, slot_mapping, num_seqs,
                                            num_tokens, block_size, max_blocks_per_seq,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

int pa_reshape_and_cache(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache,
                         void* v_cache, int64_t num_tokens, int64_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void* stream) {
  g_err.clear();
  const char* fn = "pa_reshape_and_cache";
  PA_REQUIRE(num_tokens >= 0, PA_ERR_INVALID, "%s: num_tokens must be >= 0", fn);
  PA_REQUIRE(dtype_ok(dtype), PA_ERR_UNSUPPORTED, "%s: unsupported dtype %d", fn, dtype);
  PA_REQUIRE(num_kv_heads >= 1 && head_dim >= 1, PA_ERR_INVALID, "%s: head sizes must be >= 1", fn);
  PA_REQUIRE(block_size >= 1, PA_ERR_INVALID, "%s: block_size must be >= 1", fn);
  PA_REQUIRE(num_blocks >= 1, PA_ERR_INVALID, "%s: num_blocks must be >= 1", fn);
  PA_REQUIRE(num_blocks * (int64_t)block_size <= INT_MAX, PA_ERR_INVALID,
             "%s: num_blocks * block_size must fit in int32 (slots are int32)", fn);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elem_size(dtype);
  PA_REQUIRE(row_bytes % 16 == 0 && row_bytes <= INT_MAX, PA_ERR_UNSUPPORTED,
             "%s: a token row (H_kv * D * elem) must be a multiple of 16 bytes (got %lld)", fn,
             (long long)row_bytes);
  if (num_tokens == 0) return PA_OK;
  PA_REQUIRE(k && v && slot_mapping && k_cache && v_cache, PA_ERR_INVALID, "%s: null pointer argument", fn);
  return hip_status(pa::launch_reshape_and_cache(k, v, slot_mapping, k_cache, v_cache, num_tokens,
                                                 num_blocks * block_size, (int)row_bytes,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

int pa_reshape_and_cache_fp8(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache,
                             void* v_cache, const float* k_scale, const float* v_scale, int64_t num_tokens,
                             int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                             int32_t dtype, void* stream) {
  g_err.clear();
  const char* fn = "pa_reshape_and_cache_fp8";
  PA_REQUIRE(num_tokens >= 0, PA_ERR_INVALID, "%s: num_tokens must be >= 0", fn);
  PA_REQUIRE(dtype_ok(dtype), PA_ERR_UNSUPPORTED, "%s: unsupported source dtype %d", fn, dtype);
  PA_REQUIRE(num_kv_heads >= 1 && head_dim >= 1, PA_ERR_INVALID, "%s: head sizes must be >= 1", fn);
  PA_REQUIRE(head_dim % 16 == 0, PA_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 16 (got %d)", fn,
             head_dim);
  PA_REQUIRE(block_size >= 1, PA_ERR_INVALID, "%s: block_size must be >= 1", fn);
  PA_REQUIRE(num_blocks >= 1, PA_ERR_INVALID, "%s: num_blocks must be >= 1", fn);
  PA_REQUIRE(num_blocks * (int64_t)block_size <= INT_MAX, PA_ERR_INVALID,
             "%s: num_blocks * block_size must fit in int32 (slots are int32)", fn);
  const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
  PA_REQUIRE(row_elems <= INT_MAX / 4, PA_ERR_UNSUPPORTED, "%s: token row too large", fn);
  if (num_tokens == 0) return PA_OK;
  PA_REQUIRE(k && v && slot_mapping && k_cache && v_cache && k_scale && v_scale, PA_ERR_INVALID,
             "%s: null pointer argument", fn);
  return hip_status(pa::launch_reshape_and_cache_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                                                     num_tokens, num_blocks * block_size, (int)row_elems, head_dim,
                                                     dtype, static_cast<hipStream_t>(stream)),
                    fn);
}

int pa_check_metadata(const int32_t* block_table, const int32_t* context_lens, const int32_t* cu_seqlens,
                      const int32_t* slot_mapping, int32_t num_seqs, int64_t num_tokens, int64_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, int32_t* result, void* stream) {
  g_err.clear();
  const char* fn = "pa_check_metadata";
  PA_REQUIRE(num_seqs >= 0 && num_tokens >= 0 && num_tokens <= INT_MAX, PA_ERR_INVALID, "%s: negative sizes", fn);
  PA_REQUIRE(block_size >= 1 && max_blocks_per_seq >= 1 && num_blocks >= 1, PA_ERR_INVALID,
             "%s: block_size, max_blocks_per_seq and num_blocks must be >= 1", fn);
  PA_REQUIRE(result, PA_ERR_INVALID, "%s: null result pointer", fn);
  PA_REQUIRE(num_seqs == 0 || (block_table && context_lens), PA_ERR_INVALID, "%s: null pointer argument", fn);
  return hip_status(pa::launch_check_metadata(block_table, context_lens, cu_seqlens, slot_mapping, num_seqs,
                                              num_tokens, num_blocks, block_size, max_blocks_per_seq, result,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int64_t num_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   void* stream) {
  g_err.clear();
  const char* fn = "pa_copy_blocks";
  PA_REQUIRE(num_pairs >= 0 && num_pairs <= INT_MAX / 2, PA_ERR_INVALID, "%s: num_pairs must be in [0, 2^30)", fn);
  PA_REQUIRE(dtype_ok(dtype) || dtype == PA_DTYPE_FP8_E4M3, PA_ERR_UNSUPPORTED, "%s: unsupported dtype %d", fn,
             dtype);
  PA_REQUIRE(num_kv_heads >= 1 && head_dim >= 1, PA_ERR_INVALID, "%s: head sizes must be >= 1", fn);
  PA_REQUIRE(block_size >= 1, PA_ERR_INVALID, "%s: block_size must be >= 1", fn);
  PA_REQUIRE(num_blocks >= 1, PA_ERR_INVALID, "%s: num_blocks must be >= 1", fn);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elem_size(dtype);
  PA_REQUIRE(row_bytes % 16 == 0 && row_bytes <= INT_MAX, PA_ERR_UNSUPPORTED,
             "%s: a token row (H_kv * D * elem) must be a multiple of 16 bytes (got %lld)", fn,
             (long long)row_bytes);
  if (num_pairs == 0) return PA_OK;
  PA_REQUIRE(k_cache && v_cache && block_mapping, PA_ERR_INVALID, "%s: null pointer argument", fn);
  return hip_status(pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs, num_blocks,
                                           row_bytes * block_size, static_cast<hipStream_t>(stream)),
                    fn);
}

int pa_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int32_t num_workgroups, void* stream) {
  g_err.clear();
  const char* fn = "pa_hbm_read";
  PA_REQUIRE(bytes >= 0 && bytes % 16 == 0, PA_ERR_INVALID, "%s: bytes must be a non-negative multiple of 16 (got %lld)",
             fn, (long long)bytes);
  PA_REQUIRE(num_workgroups >= 1 && num_workgroups <= (1 << 20), PA_ERR_INVALID,
             "%s: num_workgroups must be in [1, 2^20] (got %d)", fn, num_workgroups);
  if (bytes == 0) return PA_OK;
  PA_REQUIRE(src && sink, PA_ERR_INVALID, "%s: null pointer argument", fn);
  PA_REQUIRE(reinterpret_cast<uintptr_t>(src) % 16 == 0, PA_ERR_INVALID, "%s: src must be 16-byte aligned", fn);
  return hip_status(pa::launch_hbm_read(src, bytes, sink, num_workgroups, static_cast<hipStream_t>(stream)), fn);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_q_heads < 1 || head_dim < 1 || block_size < 1 || max_blocks_per_seq < 1) return 0;
  return pa::decode_workspace_size(num_seqs, num_q_heads, head_dim, block_size, max_blocks_per_seq);
}

}  // extern "C"

namespace {

// k_new / v_new non-null: decode with append (new rows of type new_dtype).
int decode_call(const char* fn, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                const float* v_scale, const int32_t* block_table, const int32_t* context_lens, float scale, void* out,
                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype, int32_t kv_dtype, void* workspace,
                size_t workspace_bytes, void* stream, const void* k_new = nullptr, const void* v_new = nullptr,
                int32_t new_dtype = 0) {
  int st = check_attn(fn, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, dtype);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  PA_REQUIRE(q && k_cache && v_cache && block_table && context_lens && out, PA_ERR_INVALID,
             "%s: null pointer argument", fn);
  PA_REQUIRE(kv_dtype != pa::kFP8E4M3 || (k_scale && v_scale), PA_ERR_INVALID, "%s: null scale pointer", fn);
  PA_REQUIRE((k_new == nullptr) == (v_new == nullptr), PA_ERR_INVALID, "%s: null new-token pointer", fn);
  const size_t need = pa::decode_workspace_size(num_seqs, num_q_heads, head_dim, block_size, max_blocks_per_seq);
  PA_REQUIRE(workspace && workspace_bytes >= need, PA_ERR_WORKSPACE,
             "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? workspace_bytes : (size_t)0);
  pa::AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.out = out;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.dtype = dtype;
  a.kv_dtype = kv_dtype;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.workspace = workspace;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_dtype = new_dtype;
  return hip_status(pa::launch_decode(a, static_cast<hipStream_t>(stream), g_ev_start, g_ev_stop), fn);
}

}  // namespace

extern "C" {

int pa_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens, float scale,
                              void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err.clear();
  return decode_call("pa_paged_decode_attention", q, k_cache, v_cache, nullptr, nullptr, block_table, context_lens,
                     scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, dtype, dtype, workspace, workspace_bytes, stream);
}

int pa_paged_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                  const float* v_scale, const int32_t* block_table, const int32_t* context_lens,
                                  float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  g_err.clear();
  return decode_call("pa_paged_decode_attention_fp8", q, k_cache, v_cache, k_scale, v_scale, block_table,
                     context_lens, scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, PA_DTYPE_BF16, pa::kFP8E4M3, workspace, workspace_bytes, stream);
}

int pa_paged_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* block_table, const int32_t* context_lens, float scale, void* out,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  const char* fn = "pa_paged_decode_append";
  PA_REQUIRE(num_seqs == 0 || (k_new && v_new), PA_ERR_INVALID, "%s: null pointer argument", fn);
  return decode_call(fn, q, k_cache, v_cache, nullptr, nullptr, block_table, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, dtype, dtype,
                     workspace, workspace_bytes, stream, k_new, v_new, dtype);
}

int pa_paged_decode_append_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const float* k_scale, const float* v_scale, const int32_t* block_table,
                               const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_blocks_per_seq, int32_t new_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  g_err.clear();
  const char* fn = "pa_paged_decode_append_fp8";
  PA_REQUIRE(dtype_ok(new_dtype), PA_ERR_UNSUPPORTED, "%s: unsupported dtype %d of the new rows", fn, new_dtype);
  PA_REQUIRE(num_seqs == 0 || (k_new && v_new), PA_ERR_INVALID, "%s: null pointer argument", fn);
  return decode_call(fn, q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, PA_DTYPE_BF16,
                     pa::kFP8E4M3, workspace, workspace_bytes, stream, k_new, v_new, new_dtype);
}

size_t pa_prefill_workspace_size(int32_t num_seqs, int64_t total_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads) {
  if (num_seqs < 0 || total_q_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1) return 0;
  return pa::prefill_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads);
}

}  // extern "C"

namespace {

// Kinds of varlen call: the prefill kernel, or the mixed prefill/decode kernel.
enum VarlenKind { kVarlenPrefill, kVarlenMixed };

int prefill_call(VarlenKind kind, const char* fn, const void* q, const void* k, const void* v,
                 const float* k_scale, const float* v_scale, const int32_t* cu_seqlens, const int32_t* block_table,
                 const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int64_t total_q_tokens,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                 int32_t max_blocks_per_seq, int32_t dtype, int32_t kv_dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int st = check_attn(fn, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, dtype);
  if (st != PA_OK) return st;
  PA_REQUIRE(total_q_tokens >= 0 && total_q_tokens <= INT_MAX, PA_ERR_INVALID,
             "%s: total_q_tokens must be in [0, 2^31)", fn);
  PA_REQUIRE(dtype == PA_DTYPE_BF16, PA_ERR_UNSUPPORTED, "%s: prefill is provided for bf16 only", fn);
  PA_REQUIRE(num_q_heads / num_kv_heads <= 64, PA_ERR_UNSUPPORTED,
             "%s: GQA group size above 64 is not provided", fn);
  PA_REQUIRE(max_blocks_per_seq <= pa::kPrefillMaxBlocks, PA_ERR_UNSUPPORTED,
             "%s: max_blocks_per_seq above %d is not provided (a request's block ids are held in LDS)", fn,
             pa::kPrefillMaxBlocks);
  PA_REQUIRE(scale > 0.0f && scale < INFINITY, PA_ERR_INVALID, "%s: scale must be positive and finite", fn);
  if (total_q_tokens == 0) return PA_OK;
  PA_REQUIRE(num_seqs >= 1, PA_ERR_INVALID, "%s: %lld query tokens but no sequence", fn,
             (long long)total_q_tokens);
  PA_REQUIRE(q && k && v && cu_seqlens && block_table && context_lens && out, PA_ERR_INVALID,
             "%s: null pointer argument", fn);
  PA_REQUIRE(kv_dtype != pa::kFP8E4M3 || (k_scale && v_scale), PA_ERR_INVALID, "%s: null scale pointer", fn);
  if (kind == kVarlenMixed) {
    PA_REQUIRE(num_seqs <= pa::mixed_max_seqs(), PA_ERR_UNSUPPORTED,
               "%s: more than %d requests is not provided (the work lists are derived on chip)", fn,
               pa::mixed_max_seqs());
    PA_REQUIRE(pa::mixed_fits(num_seqs, total_q_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                              max_blocks_per_seq),
               PA_ERR_UNSUPPORTED, "%s: the batch's work lists exceed the queue counters' range", fn);
  }
  const size_t need =
      kind == kVarlenMixed
          ? pa::mixed_workspace_size(num_seqs, num_q_heads, head_dim, block_size, max_blocks_per_seq)
          : pa::prefill_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads);
  PA_REQUIRE(workspace && workspace_bytes >= need, PA_ERR_WORKSPACE,
             "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? workspace_bytes : (size_t)0);
  pa::AttnArgs a{};
  a.q = q;
  a.k_cache = k;
  a.v_cache = v;
  a.cu_seqlens = cu_seqlens;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.out = out;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_tokens = total_q_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.dtype = dtype;
  a.kv_dtype = kv_dtype;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.workspace = workspace;
  if (kind == kVarlenMixed)
    return hip_status(pa::launch_mixed(a, static_cast<hipStream_t>(stream), g_ev_start, g_ev_stop), fn);
  return hip_status(pa::launch_prefill(a, static_cast<hipStream_t>(stream), g_ev_start, g_ev_stop), fn);
}

}  // namespace

extern "C" {

int pa_paged_prefill_attention(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                               const int32_t* block_table, const int32_t* context_lens, float scale,
                               void* out, int32_t num_seqs, int64_t total_q_tokens, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  return prefill_call(kVarlenPrefill, "pa_paged_prefill_attention", q, k, v, nullptr, nullptr, cu_seqlens,
                      block_table, context_lens, scale, out, num_seqs, total_q_tokens, num_q_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, dtype, dtype, workspace, workspace_bytes,
                      stream);
}

int pa_paged_prefill_attention_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                                   const float* v_scale, const int32_t* cu_seqlens, const int32_t* block_table,
                                   const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                                   int64_t total_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                   int32_t max_blocks_per_seq, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  g_err.clear();
  return prefill_call(kVarlenPrefill, "pa_paged_prefill_attention_fp8", q, k, v, k_scale, v_scale, cu_seqlens,
                      block_table, context_lens, scale, out, num_seqs, total_q_tokens, num_q_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, PA_DTYPE_BF16, pa::kFP8E4M3, workspace,
                      workspace_bytes, stream);
}

size_t pa_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_q_heads < 1 || head_dim < 1 || block_size < 1 || max_blocks_per_seq < 1) return 0;
  return pa::mixed_workspace_size(num_seqs, num_q_heads, head_dim, block_size, max_blocks_per_seq);
}

int pa_paged_mixed_attention(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             const int32_t* block_table, const int32_t* context_lens, float scale, void* out,
                             int32_t num_seqs, int64_t total_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  return prefill_call(kVarlenMixed, "pa_paged_mixed_attention", q, k, v, nullptr, nullptr, cu_seqlens, block_table,
                      context_lens, scale, out, num_seqs, total_q_tokens, num_q_heads, num_kv_heads, head_dim,
                      block_size, num_blocks, max_blocks_per_seq, dtype, dtype, workspace, workspace_bytes, stream);
}

int pa_paged_mixed_attention_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                                 const float* v_scale, const int32_t* cu_seqlens, const int32_t* block_table,
                                 const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                                 int64_t total_q_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err.clear();
  return prefill_call(kVarlenMixed, "pa_paged_mixed_attention_fp8", q, k, v, k_scale, v_scale, cu_seqlens,
                      block_table, context_lens, scale, out, num_seqs, total_q_tokens, num_q_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, PA_DTYPE_BF16, pa::kFP8E4M3, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode attention for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid hipMalloc).  The decode workspace lives
// in a file-scope device array; each device holds its own copy until the
// process ends.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, resolved once per device
// with that device current, and is what the kernels receive.
// ---------------------------------------------------------------------------
namespace {

__device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (the stream's device).
int scratch_address(const char* fn, hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  PA_REQUIRE(dev >= 0 && dev < kMaxDevices, PA_ERR_UNSUPPORTED, "%s: device %d beyond the first %d", fn, dev,
             kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e, fn);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, fn);
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return hip_status(e, fn);
    if (es != hipSuccess) return hip_status(es, fn);
    PA_REQUIRE(p != nullptr, PA_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_table, const int32_t* context_lens, float scale,
                                                 void* out, int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int64_t num_blocks, int32_t max_blocks_per_seq, int32_t dtype,
                                                 void* stream) {
  g_err.clear();
  const char* fn = "pa_paged_decode_attention_noalloc";
  int st = check_attn(fn, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, dtype);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  const size_t need = pa::decode_workspace_size(num_seqs, num_q_heads, head_dim, block_size, max_blocks_per_seq);
  PA_REQUIRE(need <= (size_t)PA_NOALLOC_SCRATCH_BYTES, PA_ERR_WORKSPACE,
             "%s: this batch needs %zu bytes of workspace, beyond the %zu-byte static scratch (use "
             "pa_paged_decode_attention with a workspace of that size)",
             fn, need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(fn, static_cast<hipStream_t>(stream), &ws);
  if (st != PA_OK) return st;
  return decode_call(fn, q, k_cache, v_cache, nullptr, nullptr, block_table, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, dtype, dtype,
                     ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int pa_workspace_status(void* workspace, int32_t* result, void* stream) {
  g_err.clear();
  const char* fn = "pa_workspace_status";
  PA_REQUIRE(result, PA_ERR_INVALID, "%s: null result pointer", fn);
  void* ws = workspace;
  if (!ws) {
    const int st = scratch_address(fn, static_cast<hipStream_t>(stream), &ws);
    if (st != PA_OK) return st;
  }
  return hip_status(pa::launch_workspace_status(ws, result, static_cast<hipStream_t>(stream)), fn);
}
