// C ABI entry points: argument validation on the host, then one or two
// kernel launches on the caller's stream. Nothing here reads device memory
// or synchronises, and no error path enqueues work.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pa_internal.h"

// The build writes the SHA-256 of the library's sources into this header.
#if __has_include("pa_srchash.h")
#include "pa_srchash.h"
#else
#define PA_SOURCE_SHA256 "unknown"
#endif

namespace {

constexpr int32_t kMaxBlockSize = 1024;
constexpr int32_t kMaxGridYZ = 65535;
constexpr int32_t kMaxPartition = 4096;
constexpr int32_t kMaxScoreWords = 8192;  // G * partition, bounded by LDS

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int elem_bytes(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }
bool dtype_ok(int d) { return d == PA_F32 || d == PA_BF16; }
bool group_ok(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

pa_status check_head_layout(int32_t head_dim, int32_t block_size, int32_t num_blocks) {
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!is_pow2(block_size) || block_size > kMaxBlockSize) return PA_ERR_UNSUPPORTED;
  if (num_blocks <= 0) return PA_ERR_SHAPE;
  // slots are int32
  if (static_cast<int64_t>(num_blocks) * block_size > static_cast<int64_t>(INT32_MAX) + 1) return PA_ERR_SHAPE;
  return PA_OK;
}

pa_status check_rows(const void* base, int64_t stride_elems, int64_t row_elems, int eb) {
  if (!aligned16(base)) return PA_ERR_ALIGN;
  if (stride_elems < row_elems) return PA_ERR_SHAPE;
  if ((stride_elems * eb) % 16 != 0) return PA_ERR_ALIGN;
  return PA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Partition length for a decode call, or -1 when the request is invalid.
int32_t resolve_partition(int32_t requested, int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                          int32_t block_size, int32_t max_blocks, int32_t elem_bytes) {
  if (requested < 0) return -1;
  if (requested > 0 && (requested % 64 != 0 || requested > kMaxPartition)) return -1;
  return pa::decode_partition_tokens(requested, num_seqs, num_kv_heads, group, block_size,
                                     max_blocks, elem_bytes);
}

int64_t num_partitions(int32_t partition, int32_t block_size, int32_t max_blocks) {
  return ceil_div(static_cast<int64_t>(max_blocks) * block_size, partition);
}



// Shared by pa_store_kvcache and pa_store_kvcache_fp8 (dtype already checked).
pa_status store_common(const void* key, int64_t key_row_stride, const void* value,
                       int64_t value_row_stride, void* k_cache, void* v_cache,
                       const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                       bool fp8, float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0) return PA_ERR_SHAPE;
  pa_status st = check_head_layout(head_dim, block_size, num_blocks);
  if (st != PA_OK) return st;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  if (num_tokens == 0) return PA_OK;
  if (key == nullptr || value == nullptr || slot_mapping == nullptr) return PA_ERR_NULL;
  const int eb = elem_bytes(dtype);
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  if ((st = check_rows(key, key_row_stride, row, eb)) != PA_OK) return st;
  if ((st = check_rows(value, value_row_stride, row, eb)) != PA_OK) return st;
  if (row * eb > INT32_MAX) return PA_ERR_SHAPE;
  pa::StoreArgs a{key, key_row_stride * eb, value, value_row_stride * eb, k_cache, v_cache,
                  slot_mapping, num_tokens, static_cast<int32_t>(row * eb), fp8, k_scale, v_scale};
  return pa::launch_store(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Validation and argument packing shared by pa_decode and pa_store_decode.
pa_status prepare_decode(void* out, const void* q, int64_t q_row_stride, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                         int32_t partition_size, pa_dtype dtype, pa::KvFormat kv, float k_scale,
                         float v_scale, void* workspace, size_t workspace_bytes, bool static_ws,
                         pa::DecodeArgs* a) {
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (kv == pa::KvFormat::kFp8E4m3 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PA_ERR_SHAPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  const int32_t G = num_q_heads / num_kv_heads;
  if (!group_ok(G)) return PA_ERR_UNSUPPORTED;
  if (num_seqs > kMaxGridYZ || num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  pa_status st = check_head_layout(head_dim, block_size, num_blocks);
  if (st != PA_OK) return st;
  if (!scale_ok(scale)) return PA_ERR_SHAPE;
  const int32_t part = resolve_partition(partition_size, num_seqs, num_kv_heads, G, block_size,
                                         max_blocks_per_seq,
                                         kv == pa::KvFormat::kFp8E4m3 ? 1 : kv == pa::KvFormat::kF32 ? 4 : 2);
  if (part <= 0) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(G) * part > kMaxScoreWords) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || q == nullptr || k_cache == nullptr || v_cache == nullptr ||
      block_tables == nullptr || context_lens == nullptr)
    return PA_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if (!aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  if ((st = check_rows(q, q_row_stride, static_cast<int64_t>(num_q_heads) * head_dim, eb)) != PA_OK)
    return st;
  const int64_t P = num_partitions(part, block_size, max_blocks_per_seq);
  // grid x = partitions * kv heads * sequences
  if (P * num_kv_heads * num_seqs > INT32_MAX) return PA_ERR_SHAPE;
  float* ws_acc = nullptr;
  float* ws_ml = nullptr;
  if (P > 1) {
    const size_t need = pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 block_size, max_blocks_per_seq, partition_size);
    if (static_ws) {
      // the library's fixed array, whose address the caller resolves once
      // every check has passed: only its size is checked here
      if (need > pa::kStaticWorkspaceBytes) return PA_ERR_WORKSPACE;
    } else {
      if (workspace == nullptr || workspace_bytes < need) return PA_ERR_WORKSPACE;
      if (!aligned16(workspace)) return PA_ERR_ALIGN;
      ws_acc = static_cast<float*>(workspace);
      ws_ml = ws_acc + static_cast<int64_t>(num_seqs) * num_q_heads * P * head_dim;
    }
  }
  *a = pa::DecodeArgs{};
  a->out = out;
  a->q = q;
  a->q_stride = q_row_stride;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->max_blocks = max_blocks_per_seq;
  a->context_lens = context_lens;
  a->num_seqs = num_seqs;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = num_kv_heads;
  a->head_dim = head_dim;
  a->block_size = block_size;
  a->scale = scale;
  a->partition = part;
  a->num_partitions = static_cast<int32_t>(P);
  a->ws_acc = ws_acc;
  a->ws_ml = ws_ml;
  a->kv = kv;
  a->k_scale = k_scale;
  a->v_scale = v_scale;
  return PA_OK;
}

pa_status decode_common(void* out, const void* q, int64_t q_row_stride, const void* key,
                        int64_t key_row_stride, const void* value, int64_t value_row_stride,
                        const int32_t* slot_mapping, bool fused, const void* k_cache,
                        const void* v_cache, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                        int32_t partition_size, pa_dtype dtype, pa::KvFormat kv, float k_scale,
                        float v_scale, void* workspace, size_t workspace_bytes, void* stream,
                        bool static_ws = false) {
  pa::DecodeArgs a;
  pa_status st = prepare_decode(out, q, q_row_stride, k_cache, v_cache, block_tables,
                                max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, num_blocks, scale,
                                partition_size, dtype, kv, k_scale, v_scale, workspace,
                                workspace_bytes, static_ws, &a);
  if (st != PA_OK || num_seqs == 0) return st;
  if (fused) {
    if (key == nullptr || value == nullptr || slot_mapping == nullptr) return PA_ERR_NULL;
    const int eb = elem_bytes(dtype);
    const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
    if ((st = check_rows(key, key_row_stride, row, eb)) != PA_OK) return st;
    if ((st = check_rows(value, value_row_stride, row, eb)) != PA_OK) return st;
  }
  if (static_ws && a.num_partitions > 1) {
    // every check has passed: resolve the fixed array's address on this device
    void* ws = nullptr;
    if (pa::static_workspace(&ws) != hipSuccess) return PA_ERR_HIP;
    a.ws_acc = static_cast<float*>(ws);
    a.ws_ml = a.ws_acc + static_cast<int64_t>(num_seqs) * num_q_heads * a.num_partitions * head_dim;
  }
  if (fused) {
    a.new_k = key;
    a.new_k_stride = key_row_stride;
    a.new_v = value;
    a.new_v_stride = value_row_stride;
    a.slot_mapping = slot_mapping;
  }
  return pa::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa::KvFormat kv_of(pa_dtype dtype) {
  return dtype == PA_BF16 ? pa::KvFormat::kBf16 : pa::KvFormat::kF32;
}

pa_status prefill_common(void* out, const void* q, int64_t q_row_stride, int32_t total_q,
                         const void* k, int64_t k_row_stride, const void* v, int64_t v_row_stride,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int32_t max_seqlen_q, int32_t max_seqlen_k, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, float scale, pa_dtype dtype, bool fp8, float k_scale,
                         float v_scale, void* stream, const void* new_k = nullptr,
                         int64_t new_k_stride = 0, const void* new_v = nullptr,
                         int64_t new_v_stride = 0, const int32_t* slot_mapping = nullptr) {
  if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PA_ERR_SHAPE;
  if (total_q < 0 || num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  const int32_t G = num_q_heads / num_kv_heads;
  if (!group_ok(G)) return PA_ERR_UNSUPPORTED;
  if (num_seqs > kMaxGridYZ || num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return PA_ERR_SHAPE;
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  const bool paged = block_tables != nullptr;
  pa_status st;
  if (paged) {
    if ((st = check_head_layout(head_dim, block_size, num_blocks)) != PA_OK) return st;
    if (max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
    // the caches are contiguous: a row stride, if given, must say so
    if ((k_row_stride != 0 && k_row_stride != row) || (v_row_stride != 0 && v_row_stride != row))
      return PA_ERR_SHAPE;
    k_row_stride = v_row_stride = row;
  } else {
    // packed rows: a tile of 64 rows must stay addressable with 32-bit offsets
    if (k_row_stride < row || v_row_stride < row) return PA_ERR_SHAPE;
    if (k_row_stride > (INT32_MAX / 2) / 64 || v_row_stride > (INT32_MAX / 2) / 64) return PA_ERR_SHAPE;
    if ((k_row_stride * 2) % 16 != 0 || (v_row_stride * 2) % 16 != 0) return PA_ERR_ALIGN;
  }
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PA_OK;
  if (out == nullptr || q == nullptr || k == nullptr || v == nullptr || cu_seqlens_q == nullptr ||
      cu_seqlens_k == nullptr)
    return PA_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if (!aligned16(out) || !aligned16(k) || !aligned16(v)) return PA_ERR_ALIGN;
  if ((st = check_rows(q, q_row_stride, static_cast<int64_t>(num_q_heads) * head_dim, eb)) != PA_OK)
    return st;
  const bool fused = slot_mapping != nullptr;
  if (fused) {
    if (new_k == nullptr || new_v == nullptr) return PA_ERR_NULL;
    if ((st = check_rows(new_k, new_k_stride, row, eb)) != PA_OK) return st;
    if ((st = check_rows(new_v, new_v_stride, row, eb)) != PA_OK) return st;
    // a tile of 64 new rows is addressed with 32-bit offsets, as packed k / v
    if (new_k_stride > (INT32_MAX / 2) / 64 || new_v_stride > (INT32_MAX / 2) / 64) return PA_ERR_SHAPE;
  }
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.q_stride = q_row_stride;
  a.total_q = total_q;
  a.k_cache = k;
  a.v_cache = v;
  a.k_stride = k_row_stride;
  a.v_stride = v_row_stride;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.max_seqlen_q = max_seqlen_q;
  a.max_seqlen_k = max_seqlen_k;
  a.block_tables = block_tables;
  a.max_blocks = paged ? max_blocks_per_seq : 0;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = paged ? block_size : 1;
  a.scale = scale;
  a.fp8 = fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  if (fused) {
    a.new_k = new_k;
    a.new_k_stride = new_k_stride;
    a.new_v = new_v;
    a.new_v_stride = new_v_stride;
    a.slot_mapping = slot_mapping;
  }
  return pa::launch_prefill(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer argument";
    case PA_ERR_SHAPE: return "invalid or inconsistent size";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, group size, dtype or mode";
    case PA_ERR_ALIGN: return "pointer or row stride not 16-byte aligned";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* pa_version(void) {
  return "paged_kv_cache_66_amd 0.2.0 (gfx950) src-sha256:" PA_SOURCE_SHA256;
}

pa_status pa_store_kvcache(const void* key, int64_t key_row_stride, const void* value,
                           int64_t value_row_stride, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           pa_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  return store_common(key, key_row_stride, value, value_row_stride, k_cache, v_cache, slot_mapping,
                      num_tokens, num_blocks, block_size, num_kv_heads, head_dim, dtype, false, 1.f,
                      1.f, stream);
}

pa_status pa_store_kvcache_fp8(const void* key, int64_t key_row_stride, const void* value,
                               int64_t value_row_stride, void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                               int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                               float k_scale, float v_scale, pa_dtype dtype, void* stream) {
  if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PA_ERR_SHAPE;
  return store_common(key, key_row_stride, value, value_row_stride, k_cache, v_cache, slot_mapping,
                      num_tokens, num_blocks, block_size, num_kv_heads, head_dim, dtype, true,
                      k_scale, v_scale, stream);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      head_dim <= 0 || !is_pow2(block_size) || max_blocks_per_seq <= 0)
    return 0;
  // sized for 16-bit caches: no cache format takes more partitions
  const int32_t part = resolve_partition(partition_size, num_seqs, num_kv_heads,
                                         num_q_heads / num_kv_heads, block_size, max_blocks_per_seq, 2);
  if (part <= 0) return 0;
  const int64_t P = num_partitions(part, block_size, max_blocks_per_seq);
  if (P <= 1) return 0;
  const int64_t slots = static_cast<int64_t>(num_seqs) * num_q_heads * P;
  return static_cast<size_t>(slots * head_dim * 4 + slots * 2 * 4);
}

pa_status pa_decode(void* out, const void* q, int64_t q_row_stride, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_common(out, q, q_row_stride, nullptr, 0, nullptr, 0, nullptr, false, k_cache,
                       v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                       partition_size, dtype, kv_of(dtype), 1.f, 1.f, workspace, workspace_bytes,
                       stream);
}

pa_status pa_store_decode(void* out, const void* q, int64_t q_row_stride, const void* key,
                          int64_t key_row_stride, const void* value, int64_t value_row_stride,
                          const int32_t* slot_mapping, void* k_cache, void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, float scale, int32_t partition_size,
                          pa_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return decode_common(out, q, q_row_stride, key, key_row_stride, value, value_row_stride,
                       slot_mapping, true, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_size, dtype, kv_of(dtype), 1.f, 1.f,
                       workspace, workspace_bytes, stream);
}

pa_status pa_store_decode_noalloc(void* out, const void* q, int64_t q_row_stride, const void* key,
                                  int64_t key_row_stride, const void* value, int64_t value_row_stride,
                                  const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, int32_t partition_size,
                                  pa_dtype dtype, void* stream) {
  // the split-K workspace is the library's fixed array (static_ws): looked
  // up after every other check, refused when the launch needs more
  return decode_common(out, q, q_row_stride, key, key_row_stride, value, value_row_stride,
                       slot_mapping, true, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_size, dtype, kv_of(dtype), 1.f, 1.f, nullptr, 0,
                       stream, /*static_ws=*/true);
}

pa_status pa_decode_fp8(void* out, const void* q, int64_t q_row_stride, const void* k_cache,
                        const void* v_cache, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                        float k_scale, float v_scale, int32_t partition_size, pa_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(out, q, q_row_stride, nullptr, 0, nullptr, 0, nullptr, false, k_cache,
                       v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                       partition_size, dtype, pa::KvFormat::kFp8E4m3, k_scale, v_scale,
                       workspace, workspace_bytes, stream);
}

pa_status pa_store_decode_fp8(void* out, const void* q, int64_t q_row_stride, const void* key,
                              int64_t key_row_stride, const void* value,
                              int64_t value_row_stride, const int32_t* slot_mapping,
                              void* k_cache, void* v_cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              float scale, float k_scale, float v_scale, int32_t partition_size,
                              pa_dtype dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_common(out, q, q_row_stride, key, key_row_stride, value, value_row_stride,
                       slot_mapping, true, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_size, dtype, pa::KvFormat::kFp8E4m3, k_scale,
                       v_scale, workspace, workspace_bytes, stream);
}

pa_status pa_prefill_varlen(void* out, const void* q, int64_t q_row_stride, int32_t total_q,
                            const void* k, int64_t k_row_stride, const void* v,
                            int64_t v_row_stride, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale, pa_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  return prefill_common(out, q, q_row_stride, total_q, k, k_row_stride, v, v_row_stride,
                        cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, block_tables,
                        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, dtype, false, 1.f, 1.f, stream);
}

pa_status pa_prefill_varlen_fp8(void* out, const void* q, int64_t q_row_stride, int32_t total_q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                float scale, float k_scale, float v_scale, pa_dtype dtype,
                                void* stream) {
  if (block_tables == nullptr) return PA_ERR_NULL;  // E4M3 data lives only in the paged caches
  return prefill_common(out, q, q_row_stride, total_q, k_cache, 0, v_cache, 0, cu_seqlens_q,
                        cu_seqlens_k, max_seqlen_q, max_seqlen_k, block_tables,
                        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, dtype, true, k_scale, v_scale, stream);
}

pa_status pa_store_prefill(void* out, const void* q, int64_t q_row_stride, int32_t total_q,
                           const void* key, int64_t key_row_stride, const void* value,
                           int64_t value_row_stride, const int32_t* slot_mapping, void* k_cache,
                           void* v_cache, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t max_seqlen_q, int32_t max_seqlen_k, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, float scale, pa_dtype dtype, void* stream) {
  if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (block_tables == nullptr) return PA_ERR_NULL;  // the fused call is paged only
  // an empty step stores nothing, so its slot mapping may be absent
  if (slot_mapping == nullptr && total_q > 0 && num_seqs > 0) return PA_ERR_NULL;
  return prefill_common(out, q, q_row_stride, total_q, k_cache, 0, v_cache, 0, cu_seqlens_q,
                        cu_seqlens_k, max_seqlen_q, max_seqlen_k, block_tables,
                        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, dtype, false, 1.f, 1.f, stream, key,
                        key_row_stride, value, value_row_stride, slot_mapping);
}

pa_status pa_store_prefill_fp8(void* out, const void* q, int64_t q_row_stride, int32_t total_q,
                               const void* key, int64_t key_row_stride, const void* value,
                               int64_t value_row_stride, const int32_t* slot_mapping,
                               void* k_cache, void* v_cache, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                               int32_t max_seqlen_k, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, float scale, float k_scale, float v_scale,
                               pa_dtype dtype, void* stream) {
  if (block_tables == nullptr) return PA_ERR_NULL;
  if (slot_mapping == nullptr && total_q > 0 && num_seqs > 0) return PA_ERR_NULL;
  return prefill_common(out, q, q_row_stride, total_q, k_cache, 0, v_cache, 0, cu_seqlens_q,
                        cu_seqlens_k, max_seqlen_q, max_seqlen_k, block_tables,
                        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, dtype, true, k_scale, v_scale, stream, key,
                        key_row_stride, value, value_row_stride, slot_mapping);
}

}  // extern "C"
