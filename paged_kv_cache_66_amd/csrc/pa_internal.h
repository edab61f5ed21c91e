// Internal launcher interface between the C ABI (pa_api.cpp) and the HIP
// kernels. All arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Storage format of the K/V caches. fp32 and bf16 caches share the element
// type of the queries and outputs; an E4M3 cache holds one-byte codes with a
// per-tensor scale each for K and V, next to bf16 queries and outputs.
enum class KvFormat { kF32, kBf16, kFp8E4m3 };

struct StoreArgs {
  const void* key;
  int64_t key_stride_bytes;
  const void* value;
  int64_t value_stride_bytes;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int32_t row_bytes;  // bytes of one input row: num_kv_heads * head_dim * input element bytes
  bool fp8;           // quantise bf16 input rows to E4M3 cache rows (row_bytes / 2 each)
  float k_scale;
  float v_scale;
};

hipError_t launch_store(const StoreArgs& a, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  int64_t q_stride;  // elements
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  float scale;
  int32_t partition;     // tokens per partition
  int32_t num_partitions;  // max partitions per sequence (grid x)
  float* ws_acc;         // [B, H_q, P, D] when num_partitions > 1
  float* ws_ml;          // [B, H_q, P, 2]
  KvFormat kv;
  float k_scale;         // E4M3 caches: stored code = K / k_scale (1 otherwise)
  float v_scale;
  // fused scatter of the step's new rows (slot_mapping == nullptr: plain decode)
  const void* new_k;
  int64_t new_k_stride;  // elements
  const void* new_v;
  int64_t new_v_stride;
  const int32_t* slot_mapping;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  int64_t q_stride;  // elements
  int32_t total_q;
  const void* k_cache;  // caches (paged) or packed k rows (block_tables == nullptr)
  const void* v_cache;
  int64_t k_stride;  // elements between key rows: H_kv * D for the caches
  int64_t v_stride;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  float scale;
  bool fp8;       // paged E4M3 caches (bf16 queries and outputs)
  float k_scale;
  float v_scale;
  // fused store (slot_mapping != nullptr): this step's new K/V rows, packed
  // like q (row cu_q[i] + j is position Lk - Lq + j of sequence i), are
  // written to the caches at slot_mapping[row] and read from here, never
  // from the caches, by the attention of the same launch
  const void* new_k;
  const void* new_v;
  int64_t new_k_stride;  // elements
  int64_t new_v_stride;
  const int32_t* slot_mapping;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Partition sizing shared by pa_decode and pa_decode_workspace_size
// (requested > 0 is returned as is; 0 picks the default for the shape and
// the cache element size: a one-byte cache takes partitions twice as long,
// so a workgroup still streams as many bytes). The default never shortens
// when elem_bytes shrinks, so sizing a workspace with elem_bytes = 2 covers
// every cache format.
int32_t decode_partition_tokens(int32_t requested, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t group, int32_t block_size, int32_t max_blocks,
                                int32_t elem_bytes);

// Fixed split-K workspace of the allocation-free decode entry point: its
// size, and its device address on the current device (looked up once per
// device; hipGetSymbolAddress allocates nothing).
constexpr size_t kStaticWorkspaceBytes = PA_NOALLOC_WORKSPACE_BYTES;
hipError_t static_workspace(void** ptr);

}  // namespace pa
