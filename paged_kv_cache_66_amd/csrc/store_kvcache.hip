// KV scatter through slot_mapping.
//
// The pages' store kernel runs one program per token and copies the token's
// whole K row and V row to slot * row_length ("Inference Engine Inside
// nano-vLLM", "Attention in nano-vLLM"). Here a token row is moved as
// 16-byte vectors: a group of consecutive threads covers one row, each
// thread carrying the same vector index for K and for V, so every wave issues
// fully coalesced 16-byte loads and stores and keeps two loads in flight per
// thread. A 256-thread workgroup covers 256 / vectors-per-row tokens; rows
// longer than 4 KiB are looped over. Address arithmetic is 64-bit: a pool can
// exceed 2^31 bytes.
//
// E4M3 caches (FP8): the bf16 input rows are quantised on the way, each
// element divided by the tensor's scale in fp32 and rounded to the nearest
// E4M3 code (ties to even, saturating at +-448); a 16-byte input vector
// becomes an 8-byte cache vector.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

template <bool FP8>
__global__ void __launch_bounds__(kThreads) store_kvcache_kernel(
    const char* __restrict__ key, int64_t key_stride, const char* __restrict__ value,
    int64_t value_stride, char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t vecs_per_row,
    int32_t tokens_per_block, int32_t cache_row_bytes, float k_scale, float v_scale) {
  int32_t lane_token, c0, cstep;
  if (tokens_per_block > 0) {
    lane_token = static_cast<int32_t>(threadIdx.x) / vecs_per_row;
    c0 = static_cast<int32_t>(threadIdx.x) - lane_token * vecs_per_row;
    cstep = vecs_per_row;  // one vector per thread
    if (lane_token >= tokens_per_block) return;
  } else {
    lane_token = 0;
    c0 = threadIdx.x;
    cstep = kThreads;
  }
  const int32_t t = static_cast<int32_t>(blockIdx.x) * (tokens_per_block > 0 ? tokens_per_block : 1) +
                    lane_token;
  if (t >= num_tokens) return;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;  // padding token: nothing to write
  const char* ksrc = key + static_cast<int64_t>(t) * key_stride;
  const char* vsrc = value + static_cast<int64_t>(t) * value_stride;
  const int64_t dst = static_cast<int64_t>(slot) * cache_row_bytes;
  for (int32_t c = c0; c < vecs_per_row; c += cstep) {
    const Vec16 kv = load16(ksrc + c * 16);
    const Vec16 vv = load16(vsrc + c * 16);
    if constexpr (FP8) {
      store8(k_cache + dst + c * 8, quantize8(kv, k_scale));
      store8(v_cache + dst + c * 8, quantize8(vv, v_scale));
    } else {
      store16(k_cache + dst + c * 16, kv);
      store16(v_cache + dst + c * 16, vv);
    }
  }
}

}  // namespace

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int32_t vecs = a.row_bytes / 16;
  const int32_t tpb = vecs <= kThreads ? kThreads / vecs : 0;
  const int32_t per = tpb > 0 ? tpb : 1;
  const int grid = (a.num_tokens + per - 1) / per;
  const int32_t cache_row_bytes = a.fp8 ? a.row_bytes / 2 : a.row_bytes;
  auto kernel = a.fp8 ? store_kvcache_kernel<true> : store_kvcache_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const char*>(a.key), a.key_stride_bytes,
                     static_cast<const char*>(a.value), a.value_stride_bytes,
                     static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache), a.slot_mapping,
                     a.num_tokens, vecs, tpb, cache_row_bytes, a.k_scale, a.v_scale);
  return hipGetLastError();
}

}  // namespace pa
