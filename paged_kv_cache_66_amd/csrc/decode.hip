// Paged GQA decode attention with split-K over token partitions.
//
// What is computed ("Inference Engine Inside nano-vLLM", "Attention in
// nano-vLLM", flash_attn_with_kvcache branch; "From nano-vLLM to vLLM ...",
// section 11.2): every sequence has one query token per query head and
// attends over its context_len cached rows, found through its block-table
// row ("nano-vLLM Part 2 ...", section 2.2: logical row p is in block
// table[p / block_size] at offset p % block_size).
//
// Work decomposition (MI355X): one 256-thread workgroup per (partition of
// `partition` tokens, kv head, sequence). The G = H_q / H_kv query heads of
// a kv head are handled together, so each K/V row is read from HBM once per
// kv head and applied to all G heads from registers.
//   phase 0  the partition's block ids are staged in LDS (one coalesced load
//            instead of a dependent table read per row);
//   phase 1  K rows stream in as 16-byte vectors: a row of one kv head
//            (head_dim elements) is spread over LPT lanes, a wave covers
//            64 / LPT rows per load; each lane dots its slice against the G
//            query slices held in registers and the LPT partial sums are
//            combined with cross-lane shuffles; scores (already scaled by
//            scale * log2 e) go to LDS, token-major;
//   phase 2  exact per-head max and sum of exp2(s - max) over the partition
//            (no running rescale is needed because all scores are known);
//   phase 3  V rows stream in the same way; each lane accumulates
//            p * v for its slice of head_dim and the G heads;
//   phase 4  partial sums are reduced across the rows of a wave (shuffles)
//            and across waves (LDS, fixed order), then either the
//            normalised output is written (single partition) or the
//            (max, sum, unnormalised output) partial goes to the workspace.
// A second kernel merges the partials of a (sequence, query head) with the
// log-sum-exp rule. Summation order depends only on logical positions, so
// the result is bitwise independent of where blocks sit in the pool.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;

template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = LPT / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Dynamic LDS layout of the partition kernel (in 4-byte words):
//   [0, G * max(partition, 4 * D))   scores, then reused for the wave reduction
//   then G maxima, G sums, then the partition's block ids.
template <typename T, int D, int G>
__global__ void __launch_bounds__(kThreads) decode_partition_kernel(
    void* __restrict__ out, const char* __restrict__ q, int64_t q_stride_bytes,
    const char* __restrict__ k_cache, const char* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t log2_bs, float scale_log2, int32_t partition, int32_t num_partitions,
    int32_t score_words, float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
  using E = Elem<T>;
  constexpr int EPV = E::kPerVec;    // elements per 16-byte vector
  constexpr int EB = E::kBytes;      // bytes per element
  constexpr int LPT = D / EPV;       // lanes per (token, kv head) row
  constexpr int TPW = 64 / LPT;      // rows per wave per load
  constexpr int STEP = kWaves * TPW; // rows per workgroup per load

  extern __shared__ float lds[];
  float* s_score = lds;                                   // [partition][G]
  float* s_max = lds + score_words;                       // [G]
  float* s_sum = s_max + G;                               // [G]
  int32_t* s_ids = reinterpret_cast<int32_t*>(s_sum + G);  // block ids of the partition

  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane / LPT;
  const int li = lane % LPT;

  const int n = context_lens[b];
  const int t0 = p * partition;
  const bool single = (num_partitions == 1);
  if (t0 >= n) {
    // Nothing to attend to. A one-pass call still owes its zero output row.
    if (single && p == 0) {
      for (int i = tid; i < G * D; i += kThreads) {
        const int h = g * G + i / D;
        const int d = i % D;
        const int64_t o = (static_cast<int64_t>(b) * num_q_heads + h) * D + d;
        if constexpr (EB == 2) {
          reinterpret_cast<uint16_t*>(out)[o] = 0;
        } else {
          reinterpret_cast<float*>(out)[o] = 0.f;
        }
      }
    }
    return;
  }
  const int t1 = min(n, t0 + partition);
  const int ntok = t1 - t0;
  const int bs_mask = (1 << log2_bs) - 1;
  const int jb0 = t0 >> log2_bs;
  const int nblk = ((t1 - 1) >> log2_bs) - jb0 + 1;

  // phase 0: block ids of this partition
  const int32_t* table = block_tables + static_cast<int64_t>(b) * max_blocks;
  for (int i = tid; i < nblk; i += kThreads) s_ids[i] = table[jb0 + i];

  // query slices, pre-scaled so scores land in the log2 domain
  float qf[G][EPV];
  {
    const char* qrow = q + static_cast<int64_t>(b) * q_stride_bytes;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const Vec16 v = load16(qrow + (static_cast<int64_t>(g * G + h) * D + li * EPV) * EB);
      E::to_f32(v, qf[h]);
#pragma unroll
      for (int e = 0; e < EPV; ++e) qf[h][e] *= scale_log2;
    }
  }
  __syncthreads();

  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * D * EB;
  const int64_t lane_off = static_cast<int64_t>(g) * D * EB + li * 16;
  const int my_row = wave * TPW + grp;  // row of this lane within a load step

  // phase 1: scores
  for (int base = 0; base < ntok; base += STEP * kUnroll) {
    Vec16 kv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * STEP + my_row;
      if (tl < ntok) {
        const int pos = t0 + tl;
        const int64_t blk = s_ids[(pos >> log2_bs) - jb0];
        const int64_t off = ((blk << log2_bs) + (pos & bs_mask)) * row_bytes + lane_off;
        kv[u] = load16(k_cache + off);
      } else {
        kv[u] = Vec16{{0u, 0u, 0u, 0u}};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * STEP + my_row;
      float kf[EPV];
      E::to_f32(kv[u], kf);
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc = fmaf(qf[h][e], kf[e], acc);
        sc[h] = group_sum<LPT>(acc);
      }
      if (li == 0 && tl < ntok) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_score[tl * G + h] = sc[h];
      }
    }
  }
  __syncthreads();

  // phase 2: exact max and sum of exp2(s - max) per head; p overwrites s
  for (int h = wave; h < G; h += kWaves) {
    float m = -INFINITY;
    for (int t = lane; t < ntok; t += 64) m = fmaxf(m, s_score[t * G + h]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < ntok; t += 64) {
      const float e = exp2f(s_score[t * G + h] - m);
      s_score[t * G + h] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      s_max[h] = m;
      s_sum[h] = l;
    }
  }
  __syncthreads();

  // phase 3: weighted sum of V rows
  float acc[G][EPV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[h][e] = 0.f;

  for (int base = 0; base < ntok; base += STEP * kUnroll) {
    Vec16 vv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * STEP + my_row;
      if (tl < ntok) {
        const int pos = t0 + tl;
        const int64_t blk = s_ids[(pos >> log2_bs) - jb0];
        const int64_t off = ((blk << log2_bs) + (pos & bs_mask)) * row_bytes + lane_off;
        vv[u] = load16(v_cache + off);
      } else {
        vv[u] = Vec16{{0u, 0u, 0u, 0u}};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * STEP + my_row;
      if (tl < ntok) {
        float vf[EPV];
        E::to_f32(vv[u], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float w = s_score[tl * G + h];
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[h][e] = fmaf(w, vf[e], acc[h][e]);
        }
      }
    }
  }

  // phase 4: reduce over the rows of a wave, then over waves in fixed order
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      float v = acc[h][e];
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
      acc[h][e] = v;
    }
  __syncthreads();  // all reads of p are done; the score area becomes the reduction area
  float* s_red = lds;  // [kWaves][G][D]
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPV; ++e) s_red[(wave * G + h) * D + li * EPV + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i % D;
    float v = s_red[(0 * G + h) * D + d];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += s_red[(w * G + h) * D + d];
    const int qh = g * G + h;
    if (single) {
      const float o = v / s_sum[h];
      const int64_t oi = (static_cast<int64_t>(b) * num_q_heads + qh) * D + d;
      if constexpr (EB == 2) {
        reinterpret_cast<uint16_t*>(out)[oi] = static_cast<uint16_t>(f32_to_bf16_bits(o));
      } else {
        reinterpret_cast<float*>(out)[oi] = o;
      }
    } else {
      const int64_t slot = (static_cast<int64_t>(b) * num_q_heads + qh) * num_partitions + p;
      ws_acc[slot * D + d] = v;
      if (d == 0) {
        ws_ml[slot * 2 + 0] = s_max[h];
        ws_ml[slot * 2 + 1] = s_sum[h];
      }
    }
  }
}

// Log-sum-exp merge of the partition partials of one (sequence, query head):
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  o = sum_p 2^(m_p - M) acc_p / L.
template <typename T, int D>
__global__ void __launch_bounds__(64) decode_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ context_lens, int32_t num_q_heads, int32_t partition,
    int32_t num_partitions) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int n = context_lens[b];
  const int np = (n + partition - 1) / partition;
  const int64_t slot0 = (static_cast<int64_t>(b) * num_q_heads + h) * num_partitions;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  if (np > 0) {
    float M = -INFINITY;
    for (int pp = 0; pp < np; ++pp) M = fmaxf(M, ws_ml[(slot0 + pp) * 2]);
    float L = 0.f;
    for (int pp = 0; pp < np; ++pp) {
      const float w = exp2f(ws_ml[(slot0 + pp) * 2] - M);
      L = fmaf(ws_ml[(slot0 + pp) * 2 + 1], w, L);
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] = fmaf(w, ws_acc[(slot0 + pp) * D + k * 64 + lane], o[k]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] *= inv;
  }
  const int64_t ob = (static_cast<int64_t>(b) * num_q_heads + h) * D;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if constexpr (Elem<T>::kBytes == 2) {
      reinterpret_cast<uint16_t*>(out)[ob + k * 64 + lane] = static_cast<uint16_t>(f32_to_bf16_bits(o[k]));
    } else {
      reinterpret_cast<float*>(out)[ob + k * 64 + lane] = o[k];
    }
  }
}

template <typename T, int D, int G>
hipError_t launch_decode_typed(const DecodeArgs& a, hipStream_t stream) {
  constexpr int EB = Elem<T>::kBytes;
  int log2_bs = 0;
  while ((1 << log2_bs) < a.block_size) ++log2_bs;
  const int score_words = G * (a.partition > 4 * D ? a.partition : 4 * D);
  const int max_ids = a.partition / (a.block_size < a.partition ? a.block_size : a.partition) + 2;
  const size_t lds = static_cast<size_t>(score_words + 2 * G + max_ids) * 4;
  const float scale_log2 = a.scale * kLog2e;
  dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, G>), grid, dim3(kThreads), lds, stream, a.out,
                     static_cast<const char*>(a.q), a.q_stride * EB,
                     static_cast<const char*>(a.k_cache), static_cast<const char*>(a.v_cache),
                     a.block_tables, a.max_blocks, a.context_lens, a.num_q_heads, a.num_kv_heads,
                     log2_bs, scale_log2, a.partition, a.num_partitions, score_words, a.ws_acc,
                     a.ws_ml);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_partitions == 1) return err;
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0,
                     stream, a.out, a.ws_acc, a.ws_ml, a.context_lens, a.num_q_heads, a.partition,
                     a.num_partitions);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_group(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_decode_typed<T, D, 1>(a, stream);
    case 2: return launch_decode_typed<T, D, 2>(a, stream);
    case 4: return launch_decode_typed<T, D, 4>(a, stream);
    case 8: return launch_decode_typed<T, D, 8>(a, stream);
    case 16: return launch_decode_typed<T, D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int32_t decode_partition_tokens(int32_t requested, int32_t block_size, int32_t max_blocks) {
  (void)block_size;
  (void)max_blocks;
  return requested > 0 ? requested : 512;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16) {
    return a.head_dim == 64 ? dispatch_group<BF16Tag, 64>(a, stream)
                            : dispatch_group<BF16Tag, 128>(a, stream);
  }
  return a.head_dim == 64 ? dispatch_group<float, 64>(a, stream)
                          : dispatch_group<float, 128>(a, stream);
}

}  // namespace pa
