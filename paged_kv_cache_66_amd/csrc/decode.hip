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
// `partition` tokens, kv head, sequence), kv head fastest in dispatch order
// so the workgroups that read the head slices of the same token rows run
// side by side. The G = H_q / H_kv query heads of a kv head are handled
// together, so each K/V row is read from HBM once per kv head and applied to
// all G heads from registers.
//   phase 0  the partition's block ids are staged in LDS (one coalesced load
//            instead of a dependent table read per row);
//   phase 1  K rows stream in as 16-byte vectors: a row of one kv head
//            (head_dim elements) is spread over LPT lanes, a wave covers
//            64 / LPT rows per load; each lane dots its slice against the G
//            query slices held in registers (v_dot2_f32_bf16 on bf16) and
//            the LPT partial sums are combined with DPP row operations (a
//            reduce-scatter: each lane ends with the full scores of G / LPT
//            heads); raw scores go to LDS, token-major;
//   phase 2  exact per-head max and sum of exp2(s - max) over the partition
//            (no running rescale is needed because all scores are known);
//   phase 3  V rows stream in the same way; each lane accumulates
//            p * v for its slice of head_dim and the G heads (at G >= 8
//            over half vectors, so the accumulators and the query slices
//            fit four waves per SIMD);
//   phase 4  partial sums are reduced across the rows of a wave (shuffles)
//            and across waves (LDS, fixed order), then either the
//            normalised output is written (single partition) or the
//            (max, sum, unnormalised output) partial goes to the workspace.
// At G >= 8 with blocks of 256 rows or more (and partitions a multiple of
// 256), a kernel instantiation loads each half-trip of rows through one block
// lookup and a buffer resource (block trips), and its value pass takes a
// lane's rows in pairs, one v_dot2 with bf16 weights per element and head.
// A second kernel merges the partials of a (sequence, query head) with the
// log-sum-exp rule. Summation order depends only on logical positions, so
// the result is bitwise independent of where blocks sit in the pool.
#include <mutex>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Fourth word of a raw buffer resource (untyped 32-bit data format) and the
// cache-policy argument of a non-temporal buffer load.
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kLoadNt = 2;

// DPP lane patterns (gfx9 encoding): quad permutations and row mirrors.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPT consecutive lanes; every lane of a group
// receives the group's sum. Within a 16-lane row the steps are DPP moves
// folded into the adds (quad swaps, then the half-row and row mirrors, each
// of which pairs a lane with one in the other half of its current group);
// only a 32-lane group needs a cross-row exchange.
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16 || LPT == 32, "lanes per row");
  v = dpp_add<kDppQuadXor1>(v);
  v = dpp_add<kDppQuadXor2>(v);
  if constexpr (LPT >= 8) v = dpp_add<kDppRowHalfMirror>(v);
  if constexpr (LPT >= 16) v = dpp_add<kDppRowMirror>(v);
  if constexpr (LPT == 32) v += __shfl_xor(v, 16, 64);
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

// A row's G scores go to LDS as whole 16-byte (or 8 / 4-byte) stores: the
// row's slot s_score[t * G .. + G) is aligned to its own size.
template <int G>
__device__ __forceinline__ void store_scores(float* dst, const float (&sc)[G]) {
  if constexpr (G % 4 == 0) {
#pragma unroll
    for (int h = 0; h < G; h += 4)
      *reinterpret_cast<float4*>(dst + h) = make_float4(sc[h], sc[h + 1], sc[h + 2], sc[h + 3]);
  } else if constexpr (G == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(sc[0], sc[1]);
  } else {
    dst[0] = sc[0];
  }
}

// v + the same register of lane l ^ 16, then of lane l ^ 32: the cross-row
// swaps v_permlane16_swap / v_permlane32_swap return a value and its
// partner's (in either order), so every lane of the four gets the same sum.
__device__ __forceinline__ float sum_lanes_16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// v + the same register of lane l ^ 32 (v_permlane32_swap, as above)
__device__ __forceinline__ float sum_lanes_32(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Query slice of one head held by a lane for the score pass: NV 16-byte
// vectors of the head's row (the elements that match the lane's NV cache
// vectors), in the form the dot product wants: fp32 values for fp32 caches,
// raw bf16 pairs for bf16 caches (products of two bf16 values are exact in
// fp32, so v_dot2_f32_bf16 computes the same partial sums as widening first,
// with no conversion instructions).
template <typename T, int NV> struct QSlice;

template <int NV> struct QSlice<float, NV> {
  float v[4 * NV];
  __device__ __forceinline__ void load(int n, const Vec16& x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * n + e] = __uint_as_float(x.w[e]);
  }
  template <bool kZeroStart = false>
  __device__ __forceinline__ float dot(const Vec16 (&k)[NV]) const {
    float acc = 0.f;
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(v[4 * n + e], __uint_as_float(k[n].w[e]), acc);
    return acc;
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                         false);
}

// The first product of a chain: v_dot2_f32_bf16 with the inline constant 0
// as the addend. (Left to itself the compiler starts every chain with a
// v_mov of 0 into the accumulator of the two-operand v_dot2c form: one more
// vector instruction per chain, i.e. per head and row in the score pass.)
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <int NV> struct QSlice<BF16Tag, NV> {
  uint32_t v[4 * NV];
  __device__ __forceinline__ void load(int n, const Vec16& x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) v[4 * n + w] = x.w[w];
  }
  template <bool kZeroStart = false>
  __device__ __forceinline__ float dot(const Vec16 (&k)[NV]) const {
    float acc = kZeroStart ? dot2_bf16_first(v[0], k[0].w[0]) : dot2_bf16(v[0], k[0].w[0], 0.f);
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (n > 0 || w > 0) acc = dot2_bf16(v[4 * n + w], k[n].w[w], acc);
    return acc;
  }
};

// fp8 cache: the query stays bf16 (pairs as for a bf16 cache); each pair of
// E4M3 codes is widened to a bf16 pair (exact) and fed to v_dot2_f32_bf16.
template <int NV> struct QSlice<Fp8Tag, NV> {
  uint32_t v[4 * NV];
  __device__ __forceinline__ void load(int n, const Vec16& x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) v[4 * n + w] = x.w[w];
  }
  template <bool kZeroStart = false>
  __device__ __forceinline__ float dot(const Vec8 (&k)[NV]) const {
    const uint32_t k0 = e4m3x2_to_bf16x2<false>(k[0].w[0]);
    float acc = kZeroStart ? dot2_bf16_first(v[0], k0) : dot2_bf16(v[0], k0, 0.f);
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if (n > 0 || w > 0) acc = dot2_bf16(v[4 * n + 2 * w], e4m3x2_to_bf16x2<false>(k[n].w[w]), acc);
        acc = dot2_bf16(v[4 * n + 2 * w + 1], e4m3x2_to_bf16x2<true>(k[n].w[w]), acc);
      }
    return acc;
  }
};

// Reduce-scatter of the score pass. The LPT lanes of a row each hold G
// partial dot products; LPT is 2, 4, 8 or 16 (one DPP row at most). Step s
// pairs lane i with lane i ^ M_s, M = (15, 7, 2, 1) cut to its last
// log2(LPT) entries (row mirror, half-row mirror, quad swaps). While a lane
// holds V > 1 values, a step keeps the first V / 2 and adds the partner's
// second V / 2 to them (r_j += partner's r_{j + V/2}); once one value is left
// the remaining steps add the partner's value. For that to add partial sums of
// the same head, each lane orders its query heads so that register j holds
// head head_of(i, j): follow register j forward through the halving steps
// (the second half of the registers moves to the partner lane) and number the
// lane it ends in by its bits above the pair-sum steps. At the end lane i
// holds the full scores of heads (i >> TAIL) * VF + [0, VF), and the lanes that
// differ only in their low TAIL bits hold the same values.
template <int LPT, int G>
struct ScoreScatter {
  static constexpr int log2i(int x) { return x <= 1 ? 0 : 1 + log2i(x / 2); }
  static constexpr int S = log2i(LPT);
  static constexpr int K = S < log2i(G) ? S : log2i(G);  // halving steps
  static constexpr int VF = G >> K;                      // values left per lane
  static constexpr int TAIL = S - K;                     // pair-sum steps
  static_assert((1 << S) == LPT && LPT >= 1 && LPT <= 16, "lanes per row");
  static_assert((G & (G - 1)) == 0, "power-of-two group");
  static constexpr int mask(int s) { return s + 4 - S == 0 ? 15 : s + 4 - S == 1 ? 7 : s + 4 - S == 2 ? 2 : 1; }
  template <int s>
  __device__ __forceinline__ static float from_partner(float x) {
    constexpr int m = mask(s);
    constexpr int ctrl = m == 15 ? kDppRowMirror : m == 7 ? kDppRowHalfMirror : m == 2 ? kDppQuadXor2 : kDppQuadXor1;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, true));
  }
  __device__ __forceinline__ static int head_of(int li, int j) {
    int l = li;
    int v = G;
#pragma unroll
    for (int s = 0; s < K; ++s) {
      v /= 2;
      if (j >= v) {
        l ^= mask(s);
        j -= v;
      }
    }
    return (l >> TAIL) * VF + j;
  }
  template <int s = 0>
  __device__ __forceinline__ static void reduce(float (&r)[G]) {
    if constexpr (s < S) {
      if constexpr (s < K) {
        constexpr int half = G >> (s + 1);
#pragma unroll
        for (int j = 0; j < half; ++j) r[j] += from_partner<s>(r[j + half]);
      } else {
        r[0] += from_partner<s>(r[0]);
      }
      reduce<s + 1>(r);
    }
  }
};

// Dynamic LDS layout of the partition kernel (in 4-byte words):
//   [0, G * max(partition, 4 * D))   scores, then reused for the wave reduction
//   then G maxima, G sums, then the partition's block ids.
//
// T is the cache element type (fp32, bf16, or E4M3 codes with bf16 queries
// and outputs). For an E4M3 cache the score scale already carries k_scale and
// the output is multiplied by v_scale.
//
// With FUSED the step's new K/V rows are scattered by this kernel as well
// (one launch instead of pa_store_kvcache + pa_decode): the workgroup whose
// partition holds position context_len - 1 of a sequence writes that row's
// kv head slice to the cache at slot_mapping[b] (E4M3 caches: quantised with
// k_scale / v_scale first) and takes the row from the new key/value inputs
// instead of the cache. The caller guarantees that slot is the slot of
// position context_len - 1 (or -1: no store, row read from the cache).
template <typename T, int D, int G, bool FUSED, bool BT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BT && G == 8 ? 4 : 1))) decode_partition_kernel(
    void* __restrict__ out, const char* __restrict__ q, int64_t q_stride_bytes,
    char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t max_ctx, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t log2_bs, float scale_log2, int32_t partition, int32_t num_partitions,
    int32_t score_words, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    const char* __restrict__ new_k, int64_t new_k_stride_bytes, const char* __restrict__ new_v,
    int64_t new_v_stride_bytes, const int32_t* __restrict__ slot_mapping, float k_scale,
    float v_scale) {
  using E = Elem<T>;
  using Vec = typename E::Vec;
  constexpr bool kFp8 = E::kBytes == 1;
  constexpr int EPV = E::kPerVec;    // cache elements per lane vector
  constexpr int EB = E::kBytes;      // bytes per cache element
  constexpr int QB = E::kQBytes;     // bytes per query / output element
  constexpr int VB = EPV * EB;       // bytes per lane vector (16, or 8 for fp8)
  // score pass: a (token, kv head) row is spread over LPT1 lanes holding NV1
  // vectors each. Two vectors per lane halve the reduction steps; at G >= 8
  // one vector per lane halves the query registers (16-bit and fp8 caches,
  // whose scores are combined by the reduce-scatter above; fp32 caches keep
  // the all-lanes sum).
  constexpr bool kScatter = !std::is_same<T, float>::value;
  constexpr int NV1 = (kScatter && G >= 8) ? 1 : 2;
  constexpr int LPT1 = D / (NV1 * EPV);
  constexpr int TPW1 = 64 / LPT1;
  // 8-byte vectors (E4M3) in pairs: a lane's two vectors are adjacent and
  // travel as one 16-byte load, so a load instruction takes 128 contiguous
  // bytes of each row; 16-byte vectors take the row in two halves
  constexpr bool kPair = VB == 8 && NV1 == 2;
  constexpr int kSecond = kPair ? VB : LPT1 * VB;    // byte offset of the second vector
  constexpr int kFirst = kPair ? 2 * VB : VB;        // bytes between lanes' first vectors
  constexpr int STEP1 = kWaves * TPW1;
  // rows per lane and loop trip: 256 bytes of loads per lane, at most 16
  // rows; fp8 at G <= 4 takes 8 rows (128 bytes), which frees the registers
  // for five or six waves per SIMD instead of four
  constexpr int kUnroll1 = (kFp8 && G <= 4) ? 8 : (256 / (NV1 * VB) < 16 ? 256 / (NV1 * VB) : 16);
  // value pass: LPT lanes per row, one vector each (fewer accumulators); at
  // G >= 8 (16-bit and fp8 caches) half a vector each (8 bytes, or 4 fp8
  // codes), which halves the G x elements accumulators a lane keeps
  constexpr int NVH = (kScatter && G >= 8) ? 2 : 1;
  constexpr bool kPairV = NVH == 2 && BT;  // value pass in row pairs (see accum_pair)
  constexpr int EPVV = EPV / NVH;    // elements per lane in the value pass
  constexpr int VBV = VB / NVH;      // bytes per lane and row in the value pass
  constexpr int LPT = D / EPVV;      // lanes per (token, kv head) row
  constexpr int TPW = 64 / LPT;      // rows per wave per load
  constexpr int STEP = kWaves * TPW; // rows per workgroup per load
  // value pass: 16 vector loads in flight per lane (32 half vectors), so a
  // 256-token partition's V rows come in one trip
  constexpr int kUnrollV = 16 * NVH;
  using VVec = typename std::conditional<NVH == 1, Vec, typename std::conditional<kFp8, Vec4, Vec8>::type>::type;
  auto load_vv = [](const char* p) -> VVec {
    if constexpr (NVH == 1) {
      return E::load_nt(p);
    } else if constexpr (kFp8) {
      return Vec4{{__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p))}};
    } else {
      return load8_nt(p);
    }
  };
  auto vv_to_f32 = [](const VVec& v, float (&f)[EPVV]) {
    if constexpr (NVH == 1) {
      E::to_f32(v, f);
    } else if constexpr (kFp8) {
      // v_cvt_pk_f32_fp8: two codes per instruction, exact
      typedef float f32x2_t __attribute__((ext_vector_type(2)));
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v.w[0]), false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v.w[0]), true);
      f[0] = lo.x;
      f[1] = lo.y;
      f[2] = hi.x;
      f[3] = hi.y;
    } else {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        f[2 * w] = bf16_lo(v.w[w]);
        f[2 * w + 1] = bf16_hi(v.w[w]);
      }
    }
  };

  // fused: the new row's K and V head slices, in cache format, come first
  constexpr int kNewWords = FUSED ? 2 * D * EB / 4 : 0;
  extern __shared__ float lds[];
  char* s_new = reinterpret_cast<char*>(lds);             // [2][D] cache elements
  float* s_score = lds + kNewWords;                       // [partition][G]
  float* s_max = s_score + score_words;                   // [G]
  float* s_sum = s_max + G;                               // [G]
  float* s_wred = s_sum + G;                              // [kWaves][G] per-wave maxima, then sums
  int32_t* s_ids = reinterpret_cast<int32_t*>(s_wred + kWaves * G);  // block ids of the partition

  // Dispatch order: kv head fastest, then sequence, then partition. The
  // workgroups that read the head slices of the same token rows run side by
  // side, and sequences that share prefix blocks read them at the same time.
  const int num_seqs = gridDim.x / (num_kv_heads * num_partitions);
  const int g = static_cast<int>(blockIdx.x) % num_kv_heads;
  const int b = (static_cast<int>(blockIdx.x) / num_kv_heads) % num_seqs;
  const int p = static_cast<int>(blockIdx.x) / (num_kv_heads * num_seqs);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane / LPT;
  const int li = lane % LPT;

  // a history never runs past its table row (max_ctx = max_blocks * block_size)
  const int n = min(context_lens[b], max_ctx);
  const int t0 = p * partition;
  const bool single = (num_partitions == 1);
  if (t0 >= n) {
    // Nothing to attend to. A one-pass call still owes its zero output row.
    if (single && p == 0) {
      for (int i = tid; i < G * D; i += kThreads) {
        const int h = g * G + i / D;
        const int d = i % D;
        const int64_t o = (static_cast<int64_t>(b) * num_q_heads + h) * D + d;
        if constexpr (QB == 2) {
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
  const uint32_t bs_mask = (1u << log2_bs) - 1u;
  const int jb0 = t0 >> log2_bs;
  const int nblk = ((t1 - 1) >> log2_bs) - jb0 + 1;

  // phase 0: block ids of this partition
  const int32_t* table = block_tables + static_cast<int64_t>(b) * max_blocks;
  for (int i = tid; i < nblk; i += kThreads) s_ids[i] = table[jb0 + i];

  // The step's new row (fused scatter). When this partition holds position
  // n - 1 and the slot is >= 0, new_tl = n - 1 - t0 = ntok - 1: the last row
  // of the partition. Its head slices are written to the cache slot
  // (quantised first for an E4M3 cache) and to LDS, and nothing in this
  // launch reads them back from the cache: the loops below stop one row
  // short, and the row's score and weighted value are taken from LDS after
  // them. Every lane takes its rows in increasing order, so handling the last
  // row after the loop keeps the summation order of pa_decode.
  const int row_bytes_h = D * EB;  // one kv head's slice of a cache row
  int new_tl = -1;
  if constexpr (FUSED) {
    const int slot = slot_mapping[b];
    if (slot >= 0 && n - 1 >= t0 && n - 1 < t1) {
      new_tl = n - 1 - t0;
      constexpr int kVecs = D / EPV;  // lane vectors per head slice
      if (tid < 2 * kVecs) {
        const bool is_v = tid >= kVecs;
        const int c = is_v ? tid - kVecs : tid;
        const char* row = is_v ? new_v + static_cast<int64_t>(b) * new_v_stride_bytes
                               : new_k + static_cast<int64_t>(b) * new_k_stride_bytes;
        const Vec16 x = load16(row + (static_cast<int64_t>(g) * D + c * EPV) * QB);
        Vec y;
        if constexpr (kFp8) {
          y = quantize8(x, is_v ? v_scale : k_scale);
        } else {
          y = x;
        }
        const int64_t dst = static_cast<int64_t>(slot) * static_cast<int64_t>(num_kv_heads) * row_bytes_h +
                            static_cast<int64_t>(g) * row_bytes_h + c * VB;
        *reinterpret_cast<Vec*>((is_v ? v_cache : k_cache) + dst) = y;
        *reinterpret_cast<Vec*>(s_new + (is_v ? row_bytes_h : 0) + c * VB) = y;
      }
    }
  }

  const int grp1 = lane / LPT1;
  const int li1 = lane % LPT1;
  using Scatter = ScoreScatter<(kScatter ? LPT1 : 1), G>;
  // query head of the lane's register h: in order for the all-lanes sum, the
  // reduce-scatter's per-lane order otherwise
  auto qhead = [&](int h) { return kScatter ? Scatter::head_of(li1, h) : h; };
  QSlice<T, NV1> qs[G];
  {
    // the query elements that match the lane's K vectors: 16 bytes each
    const char* qrow = q + static_cast<int64_t>(b) * q_stride_bytes;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const char* qh = qrow + static_cast<int64_t>(g * G + qhead(h)) * D * QB;
#pragma unroll
      for (int n = 0; n < NV1; ++n) qs[h].load(n, load16(qh + (li1 * kFirst + n * kSecond) / VB * EPV * QB));
    }
  }
  __syncthreads();

  const uint64_t row_bytes = static_cast<uint64_t>(num_kv_heads) * D * EB;
  const int64_t lane_off = static_cast<int64_t>(g) * D * EB + li * VBV;
  const char* vbase = v_cache + lane_off;
  const int my_row = wave * TPW + grp;  // row of this lane within a load step

  // byte offset of logical row t0 + tl (rows of the pool fit in 32 bits)
  auto row_off = [&](int tl) -> uint64_t {
    const uint32_t pos = static_cast<uint32_t>(t0 + tl);
    const uint32_t blk = static_cast<uint32_t>(s_ids[(pos >> log2_bs) - jb0]);
    return static_cast<uint64_t>((blk << log2_bs) + (pos & bs_mask)) * row_bytes;
  };

  const int nloop = new_tl >= 0 ? ntok - 1 : ntok;  // rows read from the cache
  // the partition's row of position n - 1 (or -1), and the rows the value
  // pass takes in its loop: in row pairs that last row is added after the
  // loop in both the fused call and pa_decode
  const int last_tl = t1 == n ? ntok - 1 : -1;
  const int vloop = (kPairV && last_tl >= 0) ? ntok - 1 : nloop;

  // BT (block trips): the launch guarantees that every half-trip of rows
  // (128 or 256 rows, starting at a multiple of its length from the partition
  // start) lies inside one block: blocks of at least 256 rows, partitions a
  // multiple of 256. A half-trip's addresses are then that block's base, plus
  // a lane offset fixed for the whole kernel, plus a per-row step that is the
  // same for every lane, so it loads through a buffer resource on the block
  // (one block-id lookup) with the step in a scalar register, instead of a
  // block lookup and a 64-bit address per row and lane. A half-trip that
  // starts at or past the last cached row takes the block of that row (its
  // rows stay inside an allocated block and are never used); rows past the
  // last cached one inside a half-trip are loaded and never used.
  auto block_rsrc = [&](const char* head_base, int b0) -> __amdgpu_buffer_rsrc_t {
    const uint32_t pos = static_cast<uint32_t>(t0 + b0);
    const uint32_t last = static_cast<uint32_t>(t0 + nloop - 1);
    const uint32_t bi = min(pos >> log2_bs, last >> log2_bs) - static_cast<uint32_t>(jb0);
    const uint32_t blk = __builtin_amdgcn_readfirstlane(s_ids[bi]);
    const uint64_t row0 = (static_cast<uint64_t>(blk) << log2_bs) + (pos & bs_mask);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(head_base + row0 * row_bytes), 0, 0x7fffffff,
                                             kRawBufferFlags);
  };
  const uint32_t row_bytes32 = static_cast<uint32_t>(row_bytes);

  // the lane's NV1 K vectors of a row
  const char* kbase1 = k_cache + static_cast<int64_t>(g) * D * EB + li1 * kFirst;
  auto load_krow = [&](int tl, Vec (&k)[NV1]) {
    const char* r = kbase1 + row_off(tl);
    if constexpr (kPair) {
      const Vec16 both = load16_nt(r);
      k[0] = Vec{{both.w[0], both.w[1]}};
      k[1] = Vec{{both.w[2], both.w[3]}};
    } else {
#pragma unroll
      for (int n = 0; n < NV1; ++n) k[n] = E::load_nt(r + n * kSecond);
    }
  };
  // the row's G scores from the lane's partial dots, stored by one lane per
  // head set when `store`
  auto score_row = [&](const Vec (&k)[NV1], int tl, bool store) {
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = qs[h].template dot<BT && G == 8>(k);
    if constexpr (kScatter) {
      Scatter::reduce(sc);
      if (store && (li1 & ((1 << Scatter::TAIL) - 1)) == 0) {
        float* dst = s_score + tl * G + (li1 >> Scatter::TAIL) * Scatter::VF;
#pragma unroll
        for (int j = 0; j < Scatter::VF; ++j) dst[j] = sc[j];
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = group_sum<LPT1>(sc[h]);
      if (store && li1 == 0) store_scores<G>(s_score + tl * G, sc);
    }
  };

  // phase 1: raw scores q . k (the scale is applied once per score in phase 2).
  // Each trip's rows are taken in two halves with their loads in flight while
  // the other half is scored (software pipelining in the same registers): the
  // loads of the trip's second half are issued before its first half is
  // scored, and those of the next trip's first half before the second half
  // is. Rows past the partition load the partition's last cached row (every
  // load is unconditional, so the wait counts stay exact) and are not stored.
  const int my_row1 = wave * TPW1 + grp1;
  if (nloop > 0) {
    constexpr int H1 = kUnroll1 / 2;
    constexpr int TRIP1 = STEP1 * kUnroll1;
    Vec kv[2][H1][NV1];
    const char* khead = k_cache + static_cast<int64_t>(g) * D * EB;
    const uint32_t klane = static_cast<uint32_t>(my_row1) * row_bytes32 + static_cast<uint32_t>(li1 * kFirst);
    auto load_k = [&](int base, int half) {
      const int b0 = base + half * H1 * STEP1;
      if constexpr (BT) {
        const __amdgpu_buffer_rsrc_t r = block_rsrc(khead, b0);
#pragma unroll
        for (int u = 0; u < H1; ++u) {
          const uint32_t so = static_cast<uint32_t>(u * STEP1) * row_bytes32;
          if constexpr (kPair) {
            const Vec16 both = __builtin_bit_cast(Vec16, __builtin_amdgcn_raw_buffer_load_b128(r, klane, so, kLoadNt));
            kv[half][u][0] = Vec{{both.w[0], both.w[1]}};
            kv[half][u][1] = Vec{{both.w[2], both.w[3]}};
          } else if constexpr (kFp8) {
#pragma unroll
            for (int n = 0; n < NV1; ++n)
              kv[half][u][n] = __builtin_bit_cast(Vec, __builtin_amdgcn_raw_buffer_load_b64(r, klane, so + n * kSecond, kLoadNt));
          } else {
#pragma unroll
            for (int n = 0; n < NV1; ++n)
              kv[half][u][n] = __builtin_bit_cast(Vec, __builtin_amdgcn_raw_buffer_load_b128(r, klane, so + n * kSecond, kLoadNt));
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < H1; ++u) load_krow(min(b0 + u * STEP1 + my_row1, nloop - 1), kv[half][u]);
      }
    };
    auto score_k = [&](int base, int half) {
#pragma unroll
      for (int u = 0; u < H1; ++u) {
        const int tl = base + (half * H1 + u) * STEP1 + my_row1;
        score_row(kv[half][u], tl, tl < nloop);
      }
    };
    load_k(0, 0);
    for (int base = 0; base < nloop; base += TRIP1) {
      load_k(base, 1);
      score_k(base, 0);
      if (base + TRIP1 < nloop) load_k(base + TRIP1, 0);
      score_k(base, 1);
    }
  }
  if constexpr (FUSED) {
    if (new_tl >= 0) {  // uniform: every lane joins the row-group sums
      Vec nk[NV1];
#pragma unroll
      for (int n = 0; n < NV1; ++n) nk[n] = *reinterpret_cast<const Vec*>(s_new + li1 * kFirst + n * kSecond);
      score_row(nk, new_tl, my_row1 == new_tl % STEP1);
    }
  }
  // the value pass's loads (phase 3)
  constexpr int HV = kUnrollV / 2;
  constexpr int TRIPV = STEP * kUnrollV;
  VVec vv[2][HV];
  const char* vhead = v_cache + static_cast<int64_t>(g) * D * EB;
  const uint32_t vlane = static_cast<uint32_t>(my_row) * row_bytes32 + static_cast<uint32_t>(li * VBV);
  auto load_v = [&](int base, int half) {
    const int b0 = base + half * HV * STEP;
    if constexpr (BT) {
      const __amdgpu_buffer_rsrc_t r = block_rsrc(vhead, b0);
#pragma unroll
      for (int u = 0; u < HV; ++u) {
        const uint32_t so = static_cast<uint32_t>(u * STEP) * row_bytes32;
        if constexpr (sizeof(VVec) == 16) {
          vv[half][u] = __builtin_bit_cast(VVec, __builtin_amdgcn_raw_buffer_load_b128(r, vlane, so, kLoadNt));
        } else if constexpr (sizeof(VVec) == 8) {
          vv[half][u] = __builtin_bit_cast(VVec, __builtin_amdgcn_raw_buffer_load_b64(r, vlane, so, kLoadNt));
        } else {
          vv[half][u] = __builtin_bit_cast(VVec, __builtin_amdgcn_raw_buffer_load_b32(r, vlane, so, kLoadNt));
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < HV; ++u) vv[half][u] = load_vv(vbase + row_off(min(b0 + u * STEP + my_row, nloop - 1)));
    }
  };
  __syncthreads();

  // phase 2: exact max and sum of exp2(s - max) per head, in the log2 domain
  // (s = raw score * scale * log2 e; scale > 0 so the raw max is the max);
  // p overwrites the raw score. Thread tid owns head tid % G and every
  // (256 / G)-th token of it, so its loads are independent and several are
  // in flight at once; the per-head maxima and sums combine the threads of a
  // head (lanes of a wave with the same head differ in the lane bits at and
  // above G, then the waves through LDS).
  constexpr int kTph = kThreads / G;  // threads per head
  const int hh = tid % G;
  {
    float mt = -INFINITY;
    int t = tid / G;
    for (; t + 3 * kTph < ntok; t += 4 * kTph) {
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = s_score[(t + j * kTph) * G + hh];
      mt = fmaxf(mt, fmaxf(fmaxf(e[0], e[1]), fmaxf(e[2], e[3])));
    }
    for (; t < ntok; t += kTph) mt = fmaxf(mt, s_score[t * G + hh]);
#pragma unroll
    for (int off = G; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
    if (lane < G) s_wred[wave * G + lane] = mt;
  }
  __syncthreads();
  float m = s_wred[hh];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_wred[w * G + hh]);
  m *= scale_log2;
  float l = 0.f;
  {
    int t = tid / G;
    for (; t + 3 * kTph < ntok; t += 4 * kTph) {
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = s_score[(t + j * kTph) * G + hh];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = exp2f(fmaf(e[j], scale_log2, -m));
        s_score[(t + j * kTph) * G + hh] = e[j];
        l += e[j];
      }
    }
    for (; t < ntok; t += kTph) {
      const float e = exp2f(fmaf(s_score[t * G + hh], scale_log2, -m));
      s_score[t * G + hh] = e;
      l += e;
    }
  }
#pragma unroll
  for (int off = G; off < 64; off <<= 1) l += __shfl_xor(l, off, 64);
  __syncthreads();  // every wave has read the maxima: s_wred becomes the sums
  if (lane < G) s_wred[wave * G + lane] = l;
  if (tid < G) s_max[tid] = m;
  __syncthreads();
  if (tid < G) {
    float sum = s_wred[tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += s_wred[w * G + tid];
    s_sum[tid] = sum;
  }

  // phase 3: weighted sum of V rows
  float acc[G][EPVV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPVV; ++e) acc[h][e] = 0.f;
  // G >= 8: a lane's consecutive rows tl and tl + STEP in one v_dot2 per
  // element and head, with bf16 weights: (p(tl), p(tl + STEP)) . (v(tl),
  // v(tl + STEP)). The V pairs come from byte permutes (and, for E4M3 codes,
  // the exact widening to bf16); the weights are rounded to bf16 here.
  auto accum_pair = [&](const VVec& a, const VVec& b, int tl) {
    uint32_t vp[EPVV];
    if constexpr (kFp8) {
      const uint32_t w0 = __builtin_amdgcn_perm(b.w[0], a.w[0], 0x05010400u);
      const uint32_t w1 = __builtin_amdgcn_perm(b.w[0], a.w[0], 0x07030602u);
      vp[0] = e4m3x2_to_bf16x2<false>(w0);
      vp[1] = e4m3x2_to_bf16x2<true>(w0);
      vp[2] = e4m3x2_to_bf16x2<false>(w1);
      vp[3] = e4m3x2_to_bf16x2<true>(w1);
    } else {
#pragma unroll
      for (int w = 0; w < EPVV / 2; ++w) {
        vp[2 * w] = __builtin_amdgcn_perm(b.w[w], a.w[w], 0x05040100u);
        vp[2 * w + 1] = __builtin_amdgcn_perm(b.w[w], a.w[w], 0x07060302u);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bf16x2_t pp = {static_cast<__bf16>(s_score[tl * G + h]), static_cast<__bf16>(s_score[(tl + STEP) * G + h])};
      const uint32_t pw = __builtin_bit_cast(uint32_t, pp);
#pragma unroll
      for (int e = 0; e < EPVV; ++e) acc[h][e] = dot2_bf16(pw, vp[e], acc[h][e]);
    }
  };
  auto accum_row = [&](const VVec& v, int tl) {
    float vf[EPVV];
    vv_to_f32(v, vf);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = s_score[tl * G + h];
#pragma unroll
      for (int e = 0; e < EPVV; ++e) acc[h][e] = fmaf(w, vf[e], acc[h][e]);
    }
  };

  // the same two-half pipelining as the score pass; every lane still adds its
  // rows in increasing order
  if (nloop > 0) {
    auto accum_v = [&](int base, int half) {
      if constexpr (kPairV) {
#pragma unroll
        for (int u = 0; u < HV; u += 2) {
          const int tl = base + (half * HV + u) * STEP + my_row;
          if (tl + STEP < vloop) {
            accum_pair(vv[half][u], vv[half][u + 1], tl);
          } else if (tl < vloop) {
            accum_row(vv[half][u], tl);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < HV; ++u) {
          const int tl = base + (half * HV + u) * STEP + my_row;
          if (tl < nloop) accum_row(vv[half][u], tl);
        }
      }
    };
    load_v(0, 0);
    for (int base = 0; base < nloop; base += TRIPV) {
      load_v(base, 1);
      accum_v(base, 0);
      if (base + TRIPV < nloop) load_v(base + TRIPV, 0);
      accum_v(base, 1);
    }
  }
  if constexpr (kPairV) {
    // the sequence's last row is added last, alone, in both the fused call
    // (from LDS) and pa_decode (from the cache), so the two sum alike
    if (last_tl >= 0 && my_row == last_tl % STEP) {
      VVec lv;
      if (FUSED && new_tl >= 0) {
        lv = *reinterpret_cast<const VVec*>(s_new + row_bytes_h + li * VBV);
      } else {
        lv = load_vv(vbase + row_off(last_tl));
      }
      accum_row(lv, last_tl);
    }
  } else if constexpr (FUSED) {
    // the new row is this lane's last row, so it is added last, as in pa_decode
    if (new_tl >= 0 && my_row == new_tl % STEP)
      accum_row(*reinterpret_cast<const VVec*>(s_new + row_bytes_h + li * VBV), new_tl);
  }

  // phase 4: reduce over the rows of a wave, then over waves in fixed order
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPVV; ++e) {
      float v = acc[h][e];
      if constexpr (LPT == 16) {
        v = sum_lanes_16_32(v);  // the rows of a wave: lanes l, l ^ 16, l ^ 32, l ^ 48
      } else if constexpr (LPT == 32) {
        v = sum_lanes_32(v);     // the rows of a wave: lanes l, l ^ 32
      } else {
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
      }
      acc[h][e] = v;
    }
  __syncthreads();  // all reads of p are done; the score area becomes the reduction area
  float* s_red = s_score;  // [kWaves][G][D]
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPVV; ++e) s_red[(wave * G + h) * D + li * EPVV + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i % D;
    float v = s_red[(0 * G + h) * D + d];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += s_red[(w * G + h) * D + d];
    if constexpr (kFp8) v *= v_scale;
    const int qh = g * G + h;
    if (single) {
      const float o = v / s_sum[h];
      const int64_t oi = (static_cast<int64_t>(b) * num_q_heads + qh) * D + d;
      if constexpr (QB == 2) {
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
// One workgroup of NT threads (64, or 256 for long tables) per (sequence,
// query head). M and L: each thread takes every NT-th partition, then the
// workgroup combines them. The weighted sum: D / 4 lanes cover a partial row
// with 16-byte loads, and the NT / (D / 4) lane groups take every
// group-count-th partition, in increasing order, four loads in flight; the
// groups' sums then combine in group order. Every order is fixed, so the
// result is reproducible.
template <typename T, int D, int NT>
__global__ void __launch_bounds__(NT) decode_reduce_kernel(
    void* __restrict__ out, const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ context_lens, int32_t max_ctx, int32_t num_q_heads,
    int32_t partition, int32_t num_partitions) {
  constexpr int LPR = D / 4;            // lanes per partial row
  constexpr int NG = NT / LPR;          // partition groups
  constexpr int NW = NT / 64;           // waves
  constexpr int kBatch = 4;
  __shared__ float s_wred[2 * NW];
  __shared__ float4 s_grp[NG][LPR];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = min(context_lens[b], max_ctx);  // as in the partition kernel
  const int np = (n + partition - 1) / partition;
  const int64_t slot0 = (static_cast<int64_t>(b) * num_q_heads + h) * num_partitions;
  const float* ml = ws_ml + slot0 * 2;
  const int grp = tid / LPR;
  const int c = tid % LPR;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (np > 0) {  // uniform
    float m = -INFINITY;
    for (int pp = tid; pp < np; pp += NT) m = fmaxf(m, ml[2 * pp]);
    m = wave_max(m);
    if (lane == 0) s_wred[wave] = m;
    __syncthreads();
    float M = s_wred[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_wred[w]);
    float l = 0.f;
    for (int pp = tid; pp < np; pp += NT) l += ml[2 * pp + 1] * exp2f(ml[2 * pp] - M);
    l = wave_sum(l);
    if (lane == 0) s_wred[NW + wave] = l;

    const float4* acc = reinterpret_cast<const float4*>(ws_acc + slot0 * D) + c;
    for (int p0 = grp; p0 < np; p0 += NG * kBatch) {
      float w[kBatch];
      float4 a[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int pp = p0 + u * NG;
        w[u] = pp < np ? exp2f(ml[2 * pp] - M) : 0.f;
        a[u] = pp < np ? acc[static_cast<int64_t>(pp) * LPR] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        o.x = fmaf(w[u], a[u].x, o.x);
        o.y = fmaf(w[u], a[u].y, o.y);
        o.z = fmaf(w[u], a[u].z, o.z);
        o.w = fmaf(w[u], a[u].w, o.w);
      }
    }
    s_grp[grp][c] = o;
    __syncthreads();
    if (grp == 0) {
      float L = s_wred[NW];
#pragma unroll
      for (int w = 1; w < NW; ++w) L += s_wred[NW + w];
#pragma unroll
      for (int k = 1; k < NG; ++k) {
        const float4 x = s_grp[k][c];
        o.x += x.x;
        o.y += x.y;
        o.z += x.z;
        o.w += x.w;
      }
      const float inv = 1.f / L;
      o.x *= inv;
      o.y *= inv;
      o.z *= inv;
      o.w *= inv;
    }
  }
  if (grp == 0) {
    const int64_t ob = (static_cast<int64_t>(b) * num_q_heads + h) * D + c * 4;
    if constexpr (Elem<T>::kQBytes == 2) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(o.x) | (f32_to_bf16_bits(o.y) << 16);
      pk.y = f32_to_bf16_bits(o.z) | (f32_to_bf16_bits(o.w) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + ob) = pk;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + ob) = o;
    }
  }
}

template <typename T, int D, int G, bool FUSED>
hipError_t launch_decode_typed(const DecodeArgs& a, hipStream_t stream) {
  // block trips (see the kernel): blocks of 256+ rows and partitions a
  // multiple of 256; measured worth it at G >= 8 (16-bit and fp8 caches)
  constexpr bool kBtKernels = G >= 8 && !std::is_same<T, float>::value;
  const bool bt = kBtKernels && a.block_size >= 256 && a.partition % 256 == 0;
  constexpr int QB = Elem<T>::kQBytes;
  int log2_bs = 0;
  while ((1 << log2_bs) < a.block_size) ++log2_bs;
  const int score_words = G * (a.partition > 4 * D ? a.partition : 4 * D);
  const int max_ids = a.partition / (a.block_size < a.partition ? a.block_size : a.partition) + 2;
  const int new_words = FUSED ? 2 * D * Elem<T>::kBytes / 4 : 0;  // the fused new row
  const size_t lds = static_cast<size_t>(new_words + score_words + (2 + kWaves) * G + max_ids) * 4;
  // an E4M3 cache holds K / k_scale: the score scale absorbs k_scale
  const float scale_log2 = a.scale * (Elem<T>::kBytes == 1 ? a.k_scale : 1.f) * kLog2e;
  const int64_t table_rows = static_cast<int64_t>(a.max_blocks) << log2_bs;
  const int32_t max_ctx = static_cast<int32_t>(table_rows < INT32_MAX ? table_rows : INT32_MAX);
  dim3 grid(a.num_partitions * a.num_kv_heads * a.num_seqs);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, stream, a.out, static_cast<const char*>(a.q),
                       a.q_stride * QB, static_cast<char*>(const_cast<void*>(a.k_cache)),
                       static_cast<char*>(const_cast<void*>(a.v_cache)), a.block_tables, a.max_blocks,
                       a.context_lens, max_ctx, a.num_q_heads, a.num_kv_heads, log2_bs, scale_log2, a.partition,
                       a.num_partitions, score_words, a.ws_acc, a.ws_ml, static_cast<const char*>(a.new_k),
                       a.new_k_stride * QB, static_cast<const char*>(a.new_v), a.new_v_stride * QB,
                       a.slot_mapping, a.k_scale, a.v_scale);
  };
  if constexpr (kBtKernels) {
    if (bt) {
      launch(decode_partition_kernel<T, D, G, FUSED, true>);
    } else {
      launch(decode_partition_kernel<T, D, G, FUSED, false>);
    }
  } else {
    launch(decode_partition_kernel<T, D, G, FUSED, false>);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_partitions == 1) return err;
  // a workgroup of 256 threads pays off once a head has many partials;
  // otherwise 64 (its barriers and LDS combine cost more than they save)
  if (a.num_partitions >= 64) {
    hipLaunchKernelGGL((decode_reduce_kernel<T, D, 256>), dim3(a.num_q_heads, a.num_seqs), dim3(256), 0,
                       stream, a.out, a.ws_acc, a.ws_ml, a.context_lens, max_ctx, a.num_q_heads,
                       a.partition, a.num_partitions);
  } else {
    hipLaunchKernelGGL((decode_reduce_kernel<T, D, 64>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0,
                       stream, a.out, a.ws_acc, a.ws_ml, a.context_lens, max_ctx, a.num_q_heads,
                       a.partition, a.num_partitions);
  }
  return hipGetLastError();
}

template <typename T, int D, bool FUSED>
hipError_t dispatch_group(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_decode_typed<T, D, 1, FUSED>(a, stream);
    case 2: return launch_decode_typed<T, D, 2, FUSED>(a, stream);
    case 4: return launch_decode_typed<T, D, 4, FUSED>(a, stream);
    case 8: return launch_decode_typed<T, D, 8, FUSED>(a, stream);
    case 16: return launch_decode_typed<T, D, 16, FUSED>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t dispatch_fused(const DecodeArgs& a, hipStream_t stream) {
  return a.slot_mapping != nullptr ? dispatch_group<T, D, true>(a, stream)
                                   : dispatch_group<T, D, false>(a, stream);
}

}  // namespace

int32_t decode_partition_tokens(int32_t requested, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t group, int32_t block_size, int32_t max_blocks,
                                int32_t elem_bytes) {
  if (requested > 0) return requested;
  const int64_t max_ctx = static_cast<int64_t>(max_blocks) * block_size;
  const int64_t heads = static_cast<int64_t>(num_seqs) * num_kv_heads;
  auto fits = [&](int64_t part) { return static_cast<int64_t>(group) * part <= 8192; };  // LDS scores
  auto wgs = [&](int64_t part) { return heads * ((max_ctx + part - 1) / part); };
  // stretch = tokens per byte relative to a 16-bit cache
  auto rule = [&](int64_t stretch) -> int64_t {
    // Short histories over a grid that already fills the chip: one pass, no
    // merge launch (its latency costs more than the parallelism it would buy).
    const int64_t one_pass = (max_ctx + 63) / 64 * 64;
    if (one_pass <= 1024 * stretch && fits(one_pass) && heads >= 512) return one_pass;
    // Longest partition (fewest partials to merge) that still gives the grid
    // enough workgroups to cover the chip several times when every sequence
    // is as long as its table allows.
    for (int64_t part : {1024, 512}) {
      part *= stretch;
      if (fits(part) && wgs(part) >= 8192) return part;
    }
    int64_t part = fits(256 * stretch) ? 256 * stretch : 256;
    // Small grids are latency-bound: cut the history finer, to about 512
    // workgroups, but not below 64 tokens.
    if (wgs(part) < 512) {
      const int64_t fine = (max_ctx * heads + 511) / 512;
      part = fine <= 64 ? 64 : (fine + 63) / 64 * 64;
      if (part > 256 * stretch) part = 256 * stretch;
    }
    return part;
  };
  const int64_t part16 = rule(1);
  const int64_t part = elem_bytes == 1 ? (rule(2) > part16 ? rule(2) : part16) : part16;
  return static_cast<int32_t>(part);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.kv) {
    case KvFormat::kBf16:
      return a.head_dim == 64 ? dispatch_fused<BF16Tag, 64>(a, stream)
                              : dispatch_fused<BF16Tag, 128>(a, stream);
    case KvFormat::kFp8E4m3:
      return a.head_dim == 64 ? dispatch_fused<Fp8Tag, 64>(a, stream)
                              : dispatch_fused<Fp8Tag, 128>(a, stream);
    case KvFormat::kF32:
      return a.head_dim == 64 ? dispatch_fused<float, 64>(a, stream)
                              : dispatch_fused<float, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

// Split-K workspace of pa_store_decode_noalloc, for callers that cannot
// allocate: a fixed device array, one copy per GPU, kept until the process
// ends. Host code never passes `scratch` itself to a kernel (on the host the
// name is a stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress, called once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace pa
