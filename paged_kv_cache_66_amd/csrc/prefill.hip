// Packed varlen causal prefill over a paged KV cache, on bf16 MFMA.
//
// What is computed ("Inference Engine Inside nano-vLLM", "Attention in
// nano-vLLM", flash_attn_varlen_func with k, v = k_cache, v_cache and the
// block table; "nano-vLLM Part 2 ...", sections 2.5 and 4.1): sequence i has
// Lq query rows packed at cu_seqlens_q[i] and Lk visible keys; query j sits
// at position Lk - Lq + j and attends to keys 0 .. Lk - Lq + j, all read
// through the sequence's block-table row.
//
// Design (CDNA4 / gfx950): FlashAttention-style tiling (the pages' note that
// the kernels tile Q, K and V through on-chip memory while the cache stays
// in HBM, "nano-vLLM Part 2 ...", section 1.2), written for 64-wide waves and
// the v_mfma_f32_16x16x32_bf16 matrix instruction:
// * a workgroup owns 128 (query head, query) rows of one kv head: the G
//   query heads that share the kv head are packed together, so every K/V
//   tile staged in LDS serves 128 rows whatever G is;
// * per 64-key tile the scores are formed transposed, S^T = K Q^T (K rows
//   from LDS as the A operand, Q slices held in registers as the B operand),
//   so each lane ends up with four consecutive keys of one query column;
//   softmax statistics then need only two cross-lane steps per column;
// * O^T = V^T P^T: the B operand P^T is assembled in registers straight from
//   the score accumulators (the contraction index is permuted identically on
//   both operands); V stays in LDS in its natural [key][d] layout and the A
//   operand V^T comes from two transposing LDS reads (ds_read_b64_tr_b16:
//   each lane receives one head_dim column over four consecutive keys);
// * online softmax in the log2 domain: the running max is taken on raw
//   scores and the scale is folded into the one FMA that feeds exp2; only the
//   tiles that cross the causal diagonal or the end of the keys are masked;
// * K/V tiles are double-buffered in LDS, with one barrier per tile. Two
//   kernels: bf16 tiles of whole rows (packed K/V, or blocks of at least one
//   tile) go from HBM straight into LDS (buffer loads with the LDS
//   destination), which leaves the registers to hold the next tile's scores
//   beside the current softmax, and each wave interleaves its MFMAs with the
//   softmax by hand (prefill_direct_kernel, below); E4M3 caches and blocks
//   shorter than a tile stage the rows in registers (prefill_kernel): the
//   next tile's rows travel from HBM into registers while the current tile
//   is multiplied. Tiles that lie wholly inside the keys (all but the last)
//   are fetched without per-row bounds checks.
// * E4M3 caches (FP8): tiles travel as one-byte codes and are widened to bf16
//   (exactly) on their way into LDS; k_scale joins the softmax scale and
//   v_scale the final normalisation.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWavesPerGroup = 4;
constexpr int kThreads = 64 * kWavesPerGroup;
constexpr int kRows = 32 * kWavesPerGroup;  // (head, query) rows per workgroup: 32 per wave
constexpr int kKeys = 64;   // keys per tile
constexpr int kXcds = 8;    // accelerator complex dies of an MI355X

__device__ __forceinline__ bf16x8_t as_bf16x8(const Vec16& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// 2^x on the hardware exp unit (v_exp_f32). Arguments here are <= 0;
// results below the normal range flush to zero, which softmax weights
// tolerate (they are summed against weights of order one).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values to packed bf16 (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // (1.0, 1.0) in bf16

// Headroom of the running softmax max, in log2 units: tile weights may reach
// 2^kMaxSlack before the max is moved.
constexpr float kMaxSlack = 8.f;

// Fourth word of a raw buffer resource on gfx9-family parts (untyped 32-bit
// data format); the offsets used are far below the record limit.
constexpr int kBufferFlags = 0x00020000;

// max of three floats in one v_max3_f32. Written as assembly because the
// compiler, unable to prove MFMA results are canonical floats, otherwise
// precedes every max with a canonicalising v_max(x, x); score tiles never hold
// NaN (masked keys are -inf).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes that hold
// the same MFMA column), with the cross-row swaps v_permlane16_swap and
// v_permlane32_swap: each returns the value and its partner's, in some order.
__device__ __forceinline__ float col_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2f(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// a.x * b.x + a.y * b.y + c for packed bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes i / 4 + 4k (k = 0..3). With
// lane m addressing row m / 4, columns 4 (m % 4) .. + 3 of a [row][col] tile,
// lane i gets column i of rows 0..3.
__device__ __forceinline__ s16x4_t ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_s16x4_t*>(reinterpret_cast<uintptr_t>(p)));
}

// Online softmax over one 64-key tile of S^T for this wave's 32 (head,
// query) columns, in the log2 domain: masks the keys a column may not see
// (only on tiles that cross the causal diagonal or the end of the keys),
// moves the running max m when a column's max outgrows it by more than
// kMaxSlack (the O rows and the sum l are rescaled on those tiles only),
// and leaves the weights as the bf16 P^T operand in pop[k-step][t], with l
// summed from those same bf16 weights (what the PV product sees).
template <int DT>
__device__ __forceinline__ void softmax_max(f32x4_t (&s)[4][2], bool need_mask, const int (&posq)[2],
                                            int Lk, int kt0, int gq, float scale_log2, float (&m)[2],
                                            float (&l)[2], f32x4_t (&o)[DT][2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (need_mask) {
      // key kt0 + kt*16 + gq*4 + e is visible to this column iff it is at
      // most lim (the query's position, capped by the last key)
      const int lim = min(posq[t], Lk - 1) - (kt0 + gq * 4);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[kt][t][e] = (kt * 16 + e <= lim) ? s[kt][t][e] : -INFINITY;
    }
    // raw-score max (scale > 0 keeps the order); masked keys are -inf
    float tmax = max3f(s[0][t][0], s[0][t][1], s[0][t][2]);
    tmax = max3f(tmax, s[0][t][3], s[1][t][0]);
    tmax = max3f(tmax, s[1][t][1], s[1][t][2]);
    tmax = max3f(tmax, s[1][t][3], s[2][t][0]);
    tmax = max3f(tmax, s[2][t][1], s[2][t][2]);
    tmax = max3f(tmax, s[2][t][3], s[3][t][0]);
    tmax = max3f(tmax, s[3][t][1], s[3][t][2]);
    tmax = max2f(tmax, s[3][t][3]);
    tmax = col_max(tmax);
    // The reference max moves only when some column's max exceeds it by more
    // than kMaxSlack (log2 units); otherwise the tile's weights are taken
    // against the old max and stay below 2^kMaxSlack. Softmax does not
    // depend on that reference, and fp32 sums and bf16 weights have the range
    // for it, so O and l are rescaled on the few tiles that move it.
    const float m_cand = tmax * scale_log2;
    if (__any(m_cand > m[t] + kMaxSlack)) {
      const float m_new = max2f(m[t], m_cand);
      const float alpha = fast_exp2(m[t] - m_new);
      l[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][t] *= alpha;
      m[t] = m_new;
    }
  }
}

// Weights of a tile whose running max is already in m: exp2, bf16 P^T
// operand, and the row sums.
__device__ __forceinline__ void softmax_exp(f32x4_t (&s)[4][2], float scale_log2, const float (&m)[2],
                                            float (&l)[2], Vec16 (&pop)[2][2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[kt][t][e] = fast_exp2(fmaf(s[kt][t][e], scale_log2, -m[t]));
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      pop[st][t].w[0] = pack2(s[2 * st][t][0], s[2 * st][t][1]);
      pop[st][t].w[1] = pack2(s[2 * st][t][2], s[2 * st][t][3]);
      pop[st][t].w[2] = pack2(s[2 * st + 1][t][0], s[2 * st + 1][t][1]);
      pop[st][t].w[3] = pack2(s[2 * st + 1][t][2], s[2 * st + 1][t][3]);
    }
    // two weights at a time with v_dot2 against (1, 1)
    float lsum = l[t];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int w = 0; w < 4; ++w) lsum = dot2_bf16(pop[st][t].w[w], kOnesBf16x2, lsum);
    l[t] = lsum;
  }
}

// Online softmax over one 64-key tile of S^T for this wave's 32 (head,
// query) columns, in the log2 domain: masks the keys a column may not see
// (only on tiles that cross the causal diagonal or the end of the keys),
// moves the running max m when a column's max outgrows it by more than
// kMaxSlack (the O rows and the sum l are rescaled on those tiles only),
// and leaves the weights as the bf16 P^T operand in pop[k-step][t], with l
// summed from those same bf16 weights (what the PV product sees).
template <int DT>
__device__ __forceinline__ void softmax_tile(f32x4_t (&s)[4][2], bool need_mask, const int (&posq)[2],
                                             int Lk, int kt0, int gq, float scale_log2, float (&m)[2],
                                             float (&l)[2], f32x4_t (&o)[DT][2], Vec16 (&pop)[2][2]) {
  softmax_max<DT>(s, need_mask, posq, Lk, kt0, gq, scale_log2, m, l, o);
  softmax_exp(s, scale_log2, m, l, pop);
}

// Normalised bf16 output of this wave's two 16-column groups.
template <int D>
__device__ __forceinline__ void write_out(uint16_t* out, const f32x4_t (&o)[D / 16][2], const float (&l)[2],
                                          const int (&orow)[2], const int (&ohead)[2], int num_q_heads,
                                          int gq, float v_scale) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float lt = col_sum(l[t]);
    if (orow[t] < 0) continue;
    const float inv = v_scale / lt;
    uint16_t* orow_ptr = out + (static_cast<int64_t>(orow[t]) * num_q_heads + ohead[t]) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      uint2 w;
      w.x = pack2(o[dt][t][0] * inv, o[dt][t][1] * inv);
      w.y = pack2(o[dt][t][2] * inv, o[dt][t][3] * inv);
      *reinterpret_cast<uint2*>(orow_ptr + dt * 16 + gq * 4) = w;
    }
  }
}

// Workgroup -> (sequence i, kv head g, query tile x). Workgroups are handed
// to the 8 XCDs round-robin by linear id, and each XCD has its own L2: every
// kv head goes to one XCD (g % 8 == id % 8) and the query tiles of a
// (sequence, kv head) sit next to each other, so the tiles that stream the
// same K/V rows share an L2.
__device__ __forceinline__ void tile_of_workgroup(int L, int num_kv_heads, int max_qt, int& i, int& g,
                                                  int& x) {
  if (num_kv_heads % kXcds == 0) {
    const int xcd = L % kXcds;
    const int r = L / kXcds;
    const int heads_per_xcd = num_kv_heads / kXcds;
    x = r % max_qt;
    const int r2 = r / max_qt;
    g = (r2 % heads_per_xcd) * kXcds + xcd;
    i = r2 / heads_per_xcd;
  } else {
    x = L % max_qt;
    const int r = L / max_qt;
    g = r % num_kv_heads;
    i = r / num_kv_heads;
  }
}

// Q operands (B of S^T = K Q^T) of this wave's two 16-column groups: column
// r of the workgroup's 128 is query head g * G + r / QT at query q_lo + r % QT
// (heads of the group packed together), with its absolute position and its
// output row (-1 for padding columns past the chunk).
// Keys a sequence's attention reads: Lk, cut in paged mode to the rows its
// block-table row can name (max_blocks << log2_bs), so no tile walks past the
// row whatever cu_seqlens_k says.
__device__ __forceinline__ int clamp_keys(int lk, bool paged, int max_blocks, int log2_bs) {
  const int64_t rows = static_cast<int64_t>(max_blocks) << log2_bs;
  return paged && lk > rows ? static_cast<int>(rows) : lk;
}

template <int D, int G>
__device__ __forceinline__ void load_q(const char* q, int64_t q_stride_bytes, int q0, int Lq, int q_lo,
                                       int start, int g, int wave, int col, int gq,
                                       bf16x8_t (&qop)[2][D / 32], int (&posq)[2], int (&orow)[2],
                                       int (&ohead)[2]) {
  constexpr int QT = kRows / G;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = wave * 32 + t * 16 + col;
    const int hl = r / QT;
    const int ql = r % QT;
    const int qi = q_lo + ql;
    const int head = g * G + hl;
    posq[t] = start + qi;
    orow[t] = qi < Lq ? q0 + qi : -1;
    ohead[t] = head;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      Vec16 v{{0u, 0u, 0u, 0u}};
      if (qi < Lq) {
        v = load16(q + static_cast<int64_t>(q0 + qi) * q_stride_bytes +
                   (static_cast<int64_t>(head) * D + ks * 32 + gq * 8) * 2);
      }
      qop[t][ks] = as_bf16x8(v);
    }
  }
}

// Eight key / value elements as the tile loads carry them (bf16, or E4M3
// codes) and their bf16 form for LDS.
template <bool FP8> struct TileVec;
template <> struct TileVec<false> {
  using Vec = Vec16;
  __device__ __forceinline__ static Vec load(const char* p) { return load16(p); }
  // a tile row chunk at a 32-bit offset from a uniform base: buffer load with
  // the base in scalar registers, so no 64-bit address arithmetic per lane
  __device__ __forceinline__ static Vec load(__amdgpu_buffer_rsrc_t base, uint32_t off) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(base, off, 0, 0);
    return Vec16{{v.x, v.y, v.z, v.w}};
  }
  __device__ __forceinline__ static Vec16 to_bf16(const Vec& v) { return v; }
};
template <> struct TileVec<true> {
  using Vec = Vec8;
  __device__ __forceinline__ static Vec load(const char* p) { return load8(p); }
  __device__ __forceinline__ static Vec load(__amdgpu_buffer_rsrc_t base, uint32_t off) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(base, off, 0, 0);
    return Vec8{{v.x, v.y}};
  }
  __device__ __forceinline__ static Vec16 to_bf16(const Vec& v) {
    return Vec16{{e4m3x2_to_bf16x2<false>(v.w[0]), e4m3x2_to_bf16x2<true>(v.w[0]),
                  e4m3x2_to_bf16x2<false>(v.w[1]), e4m3x2_to_bf16x2<true>(v.w[1])}};
  }
};

// Fused store (bf16 caches): the query rows of this workgroup are this
// step's new tokens. Their K and V rows of kv head g (16-byte chunks of the
// packed rows of new_k / new_v) go to the cache slots slot_mapping[row]; slot
// -1 stores nothing. Every (row, kv head) pair belongs to exactly one
// workgroup.
template <int D>
__device__ __forceinline__ void store_new_rows(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                               int64_t cache_row_bytes, const char* __restrict__ new_k,
                                               const char* __restrict__ new_v, int64_t nk_stride_bytes,
                                               int64_t nv_stride_bytes, const int32_t* __restrict__ slot_mapping,
                                               int row0, int nrows, int g) {
  constexpr int CH = D / 8;  // 8-element chunks per head slice
  const int n = nrows * 2 * CH;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int c = idx % CH;
    const int rv = idx / CH;
    const bool is_v = rv & 1;
    const int r = row0 + (rv >> 1);
    const int slot = slot_mapping[r];
    if (slot < 0) continue;
    const Vec16 x = load16((is_v ? new_v + r * nv_stride_bytes : new_k + r * nk_stride_bytes) +
                           (static_cast<int64_t>(g) * D + c * 8) * 2);
    store16((is_v ? v_cache : k_cache) + static_cast<int64_t>(slot) * cache_row_bytes +
                (static_cast<int64_t>(g) * D + c * 8) * 2,
            x);
  }
}

template <int D, int G, bool FP8, bool FUSED>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(
    uint16_t* __restrict__ out, const char* __restrict__ q, int64_t q_stride_bytes,
    const char* __restrict__ k_cache, const char* __restrict__ v_cache, int64_t k_stride_bytes,
    int64_t v_stride_bytes, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ block_tables, int32_t max_blocks, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t log2_bs, float scale_log2, int32_t max_qt, float v_scale,
    const char* __restrict__ new_k, const char* __restrict__ new_v, int64_t nk_stride_bytes,
    int64_t nv_stride_bytes, const int32_t* __restrict__ slot_mapping) {
  static_assert(!(FUSED && FP8), "E4M3 caches take the scatter as a launch of its own");
  using TV = TileVec<FP8>;
  using KVec = typename TV::Vec;
  constexpr int KB = FP8 ? 1 : 2;  // bytes per cache element
  constexpr int CB = 8 * KB;       // bytes per 8-element chunk
  constexpr int QT = kRows / G;    // queries per workgroup
  constexpr int KS = D / 32;       // MFMA k-steps over head_dim
  constexpr int DT = D / 16;       // 16-wide head_dim tiles of the output
  constexpr int KPITCH = D + 8;    // bf16 per K row in LDS (padding spreads banks)
  // bf16 per V row in LDS: a 16-element shift of the banks per row keeps the
  // transposing reads (four rows of 32 bytes per 16 lanes) conflict-free
  constexpr int VPITCH = D + 16;
  constexpr int KCH = D / 8;       // 8-element chunks per K / V row
  constexpr int KLOADS = kKeys * KCH / kThreads;  // K (and V) chunks per thread per tile

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKeys * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kKeys * VPITCH];

  int i, g, x;
  tile_of_workgroup(blockIdx.x, num_kv_heads, max_qt, i, g, x);
  const int q0 = cu_q[i];
  const int Lq = cu_q[i + 1] - q0;
  // paged keys never run past the sequence's table row
  const int Lk = clamp_keys(cu_k[i + 1] - cu_k[i], block_tables != nullptr, max_blocks, log2_bs);
  const int n_qt = (Lq + QT - 1) / QT;
  if (x >= n_qt) return;
  const int qt = n_qt - 1 - x;  // heaviest tiles first
  const int q_lo = qt * QT;
  const int q_hi = min(q_lo + QT, Lq);
  const int start = Lk - Lq;
  const int kmax = min(Lk, start + q_hi);
  const int nkt = (kmax + kKeys - 1) / kKeys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;  // MFMA column / row-in-operand index
  const int gq = lane >> 4;   // MFMA lane group

  // ---- Q operands (B of S^T = K Q^T), positions and output rows ----
  bf16x8_t qop[2][KS];
  int posq[2];
  int orow[2];   // packed query row, -1 when this column is padding
  int ohead[2];
  load_q<D, G>(q, q_stride_bytes, q0, Lq, q_lo, start, g, wave, col, gq, qop, posq, orow, ohead);

  // Key rows come either from the paged caches (row stride H_kv * D) through
  // the block table, or, without a table, from packed k / v tensors where key
  // t of sequence i is row cu_k[i] + t (row strides given by the caller).
  const bool paged = block_tables != nullptr;
  const int64_t head_off = static_cast<int64_t>(g) * D * KB;
  const int32_t* table = paged ? block_tables + static_cast<int64_t>(i) * max_blocks : nullptr;
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t k0_row = paged ? 0 : cu_k[i];

  // Byte offset of key row `key` in the paged caches (kv head slice included).
  // With blocks of at least one tile (64 keys) a tile lies inside one block,
  // so its block id is read once per tile; smaller blocks look up every row.
  // Packed rows are always contiguous.
  const bool tile_contiguous = !paged || log2_bs >= 6;
  auto row_addr = [&](int key) -> int64_t {
    const int64_t blk = table[key >> log2_bs];
    return ((blk << log2_bs) + (key & bs_mask)) * k_stride_bytes + head_off;
  };

  // ---- tile fetch into registers ----
  // Thread tid carries chunks tid + u * kThreads of the tile (row item / KCH,
  // chunk item % KCH) for K and for V alike.
  KVec kreg[KLOADS];
  KVec vreg[KLOADS];
  // Byte offsets of this thread's K and V chunks inside a contiguous tile
  // (rows x row stride + chunk: under 2^31 for any supported shape); fixed for
  // the whole kernel, so a tile fetch adds one uniform base.
  uint32_t koff[KLOADS];
  uint32_t voff[KLOADS];
#pragma unroll
  for (int u = 0; u < KLOADS; ++u) {
    const int item = tid + u * kThreads;
    koff[u] = static_cast<uint32_t>((item / KCH) * k_stride_bytes + (item % KCH) * CB);
    voff[u] = static_cast<uint32_t>((item / KCH) * v_stride_bytes + (item % KCH) * CB);
  }

  auto fetch = [&](int kt0) {
    if constexpr (FUSED) {
      // keys at or after `start` are this step's rows: read them from new_k
      // / new_v, never from the caches
      if (kt0 + kKeys > start) {
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
          const int item = tid + u * kThreads;
          const int key = kt0 + item / KCH;
          const int c = item % KCH;
          if (key >= Lk) {
            kreg[u] = KVec{};
            vreg[u] = KVec{};
          } else if (key < start) {
            const int64_t ra = row_addr(key) + c * CB;
            kreg[u] = TV::load(k_cache + ra);
            vreg[u] = TV::load(v_cache + ra);
          } else {
            const int64_t r = q0 + key - start;
            const int64_t ho = (static_cast<int64_t>(g) * D + c * 8) * 2;
            kreg[u] = load16(new_k + r * nk_stride_bytes + ho);
            vreg[u] = load16(new_v + r * nv_stride_bytes + ho);
          }
        }
        return;
      }
    }
    if (tile_contiguous) {
      // kt0 < Lk always, so the tile's first row exists
      const char* kb = paged ? k_cache + row_addr(kt0) : k_cache + (k0_row + kt0) * k_stride_bytes + head_off;
      const char* vb = paged ? v_cache + row_addr(kt0) : v_cache + (k0_row + kt0) * v_stride_bytes + head_off;
      if (kt0 + kKeys <= Lk) {
        // a full tile: no row can be past the keys
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb), 0, 0x7fffffff, kBufferFlags);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vb), 0, 0x7fffffff, kBufferFlags);
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
          kreg[u] = TV::load(kr, koff[u]);
          vreg[u] = TV::load(vr, voff[u]);
        }
        return;
      }
#pragma unroll
      for (int u = 0; u < KLOADS; ++u) {
        const int key = kt0 + (tid + u * kThreads) / KCH;
        kreg[u] = key < Lk ? TV::load(kb + koff[u]) : KVec{};
        vreg[u] = key < Lk ? TV::load(vb + voff[u]) : KVec{};
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int item = tid + u * kThreads;
      const int key = kt0 + item / KCH;
      const int64_t ra = key < Lk ? row_addr(key) + (item % KCH) * CB : 0;
      kreg[u] = key < Lk ? TV::load(k_cache + ra) : KVec{};
      vreg[u] = key < Lk ? TV::load(v_cache + ra) : KVec{};
    }
  };
  // K and V rows keep their natural [key][d] layout in LDS
  auto commit = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
      const int item = tid + u * kThreads;
      const int r = item / KCH;
      const int c = item % KCH;
      *reinterpret_cast<Vec16*>(&sK[buf][r * KPITCH + c * 8]) = TV::to_bf16(kreg[u]);
      *reinterpret_cast<Vec16*>(&sV[buf][r * VPITCH + c * 8]) = TV::to_bf16(vreg[u]);
    }
  };

  f32x4_t o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t) o[dt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};

  // Tile j is multiplied from LDS buffer j % 2 while tile j + 1 travels from
  // HBM into registers; it is written to the other buffer after the softmax,
  // and a single barrier per tile separates the writes from the next reads.
  fetch(0);
  commit(0);
  __syncthreads();
  for (int j = 0; j < nkt; ++j) {
    const int kt0 = j * kKeys;
    const int buf = j & 1;
    if (j + 1 < nkt) fetch(kt0 + kKeys);

    // S^T tile: 64 keys x 32 (head, query) columns per wave
    f32x4_t s[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[kt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const Vec16 kv = *reinterpret_cast<const Vec16*>(&sK[buf][(kt * 16 + col) * KPITCH + ks * 32 + gq * 8]);
        const bf16x8_t ka = as_bf16x8(kv);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          s[kt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop[t][ks], s[kt][t], 0, 0, 0);
      }
    }

    const bool need_mask = !(kt0 + kKeys - 1 <= start + q_lo && kt0 + kKeys <= Lk);
    Vec16 pop[2][2];  // [k-step of 32 keys][t]: P^T operand, 8 bf16
    softmax_tile<DT>(s, need_mask, posq, Lk, kt0, gq, scale_log2, m, l, o, pop);
    // the next tile goes to the other buffer (free since the last barrier)
    // here, between the softmax and P V, rather than in a burst before the
    // barrier
    if (j + 1 < nkt) commit(buf ^ 1);

    // O^T += V^T P^T
    // A operand of lane (gq, col): V[key][dt * 16 + col] for the keys
    // st * 32 + gq * 4 + 0..3 and st * 32 + 16 + gq * 4 + 0..3, the order in
    // which the P^T operand holds them
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint16_t* vsrc = &sV[buf][(st * 32 + gq * 4 + (col >> 2)) * VPITCH + dt * 16 + 4 * (col & 3)];
        const s16x4_t lo = ds_read_tr16(vsrc);
        const s16x4_t hi = ds_read_tr16(vsrc + 16 * VPITCH);
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          o[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(pop[st][t]), o[dt][t], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  write_out<D>(out, o, l, orow, ohead, num_q_heads, gq, FP8 ? v_scale : 1.f);
  // the caches' copy of this workgroup's rows is read by no workgroup of
  // this launch, so the scatter goes last, behind the attention
  if constexpr (FUSED)
    store_new_rows<D>(const_cast<char*>(k_cache), const_cast<char*>(v_cache), k_stride_bytes, new_k, new_v,
                      nk_stride_bytes, nv_stride_bytes, slot_mapping, q0 + q_lo, q_hi - q_lo, g);
}

// ---------------------------------------------------------------------------
// bf16 caches, tiles of whole rows (packed K/V, or blocks of >= 64 keys):
// K and V tiles travel from HBM straight into LDS (buffer loads with the LDS
// destination), unpadded, with the 16-byte chunks of each row permuted by
// chunk_swz so that the MFMA operand reads hit distinct banks. No tile passes
// through registers, so the scores of the next tile fit beside the current
// one, and each wave interleaves its matrix and vector work by hand:
// iteration j forms S(j+1) = K(j+1) Q^T with three softmax instructions of
// tile j (exp2, packing, row sums) after every MFMA, then adds P(j) V(j) with
// the pieces of tile j+1's max between the MFMAs; the loads of K(j+2) and
// V(j+1) are issued at its start and have the whole iteration to land.
// ---------------------------------------------------------------------------

// position of 16-byte chunk c of tile row r: c ^ kSwz(r) (conflict-free for
// the 16-row K operand reads and the 4-row transposing V reads)
template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (D == 128) {
    return ((r & 7) << 1) | ((r >> 3) & 1);
  } else {
    return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;

template <int D, int G, bool FUSED>
__global__ void __launch_bounds__(kThreads, 2) prefill_direct_kernel(
    uint16_t* __restrict__ out, const char* __restrict__ q, int64_t q_stride_bytes,
    const char* __restrict__ k_cache, const char* __restrict__ v_cache, int64_t k_stride_bytes,
    int64_t v_stride_bytes, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ block_tables, int32_t max_blocks, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t log2_bs, float scale_log2, int32_t max_qt,
    const char* __restrict__ new_k, const char* __restrict__ new_v, int64_t nk_stride_bytes,
    int64_t nv_stride_bytes, const int32_t* __restrict__ slot_mapping) {
  constexpr int QT = kRows / G;      // queries per workgroup
  constexpr int KS = D / 32;         // MFMA k-steps over head_dim
  constexpr int DT = D / 16;         // 16-wide head_dim tiles of the output
  constexpr int ROWB = D * 2;        // bytes per tile row
  constexpr int NCH = ROWB / 16;     // 16-byte chunks per row
  constexpr int LOADS = kKeys * ROWB / (kThreads * 16);  // 1 KiB wave loads per wave and tile
  constexpr int ROWS_PER_LOAD = 1024 / ROWB;

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKeys * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kKeys * D];

  int i, g, x;
  tile_of_workgroup(blockIdx.x, num_kv_heads, max_qt, i, g, x);
  const int q0 = cu_q[i];
  const int Lq = cu_q[i + 1] - q0;
  // paged keys never run past the sequence's table row
  const int Lk = clamp_keys(cu_k[i + 1] - cu_k[i], block_tables != nullptr, max_blocks, log2_bs);
  const int n_qt = (Lq + QT - 1) / QT;
  if (x >= n_qt) return;
  const int qt = n_qt - 1 - x;  // heaviest tiles first
  const int q_lo = qt * QT;
  const int q_hi = min(q_lo + QT, Lq);
  const int start = Lk - Lq;
  const int kmax = min(Lk, start + q_hi);
  const int nkt = (kmax + kKeys - 1) / kKeys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;  // MFMA column / row-in-operand index
  const int gq = lane >> 4;   // MFMA lane group

  bf16x8_t qop[2][KS];
  int posq[2];
  int orow[2];
  int ohead[2];
  load_q<D, G>(q, q_stride_bytes, q0, Lq, q_lo, start, g, wave, col, gq, qop, posq, orow, ohead);

  // Tile row r of key kt0 + r: paged rows of one block (block size >= 64, so
  // a tile never straddles blocks), or packed rows cu_k[i] + kt0 + r.
  const bool paged = block_tables != nullptr;
  const int64_t head_off = static_cast<int64_t>(g) * ROWB;
  const int32_t* table = paged ? block_tables + static_cast<int64_t>(i) * max_blocks : nullptr;
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t k0_row = paged ? 0 : cu_k[i];
  // The K (which = 0) and V (which = 1) tile streams each remember the last
  // block they looked up, so a tile in the same block as its stream's
  // previous tile needs no table read (three of every four tiles at a block
  // size of 256: chunked prefill ~1.4 % faster).
  int cached_bi[2] = {-1, -1};
  int32_t cached_blk[2] = {0, 0};
  auto tile_row0 = [&](int kt0, int which) -> int64_t {  // row index of key kt0 in the K / V tensors
    if (paged) {
      const int bi = kt0 >> log2_bs;
      if (bi != cached_bi[which]) {
        // the block id is uniform: read it through the scalar cache (the
        // compiler would make it a vector load behind the LDS-bound loads and
        // wait for those)
        const int32_t* e = table + bi;
        int32_t blk;
        asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(blk) : "s"(e) : "memory");
        cached_bi[which] = bi;
        cached_blk[which] = blk;
      }
      return (static_cast<int64_t>(cached_blk[which]) << log2_bs) + (kt0 & bs_mask);
    }
    return k0_row + kt0;
  };

  // This lane's part of wave load j: LDS bytes [(wave * LOADS + j) KiB +
  // lane * 16, + 16) = tile row r, chunk position p, filled from chunk
  // p ^ kSwz(r) of the row.
  int lrow[LOADS];
  uint32_t kload[LOADS], vload[LOADS];  // byte offsets inside a tile of whole rows
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int o = (wave * LOADS + j) * 1024 + lane * 16;
    lrow[j] = o / ROWB;
    const int p = (o % ROWB) / 16;
    const uint32_t c = static_cast<uint32_t>(((p ^ chunk_swz<D>(lrow[j])) % NCH) * 16);
    kload[j] = static_cast<uint32_t>(lrow[j] * k_stride_bytes) + c;
    vload[j] = static_cast<uint32_t>(lrow[j] * v_stride_bytes) + c;
  }
  // The loads are written as inline assembly on purpose: the compiler would
  // otherwise track the LDS they fill and wait for them before every LDS
  // read of the other buffer. Their completion is awaited explicitly
  // (s_waitcnt, then a barrier) before any wave reads what they filled.
  // LDS byte address of this wave's first 1 KiB in each buffer (uniform)
  auto wave_lds = [&](uint16_t* buf) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf + wave * LOADS * 512)));
  };
  const uint32_t lds_k[2] = {wave_lds(sK[0]), wave_lds(sK[1])};
  const uint32_t lds_v[2] = {wave_lds(sV[0]), wave_lds(sV[1])};
  auto issue = [&](const char* base, int64_t stride, const uint32_t (&off)[LOADS], uint32_t lds, int kt0, int which) {
    const uint64_t tile = reinterpret_cast<uint64_t>(base + tile_row0(kt0, which) * stride + head_off);
    u32x4_t rs;  // raw buffer resource: base, no stride, 2^31 - 1 bytes
    rs.x = static_cast<uint32_t>(tile);
    rs.y = static_cast<uint32_t>(tile >> 32) & 0xffffu;
    rs.z = 0x7fffffffu;
    rs.w = static_cast<uint32_t>(kBufferFlags);
    if (kt0 + kKeys <= Lk) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(off[j]), "s"(rs), "s"(lds + j * 1024)
                     : "memory");
      return;
    }
    // last tile: rows past the keys read the last key's row instead (its
    // scores are masked and its weights are 0, and it is finite)
    const int rmax = Lk - 1 - kt0;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const uint32_t o = lrow[j] <= rmax ? off[j] : off[j] - static_cast<uint32_t>((lrow[j] - rmax) * stride);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(o), "s"(rs), "s"(lds + j * 1024)
                   : "memory");
    }
  };
  // K (is_v false) or V tile at kt0 into LDS. Fused store: keys at or after
  // `start` are this step's rows, read from new_k / new_v (the caches' copy
  // is written by this launch). A tile wholly past `start` is one buffer load
  // per lane as from the caches, with the new rows' stride; the one tile that
  // holds `start` mixes sources and takes one global address per lane
  // (global_load_lds_dwordx4), cache rows before `start`, new rows after.
  auto issue_tile = [&](bool is_v, uint32_t lds, int kt0) {
    const char* cache = is_v ? v_cache : k_cache;
    const int64_t stride = is_v ? v_stride_bytes : k_stride_bytes;
    const uint32_t(&off)[LOADS] = is_v ? vload : kload;
    if (!FUSED || kt0 + kKeys <= start) {
      issue(cache, stride, off, lds, kt0, is_v ? 1 : 0);
      return;
    }
    const char* nb = is_v ? new_v : new_k;
    const int64_t ns = is_v ? nv_stride_bytes : nk_stride_bytes;
    const int rmax = Lk - 1 - kt0;  // rows past the keys repeat the last key
    if (kt0 >= start) {
      const uint64_t tile = reinterpret_cast<uint64_t>(nb + (q0 + kt0 - start) * ns + head_off);
      u32x4_t rs;
      rs.x = static_cast<uint32_t>(tile);
      rs.y = static_cast<uint32_t>(tile >> 32) & 0xffffu;
      rs.z = 0x7fffffffu;
      rs.w = static_cast<uint32_t>(kBufferFlags);
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        // off[j] = lrow[j] * stride + chunk: swap the row part
        const uint32_t o = off[j] - static_cast<uint32_t>(lrow[j] * stride) +
                           static_cast<uint32_t>(min(lrow[j], rmax) * ns);
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(o), "s"(rs), "s"(lds + j * 1024)
                     : "memory");
      }
      return;
    }
    const int64_t crow0 = tile_row0(kt0, is_v ? 1 : 0);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int r = min(lrow[j], rmax);
      const uint32_t c = off[j] - static_cast<uint32_t>(lrow[j] * stride);
      const int t = kt0 + r;
      const char* src = t < start ? cache + (crow0 + r) * stride + head_off + c
                                  : nb + (q0 + t - start) * ns + head_off + c;
      const uint64_t a = reinterpret_cast<uint64_t>(src);
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(a), "s"(lds + j * 1024)
                   : "memory");
    }
  };

  // Loop-invariant LDS byte offsets of the operand reads. The swizzle of row
  // r depends on r % 16 only, so rows that differ by whole 16-row steps
  // (kt for K, st and the second half for V) reuse one offset plus an
  // immediate.
  //   K (A of S^T): lane (gq, col) reads row kt * 16 + col, chunk ks * 4 + gq
  //   V (tr reads): lane m of group gq addresses row kbase + gq * 4 + m / 4,
  //                 columns dt * 16 + 4 (m % 4) .. + 3
  uint32_t krd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    krd[ks] = static_cast<uint32_t>(col * ROWB + (((ks * 4 + gq) ^ chunk_swz<D>(col)) % NCH) * 16);
  uint32_t vrd[DT];
  {
    const int rr = gq * 4 + (col >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vrd[dt] = static_cast<uint32_t>(rr * ROWB + (((dt * 2 + ((col & 3) >> 1)) ^ chunk_swz<D>(rr)) % NCH) * 16 +
                                      (col & 1) * 8);
  }

  // S^T tile from K rows in LDS
  auto qk = [&](const uint16_t* kt_lds, f32x4_t (&s)[4][2]) {
    const char* kb = reinterpret_cast<const char*>(kt_lds);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[kt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8_t ka = as_bf16x8(*reinterpret_cast<const Vec16*>(kb + krd[ks] + kt * 16 * ROWB));
#pragma unroll
        for (int t = 0; t < 2; ++t)
          s[kt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop[t][ks], s[kt][t], 0, 0, 0);
      }
    }
  };

  f32x4_t o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t) o[dt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};

  issue_tile(false, lds_k[0], 0);
  issue_tile(true, lds_v[0], 0);
  if (nkt > 1) issue_tile(false, lds_k[1], kKeys);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x4_t s_cur[4][2];
  qk(sK[0], s_cur);

  // running-max helpers: masking of a tile that crosses the diagonal or the
  // key end; the tile max in eight pieces (so it can be spread over MFMAs);
  // and the lazy move of the reference max (O and l rescaled), which must
  // come after every P V product that used the old max
  auto mask_tile = [&](f32x4_t (&sx)[4][2], int kt0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int lim = min(posq[t], Lk - 1) - (kt0 + gq * 4);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sx[kt][t][e] = (kt * 16 + e <= lim) ? sx[kt][t][e] : -INFINITY;
    }
  };
  float tm[2], mc[2];
  auto max_piece = [&](int c, const f32x4_t (&sx)[4][2]) {
    const int t = c / 4;
    switch (c % 4) {
      case 0:
        tm[t] = max3f(sx[0][t][0], sx[0][t][1], sx[0][t][2]);
        tm[t] = max3f(tm[t], sx[0][t][3], sx[1][t][0]);
        break;
      case 1:
        tm[t] = max3f(tm[t], sx[1][t][1], sx[1][t][2]);
        tm[t] = max3f(tm[t], sx[1][t][3], sx[2][t][0]);
        break;
      case 2:
        tm[t] = max3f(tm[t], sx[2][t][1], sx[2][t][2]);
        tm[t] = max3f(tm[t], sx[2][t][3], sx[3][t][0]);
        tm[t] = max3f(tm[t], sx[3][t][1], sx[3][t][2]);
        tm[t] = max2f(tm[t], sx[3][t][3]);
        break;
      default:
        mc[t] = col_max(tm[t]) * scale_log2;
        break;
    }
  };
  auto move_max = [&]() {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (__any(mc[t] > m[t] + kMaxSlack)) {
        const float m_new = max2f(m[t], mc[t]);
        const float alpha = fast_exp2(m[t] - m_new);
        l[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][t] *= alpha;
        m[t] = m_new;
      }
    }
  };
  auto need_mask_at = [&](int kt0) { return !(kt0 + kKeys - 1 <= start + q_lo && kt0 + kKeys <= Lk); };

  if (need_mask_at(0)) mask_tile(s_cur, 0);
#pragma unroll
  for (int c = 0; c < 8; ++c) max_piece(c, s_cur);
  move_max();

  for (int j = 0; j < nkt; ++j) {
    const int kt0 = j * kKeys;
    // everything issued in the previous iteration has landed, and every wave
    // is done with K(j) (read for S(j) one iteration ago) and V(j - 1)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < nkt) issue_tile(false, lds_k[j & 1], kt0 + 2 * kKeys);
    if (j + 1 < nkt) issue_tile(true, lds_v[(j + 1) & 1], kt0 + kKeys);

    f32x4_t s_next[4][2];
    Vec16 pop[2][2];
    // The S phase (matrix and vector work interleaved) runs at the highest
    // wave priority, the P V phase (mostly matrix work) at the lowest: when
    // the two waves of a SIMD are in different phases, the arbiter then
    // issues the mixed phase first and the MFMA-only phase fills the gaps
    // (chunked prefill -1.7%, uniform 8 x 2048 -4.7%, bitwise equal).
    __builtin_amdgcn_s_setprio(3);
    // S(j+1) = K(j+1) Q^T on the matrix cores, interleaved by hand with this
    // tile's exp2 / packing / row sums on the vector ALU: after every MFMA,
    // three of the 96 vector instructions; K operands are read one k-step
    // ahead. (On the last tile the K buffer is stale; those scores are never
    // used.) A scheduling fence after each slot keeps the order.
    {
      const char* kb = reinterpret_cast<const char*>(sK[(j + 1) & 1]);
      bf16x8_t kop[2][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kop[0][kt] = as_bf16x8(*reinterpret_cast<const Vec16*>(kb + krd[0] + kt * 16 * ROWB));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t) s_next[kt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float lsum[2] = {l[0], l[1]};
      auto vop = [&](int k) {
        const int t = k / 48;
        const int r = k % 48;
        if (r < 32) {
          const int el = r / 2;
          const int kt = el / 4, e = el % 4;
          if ((r & 1) == 0) s_cur[kt][t][e] = fmaf(s_cur[kt][t][e], scale_log2, -m[t]);
          else s_cur[kt][t][e] = fast_exp2(s_cur[kt][t][e]);
        } else if (r < 40) {
          const int q = r - 32, st = q / 4, w = q % 4;
          const int kt = 2 * st + w / 2, e0 = 2 * (w % 2);
          pop[st][t].w[w] = pack2(s_cur[kt][t][e0], s_cur[kt][t][e0 + 1]);
        } else {
          const int q = r - 40, st = q / 4, w = q % 4;
          lsum[t] = dot2_bf16(pop[st][t].w[w], kOnesBf16x2, lsum[t]);
        }
      };
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            kop[(ks + 1) & 1][kt] = as_bf16x8(*reinterpret_cast<const Vec16*>(kb + krd[ks + 1] + kt * 16 * ROWB));
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int i = (ks * 4 + kt) * 2 + t;
            s_next[kt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks & 1][kt], qop[t][ks], s_next[kt][t], 0, 0, 0);
            constexpr int PER_MFMA = 96 / (KS * 8);
#pragma unroll
            for (int u = 0; u < PER_MFMA; ++u) vop(PER_MFMA * i + u);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      l[0] = lsum[0];
      l[1] = lsum[1];
      // keep the weights computed here, beside the MFMAs (the compiler would
      // otherwise sink them past the masking branch below)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          asm volatile("" :: "v"(pop[st][t].w[0]), "v"(pop[st][t].w[1]), "v"(pop[st][t].w[2]), "v"(pop[st][t].w[3]));
      asm volatile("" :: "v"(l[0]), "v"(l[1]));
    }
    __builtin_amdgcn_s_setprio(0);
    const bool has_next = j + 1 < nkt;
    if (has_next && need_mask_at(kt0 + kKeys)) mask_tile(s_next, kt0 + kKeys);

    // O^T += V^T P^T, interleaved with the next tile's max (eight pieces);
    // lane (gq, col) takes column dt * 16 + col of the keys st * 32 + gq * 4
    // + 0..3 and st * 32 + 16 + gq * 4 + 0..3 (the order in which the P^T
    // operand holds them); V operands are read one head_dim tile ahead
    {
      const char* vt = reinterpret_cast<const char*>(sV[j & 1]);
      s16x4_t va[2][2][2];
      auto vread = [&](int dt, int bufi) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          va[bufi][st][0] = ds_read_tr16(reinterpret_cast<const uint16_t*>(vt + vrd[dt] + st * 32 * ROWB));
          va[bufi][st][1] = ds_read_tr16(reinterpret_cast<const uint16_t*>(vt + vrd[dt] + (st * 32 + 16) * ROWB));
        }
      };
      vread(0, 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if (dt + 1 < DT) vread(dt + 1, (dt + 1) & 1);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const s16x4_t lo = va[dt & 1][st][0];
          const s16x4_t hi = va[dt & 1][st][1];
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int i = (dt * 2 + st) * 2 + t;
            o[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(pop[st][t]), o[dt][t], 0, 0, 0);
            constexpr int EVERY = (DT * 4) / 8;
            if (i % EVERY == EVERY - 1) max_piece(i / EVERY, s_next);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    if (has_next) move_max();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int t = 0; t < 2; ++t) s_cur[kt][t] = s_next[kt][t];
  }

  write_out<D>(out, o, l, orow, ohead, num_q_heads, gq, 1.f);
  if constexpr (FUSED)  // last, as in prefill_kernel
    store_new_rows<D>(const_cast<char*>(k_cache), const_cast<char*>(v_cache), k_stride_bytes, new_k, new_v,
                      nk_stride_bytes, nv_stride_bytes, slot_mapping, q0 + q_lo, q_hi - q_lo, g);
}

template <int D, int G, bool FP8, bool FUSED>
hipError_t launch_prefill_typed(const PrefillArgs& a, hipStream_t stream) {
  constexpr int KB = FP8 ? 1 : 2;
  constexpr int QT = kRows / G;
  int log2_bs = 0;
  while ((1 << log2_bs) < a.block_size) ++log2_bs;
  const int max_qt = (a.max_seqlen_q + QT - 1) / QT;
  if (max_qt == 0 || a.num_seqs == 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(max_qt) * a.num_kv_heads * a.num_seqs;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid(static_cast<uint32_t>(total));
  // an E4M3 cache holds K / k_scale: the score scale absorbs k_scale
  const float scale_log2 = a.scale * (FP8 ? a.k_scale : 1.f) * kLog2e;
  const bool whole_rows = a.block_tables == nullptr || log2_bs >= 6;
  if (!FP8 && whole_rows) {
    hipLaunchKernelGGL((prefill_direct_kernel<D, G, FUSED>), grid, dim3(kThreads), 0, stream,
                       static_cast<uint16_t*>(a.out), static_cast<const char*>(a.q), a.q_stride * 2,
                       static_cast<const char*>(a.k_cache), static_cast<const char*>(a.v_cache),
                       a.k_stride * KB, a.v_stride * KB, a.cu_q, a.cu_k, a.block_tables, a.max_blocks,
                       a.num_q_heads, a.num_kv_heads, log2_bs, scale_log2, max_qt,
                       static_cast<const char*>(a.new_k), static_cast<const char*>(a.new_v), a.new_k_stride * 2,
                       a.new_v_stride * 2, a.slot_mapping);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_kernel<D, G, FP8, FUSED>), grid, dim3(kThreads), 0, stream,
                     static_cast<uint16_t*>(a.out), static_cast<const char*>(a.q), a.q_stride * 2,
                     static_cast<const char*>(a.k_cache), static_cast<const char*>(a.v_cache),
                     a.k_stride * KB, a.v_stride * KB, a.cu_q,
                     a.cu_k, a.block_tables, a.max_blocks, a.num_q_heads, a.num_kv_heads, log2_bs,
                     scale_log2, max_qt, a.v_scale, static_cast<const char*>(a.new_k),
                     static_cast<const char*>(a.new_v), a.new_k_stride * 2, a.new_v_stride * 2, a.slot_mapping);
  return hipGetLastError();
}

template <int D, bool FP8, bool FUSED>
hipError_t dispatch_prefill_group(const PrefillArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefill_typed<D, 1, FP8, FUSED>(a, stream);
    case 2: return launch_prefill_typed<D, 2, FP8, FUSED>(a, stream);
    case 4: return launch_prefill_typed<D, 4, FP8, FUSED>(a, stream);
    case 8: return launch_prefill_typed<D, 8, FP8, FUSED>(a, stream);
    case 16: return launch_prefill_typed<D, 16, FP8, FUSED>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool FP8, bool FUSED>
hipError_t dispatch_prefill_dim(const PrefillArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? dispatch_prefill_group<64, FP8, FUSED>(a, stream)
                          : dispatch_prefill_group<128, FP8, FUSED>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const bool fused = a.slot_mapping != nullptr;
  if (a.fp8) {
    if (fused) {
      // E4M3: every query tile that reads a new row would quantise it again
      // (per element an fp32 division and a rounding), which costs more than
      // the scatter's own launch; so the scatter runs first, as its own
      // kernel, and the attention reads all keys from the caches.
      const int32_t row_bytes = a.num_kv_heads * a.head_dim * 2;
      const StoreArgs st{a.new_k, a.new_k_stride * 2, a.new_v, a.new_v_stride * 2,
                         const_cast<void*>(a.k_cache), const_cast<void*>(a.v_cache), a.slot_mapping,
                         a.total_q, row_bytes, true, a.k_scale, a.v_scale};
      const hipError_t e = launch_store(st, stream);
      if (e != hipSuccess) return e;
    }
    return dispatch_prefill_dim<true, false>(a, stream);
  }
  return fused ? dispatch_prefill_dim<false, true>(a, stream) : dispatch_prefill_dim<false, false>(a, stream);
}

}  // namespace pa
